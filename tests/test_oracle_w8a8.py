"""Pins for the oracle's quantizers and scaled GEMM (CPU only).

Pinned by the pages' worked examples (tests/golden), by exact rational
arithmetic (Fraction), by closed forms and by invariants the pages state.
"""

from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden
from exact import nearest_bf16, nearest_f32
from oracle import fp8, w8a8
from oracle.fp8 import E4M3, E5M2
from workloads import f32_from_bf16_bits, tiny_w8a8


def _golden_dict(name):
    return {r[0]: [float(v) for v in r[1:]] for r in read_golden(name)}


# ------------------------------------------------------------ float32 division

def test_f32_div_is_correctly_rounded():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))).astype(np.float32)
    b = (np.abs(rng.standard_normal(3000)) * np.exp2(rng.integers(-60, 60, 3000))).astype(np.float32)
    # include subnormal quotients and bf16-valued numerators
    a = np.concatenate([a, np.float32([1e-38, 3e-39, 2.0 ** -133, 7.0, 0.01]), f32_from_bf16_bits(
        rng.integers(0, 1 << 15, 500, dtype=np.uint16))])
    b = np.concatenate([b, np.float32([3.0, 1e3, 448.0, 0.268, 0.402]),
                        np.full(500, np.float32(0.0071428571), np.float32)])
    keep = np.isfinite(a) & np.isfinite(b) & (b != 0)
    a, b = a[keep], b[keep]
    q = w8a8.f32_div(a, b)
    for x, y, z in zip(a, b, q):
        assert z == nearest_f32(Fraction(float(x)) / Fraction(float(y))), (x, y, z)


# ------------------------------------------------------------ worked examples

def test_row_outlier_example_readback():
    g = _golden_dict("row_outlier_example.txt")
    row = np.float32([g["input"]])
    q, s = w8a8.quant_per_token(row)
    readback = fp8.decode(q[0]) * np.float64(s[0])
    assert np.round(readback, 4).tolist() == g["readback"]
    # the outlier maps to the top code, the scale is amax / 448
    assert q[0, -1] == 0x7E
    assert s[0] == np.float32(400.0) / np.float32(448.0)


def test_token_ab_dynamic_and_static():
    g = _golden_dict("token_ab_example.txt")
    a = np.float32([g["token_a"]])
    b = np.float32([g["token_b"]])
    qa, sa = w8a8.quant_per_token(a)
    qb, sb = w8a8.quant_per_token(b)
    assert round(float(sa[0]), 5) == g["dyn_scale_a"][0]
    assert round(float(sb[0]), 3) == g["dyn_scale_b"][0]
    # each token's maximum lands exactly on 448
    assert fp8.decode(qa[0, 2:]) == 448 and fp8.decode(qb[0, 2:]) == 448
    assert round(float(fp8.decode(qa[0, :1])[0] * sa[0]), 4) == g["dyn_a_readback0"][0]
    s = w8a8.f32_div(np.float32(120.0), np.float32(448.0))
    assert round(float(s), 3) == g["static_scale"][0]
    qa_s = w8a8.quant_static(a[0], s)
    qb_s = w8a8.quant_static(b[0], s)
    ra = fp8.decode(qa_s) * np.float64(s)
    rb = fp8.decode(qb_s) * np.float64(s)
    assert round(ra[0], 4) == g["static_a_readback0"][0]
    assert round(abs(ra[0] - 0.01) / 0.01, 3) == g["static_a_relerr0"][0]
    assert round(float(w8a8.f32_div(np.float32(180.0), s))) == g["static_b_ratio2"][0]
    assert qb_s[2] == 0x7E and round(rb[2], 4) == g["static_b_readback2"][0]


def test_static_tie_reading():
    # -45 / RN32(120/448) is exactly -168.0 in float32: a tie between -160 and
    # -176, which round-half-to-even resolves to -160 (code 0xF2).
    s = w8a8.f32_div(np.float32(120.0), np.float32(448.0))
    assert w8a8.f32_div(np.float32(-45.0), s) == np.float32(-168.0)
    assert w8a8.quant_static(np.float32([-45.0]), s)[0] == 0xF2


# ------------------------------------------------------------ invariants

def test_row_maximum_maps_to_top_code():
    x, w = tiny_w8a8(0)
    for arr in (x, w):
        q, s = w8a8.quant_rows_dynamic(arr)
        idx = np.abs(arr).argmax(axis=1)
        top = q[np.arange(arr.shape[0]), idx]
        assert ((top & 0x7F) == 0x7E).all()
        # scale is the float32 quotient of the row maximum by 448
        for i in range(arr.shape[0]):
            amax = np.abs(arr[i]).max()
            assert s[i] == nearest_f32(Fraction(float(amax)) / 448)


def test_quotient_never_exceeds_saturation_in_dynamic_rows():
    rng = np.random.default_rng(2)
    x = (rng.standard_t(3, size=(64, 512)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    q, s = w8a8.quant_rows_dynamic(x)
    t = w8a8.f32_div(x, s[:, None])
    assert (np.abs(t) <= np.float32(448.0) * np.float32(1 + 2 ** -22)).all()
    # dequantized values are within half a step (relative 1/16) of the inputs, for normals
    r = fp8.decode(q) * s[:, None].astype(np.float64)
    normal = np.abs(t) >= 2.0 ** -6
    assert (np.abs(r - x)[normal] <= np.abs(x)[normal] / 16 * (1 + 2 ** -20)).all()


def test_zero_row_gets_unit_scale_and_signed_zero_codes():
    x = np.float32([[0.0, -0.0, 0.0, 0.0], [1.0, -2.0, 0.5, 448.0]])
    q, s = w8a8.quant_rows_dynamic(x)
    assert s[0] == 1.0 and q[0].tolist() == [0x00, 0x80, 0x00, 0x00]
    assert s[1] == 1.0 and q[1].tolist() == [0x38, 0xC0, 0x30, 0x7E]


def test_e5m2_rows_use_57344():
    x = np.float32([[1.0, -57344.0 * 3, 2.0]])
    q, s = w8a8.quant_rows_dynamic(x, E5M2)
    assert s[0] == np.float32(3.0) and q[0, 1] == 0xFB


# ------------------------------------------------------------ GEMM

def test_gemm_exact_against_fractions():
    rng = np.random.default_rng(4)
    finite = np.array([c for c in range(256) if np.isfinite(E4M3.values[c])], dtype=np.uint8)
    a = rng.choice(finite, size=(5, 64))
    w = rng.choice(finite, size=(7, 64))
    acc = w8a8.gemm_acc_exact(a, w)
    dec = {c: Fraction(float(E4M3.values[c])) for c in range(256) if np.isfinite(E4M3.values[c])}
    for i in range(5):
        for j in range(7):
            exact = sum(dec[int(a[i, k])] * dec[int(w[j, k])] for k in range(64))
            assert Fraction(float(acc[i, j])) == exact


def test_gemm_exact_tiny_workload_against_fractions():
    x, w = tiny_w8a8(0)
    aq, sa = w8a8.quant_per_token(x)
    wq, sw = w8a8.quant_weight_per_channel(w)
    y, acc = w8a8.scaled_gemm_bf16(aq, sa, wq, sw)
    dec = {c: Fraction(float(E4M3.values[c])) for c in range(256) if np.isfinite(E4M3.values[c])}
    rng = np.random.default_rng(9)
    for _ in range(60):
        i, j = int(rng.integers(16)), int(rng.integers(512))
        exact = sum(dec[int(aq[i, k])] * dec[int(wq[j, k])] for k in range(256))
        assert Fraction(float(acc[i, j])) == exact
        # scales factor out of the K-sum: y = s_a s_w sum(...), rounded once to bf16
        yv = exact * Fraction(float(sa[i])) * Fraction(float(sw[j]))
        got = Fraction(float(fp8.bf16_bits_to_f64(y[i:i + 1, j])[0]))
        assert got == nearest_bf16(yv)


def test_gemm_abs_sum_against_fractions():
    """sum_k |a_ik w_jk| -- the scale of the accumulator tolerance -- against exact
    rationals on the tiny workload's codes, and two closed forms: where every
    product is non-negative it equals the exact accumulator itself, and for
    all-maximum codes it is K * 448^2."""
    x, w = tiny_w8a8(0)
    aq, _ = w8a8.quant_per_token(x)
    wq, _ = w8a8.quant_weight_per_channel(w)
    s = w8a8.gemm_abs_sum(aq, wq)
    dec = {c: Fraction(float(E4M3.values[c])) for c in range(256) if np.isfinite(E4M3.values[c])}
    rng = np.random.default_rng(12)
    for _ in range(60):
        i, j = int(rng.integers(16)), int(rng.integers(512))
        exact = sum(abs(dec[int(aq[i, k])] * dec[int(wq[j, k])]) for k in range(256))
        assert Fraction(float(s[i, j])) == exact
    # clearing the sign bits makes every product non-negative: then sum|a w| is the sum itself
    a_pos, w_pos = aq & np.uint8(0x7F), wq & np.uint8(0x7F)
    assert np.array_equal(w8a8.gemm_abs_sum(aq, wq), w8a8.gemm_acc_exact(a_pos, w_pos))
    assert np.array_equal(w8a8.gemm_abs_sum(a_pos, w_pos), w8a8.gemm_acc_exact(a_pos, w_pos))
    k = 4096
    big = w8a8.gemm_abs_sum(np.full((2, k), 0xFE, np.uint8), np.full((3, k), 0x7E, np.uint8))
    assert (big == k * 448.0 * 448.0).all()


def test_gemm_one_hot_weights_reproduce_activations():
    rng = np.random.default_rng(6)
    finite = np.array([c for c in range(256) if np.isfinite(E4M3.values[c])], dtype=np.uint8)
    a = rng.choice(finite, size=(8, 32))
    w = np.zeros((32, 32), dtype=np.uint8)
    w[np.arange(32), np.arange(32)] = 0x38  # 1.0
    acc = w8a8.gemm_acc_exact(a, w)
    assert np.array_equal(acc, fp8.decode(a))


def test_gemm_all_max_closed_form():
    k = 14336
    a = np.full((2, k), 0x7E, dtype=np.uint8)
    w = np.full((3, k), 0xFE, dtype=np.uint8)
    acc = w8a8.gemm_acc_exact(a, w)
    assert (acc == -k * 448.0 * 448.0).all()
    assert float(np.float32(acc[0, 0])) == acc[0, 0]  # exact in float32 too


def test_scaled_output_per_tensor_scale_equals_vector_of_same():
    x, w = tiny_w8a8(0)
    wq, sw = w8a8.quant_weight_per_channel(w)
    s = np.float32(0.05)
    aq = w8a8.quant_static(x, s)
    y1, _ = w8a8.scaled_gemm_bf16(aq, s, wq, sw)
    y2, _ = w8a8.scaled_gemm_bf16(aq, np.full(16, s, np.float32), wq, sw)
    assert np.array_equal(y1, y2)


def test_relative_frobenius():
    ref = np.array([[3.0, 4.0]])
    assert w8a8.relative_frobenius(ref * 1.1, ref) == pytest.approx(0.1)
