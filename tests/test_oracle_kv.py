"""Pins for the oracle's FP8 KV-cache functions (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from conftest import parse_num, read_golden
from exact import nearest_bf16, nearest_f32
from oracle import fp8, kv, w8a8
from oracle.fp8 import E4M3, E5M2
from workloads import bf16_bits_from_f32, f32_from_bf16_bits, kv_append_inputs, kv_inputs

FMTS = [E4M3, E5M2]


def small_kv(seed=0):
    k, v, kc, vc = kv_inputs(seed, b=2, s=48, h=4, d=32, n_out=3)
    return k, v, kc, vc


def test_unit_scale_facts():
    """With the uncalibrated scale 1.0: 0.001 rounds up to 2^-9, a little smaller
    becomes 0, and magnitudes beyond 448 clip."""
    rows = read_golden("kv_unit_scale.txt")
    x = np.float32([parse_num(r[0]) for r in rows])
    want = np.array([parse_num(r[1]) for r in rows])
    codes = kv.kv_quant(bf16_bits_from_f32(x).reshape(1, 1, 1, -1), np.float32([1.0]), E4M3)
    # bf16 rounding of 0.001 keeps it strictly between 2^-10 and 2^-9
    got = fp8.decode(codes.ravel(), E4M3)
    assert got.tolist() == want.tolist()


@pytest.mark.parametrize("fmt", FMTS)
def test_calibrate_matches_head_amax(fmt):
    k, v, kc, vc = small_kv()
    for t in (k, v):
        s = kv.kv_calibrate(t, fmt)
        x = f32_from_bf16_bits(t)
        for h in range(t.shape[2]):
            amax = np.abs(x[:, :, h, :]).max()
            assert s[h] == nearest_f32(Fraction(float(amax)) / Fraction(fmt.max_finite))
        # each head's maximum lands on the top code
        q = kv.kv_quant(t, s, fmt)
        for h in range(t.shape[2]):
            xa = np.abs(x[:, :, h, :])
            idx = np.unravel_index(xa.argmax(), xa.shape)
            assert q[idx[0], idx[1], h, idx[2]] & 0x7F == fmt.max_code


@pytest.mark.parametrize("fmt", FMTS)
def test_quant_is_given_scale_rule_per_head(fmt):
    k, _, _, _ = small_kv(1)
    s = np.float32([0.01, 0.5, 3.0, 1e-3])
    q = kv.kv_quant(k, s, fmt)
    x = f32_from_bf16_bits(k)
    for h in range(4):
        assert np.array_equal(q[:, :, h, :], w8a8.quant_static(x[:, :, h, :], s[h], fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_round_trip_of_representable_values(fmt):
    """x = s_h * (an FMT value), with s_h of few significant bits so that x is an
    exact bf16: quant then dequant returns x exactly."""
    rng = np.random.default_rng(2)
    s = np.float32([0.75, 2.0 ** -3 * 1.25, 3.0, 1.0])
    finite = np.array([c for c in range(256) if np.isfinite(fmt.values[c])], dtype=np.uint8)
    codes = rng.choice(finite, size=(2, 5, 4, 16))
    x = (fp8.decode(codes, fmt) * s.reshape(1, 1, 4, 1).astype(np.float64)).astype(np.float32)
    xb = bf16_bits_from_f32(x)
    assert np.array_equal(f32_from_bf16_bits(xb), x)
    q = kv.kv_quant(xb, s, fmt)
    back = kv.kv_dequant(q, s, fmt)
    # codes of +-0 may differ in sign only if x is zero; compare values
    assert np.array_equal(f32_from_bf16_bits(back), x)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_is_f32_product_then_bf16(fmt):
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, size=(1, 3, 2, 64), dtype=np.uint8)
    q = np.where(np.isfinite(fmt.values[q]), q, 0).astype(np.uint8)
    s = np.float32([0.0123, 7.77e-3])
    y = kv.kv_dequant(q, s, fmt)
    for idx in np.ndindex(q.shape):
        p = nearest_f32(Fraction(float(fmt.values[q[idx]])) * Fraction(float(s[idx[2]])))
        want = nearest_bf16(Fraction(float(p)))
        got = f32_from_bf16_bits(np.uint16([y[idx]]))[0]
        assert Fraction(float(got)) == want


def test_saturation_count():
    k, _, _, _ = small_kv(4)
    s = np.float32([0.002, 0.002, 0.002, 0.002])
    q = kv.kv_quant(k, s, E4M3)
    t = w8a8.f32_div(f32_from_bf16_bits(k), s.reshape(1, 1, -1, 1))
    # the top code collects every |t| from the 416/448 midpoint (a tie, resolved to
    # the even code 0x7E) upward, the saturated values |t| >= 448 among them
    assert (np.abs(t) >= 448).sum() > 0
    assert ((q & 0x7F) == 0x7E).sum() == (np.abs(t) >= 432).sum()


def test_append_writes_only_the_given_positions():
    k, v, kc, vc = small_kv(5)
    s = kv.kv_calibrate(k, E4M3)
    cache = np.full((2, 50, 4, 32), 0xA5, dtype=np.uint8)
    cache[:, :48] = kv.kv_quant(k, s, E4M3)
    kn, _ = kv_append_inputs(kc, vc, seed=5, b=2, h=4, d=32)
    pos = np.array([48, 7])
    out = kv.kv_append(cache, kn, pos, s, E4M3)
    changed = np.nonzero((out != cache).any(axis=(2, 3)))
    assert set(zip(*changed)) <= {(0, 48), (1, 7)}
    x = f32_from_bf16_bits(kn)
    for b, p in enumerate(pos):
        for h in range(4):
            assert np.array_equal(out[b, p, h], w8a8.quant_static(x[b, h], s[h], E4M3))
