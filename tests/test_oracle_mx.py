"""Pins of the MXFP8 oracle (oracle/mx.py) to facts that do not come from the
oracle itself: the definition of a biased power-of-two exponent, a brute-force
search for the scale rule, a block worked by hand from the E4M3 grid, exact
rational arithmetic for the GEMM, the plain product of the dequantized
operands, and the per-token GEMM's exact accumulator when every scale is 1."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import mx, w8a8
from oracle.fp8 import E4M3, E5M2, decode


def _brute_k(amax: float, fmax: float) -> int:
    if amax == 0:
        return 0
    for k in range(-127, 128):
        if Fraction(amax) <= Fraction(fmax) * Fraction(2) ** k:
            return k
    raise AssertionError("no scale fits")


def test_e8m0_is_a_biased_power_of_two():
    e = np.arange(0, 255)
    v = mx.e8m0_value(e)
    assert v[127] == 1.0 and v[128] == 2.0 and v[126] == 0.5
    assert v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.all(v[1:] / v[:-1] == 2.0)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scale_exponent_is_the_smallest_power_of_two_that_fits(fmt):
    rng = np.random.default_rng(3)
    fmax = float(fmt.max_finite)
    vals = [0.0, fmax, float(np.nextafter(np.float32(fmax), np.float32(np.inf))),
            float(np.nextafter(np.float32(fmax), np.float32(0))), 1.0, 2.0 ** -149, 2.0 ** -126, 3.0e38]
    for k in (-20, -3, 0, 1, 7, 40):
        b = np.float32(fmax * 2.0 ** k)
        vals += [float(b), float(np.nextafter(b, np.float32(np.inf))), float(np.nextafter(b, np.float32(0)))]
    vals += list(np.exp2(rng.uniform(-150, 127, 400)).astype(np.float32).astype(float))
    a = np.array(vals, np.float32)
    got = mx.scale_exponent(a, fmt)
    want = np.array([max(-127, min(127, _brute_k(float(v), fmax))) for v in a])
    assert np.array_equal(got, want)


def _blocks(seed, R=6, K=256):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, K)).astype(np.float32)
    x[:, rng.integers(0, K, 5)] *= 60.0           # outliers in some blocks
    x[1, 32:64] = 0.0                               # an all-zero block
    x[2, 64:96] *= np.float32(2.0 ** -130)          # a block below the smallest scale
    x[3, :32] = np.float32(448.0)                   # a block whose maximum is exactly FMAX
    return x


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_no_element_saturates_and_the_block_maximum_uses_the_top_binade(fmt):
    x = _blocks(1)
    q, e8 = mx.quant_mx(x, fmt)
    fmax = float(fmt.max_finite)
    k = e8.astype(np.int64) - 127
    t = np.abs(x.astype(np.float64)) / np.repeat(np.ldexp(1.0, k), 32, axis=1)
    assert (t <= fmax).all()                         # nothing beyond the format maximum
    amax = np.abs(x).reshape(x.shape[0], -1, 32).max(axis=-1).astype(np.float64)
    top = np.abs(decode(q, fmt)).reshape(x.shape[0], -1, 32).max(axis=-1)
    live = (amax > 0) & (k > -127)
    # the largest code of a block lies in the format's top binade: amax > FMAX * 2^(k - 1)
    assert (top[live] >= fmax / 2).all()
    assert e8[1, 1] == 127 and (q[1, 32:64] == 0).all()      # zero block: unit scale, +0 codes
    assert e8[3, 0] == 127 + (0 if fmt is E4M3 else -7)       # 448 fits 448 * 2^0 (E5M2: 57344 * 2^-7)


def test_a_block_worked_by_hand():
    # amax 900: 900 / 448 = 2.01 -> s = 4 (2^1 * 448 = 896 < 900 <= 1792).  900 / 4 = 225
    # lies between the E4M3 values 224 (1.75 * 2^7) and 240 (1.875 * 2^7): 224.
    # 1 / 4 = 0.25 = 2^-2, -3 / 4 = -0.75 = -1.5 * 2^-1, 0.01 / 4 = 0.0025 lies between
    # the subnormals 1 * 2^-9 and 2 * 2^-9 (0.00195, 0.00391): 2^-9.
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [900.0, 1.0, -3.0, 0.01]
    q, e8 = mx.quant_mx(x, E4M3)
    assert int(e8[0, 0]) == 129
    want = {0: 0b0_1110_110, 1: 0b0_0101_000, 2: 0b1_0110_100, 3: 0b0_0000_001}
    for i, c in want.items():
        assert int(q[0, i]) == c, (i, hex(int(q[0, i])))
    assert (q[0, 4:] == 0).all()
    assert np.array_equal(mx.dequant_mx(q, e8)[0, :4], [896.0, 1.0, -3.0, 4 * 2.0 ** -9])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_round_trip_of_representable_blocks(fmt):
    rng = np.random.default_rng(5)
    R, K = 4, 128
    codes = rng.integers(0, 0x7E if fmt is E4M3 else 0x7B, (R, K), dtype=np.uint8)
    codes |= (rng.integers(0, 2, (R, K), dtype=np.uint8) << 7)
    codes[:, ::32] = 0x7E if fmt is E4M3 else 0x7B      # each block holds the format maximum
    e8 = rng.integers(100, 150, (R, K // 32)).astype(np.uint8)
    x = mx.dequant_mx(codes, e8, fmt).astype(np.float32)
    q, e = mx.quant_mx(x, fmt)
    assert np.array_equal(e, e8)
    assert np.array_equal(decode(q, fmt), decode(codes, fmt))   # -0 / +0 aside


def _mx_case(seed, M=5, N=7, K=128, a_fmt=E4M3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.integers(0, K, 3)] *= 50.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[rng.integers(0, N, 2), :32] *= 100.0             # blocks with very different scales
    aq, ae = mx.quant_mx(x, a_fmt)
    wq, we = mx.quant_mx(w, E4M3)
    return aq, ae, wq, we


@pytest.mark.parametrize("a_fmt", [E4M3, E5M2])
def test_gemm_equals_rational_brute_force(a_fmt):
    aq, ae, wq, we = _mx_case(7, M=3, N=4, K=64, a_fmt=a_fmt)
    y = mx.gemm_mx_exact(aq, ae, wq, we, a_fmt)
    for m in range(3):
        for n in range(4):
            tot = Fraction(0)
            for k in range(64):
                b = k // 32
                sa = Fraction(2) ** (int(ae[m, b]) - 127)
                sw = Fraction(2) ** (int(we[n, b]) - 127)
                tot += Fraction(float(decode(aq[m, k:k + 1], a_fmt)[0])) * sa * \
                    Fraction(float(decode(wq[n, k:k + 1], E4M3)[0])) * sw
            assert abs(Fraction(y[m, n]) - tot) <= abs(tot) * Fraction(1, 2 ** 50)


def test_gemm_equals_product_of_dequantized_operands():
    aq, ae, wq, we = _mx_case(8, M=9, N=11, K=512)
    y = mx.gemm_mx_exact(aq, ae, wq, we)
    ref = mx.dequant_mx(aq, ae) @ mx.dequant_mx(wq, we).T
    absum = np.abs(mx.dequant_mx(aq, ae)) @ np.abs(mx.dequant_mx(wq, we)).T
    assert np.all(np.abs(y - ref) <= 1e-14 * absum)
    assert np.allclose(mx.gemm_mx_abs(aq, ae, wq, we), absum, rtol=1e-14, atol=0)


def test_unit_scales_give_the_plain_accumulator():
    aq, _, wq, _ = _mx_case(9, M=6, N=5, K=256)
    ones_a = np.full((6, 8), 127, np.uint8)
    ones_w = np.full((5, 8), 127, np.uint8)
    assert np.array_equal(mx.gemm_mx_exact(aq, ones_a, wq, ones_w), w8a8.gemm_acc_exact(aq, wq))


def test_quantization_error_is_bounded_by_half_a_step():
    x = _blocks(11)
    q, e8 = mx.quant_mx(x, E4M3)
    back = mx.dequant_mx(q, e8)
    k = np.repeat(e8.astype(np.int64) - 127, 32, axis=1)
    # E4M3 steps: 2^(e - 3) for normals (e >= -6), 2^-9 for subnormals; scaled by 2^k
    a = np.abs(x.astype(np.float64)) / np.ldexp(1.0, k)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.ldexp(np.where(a >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9), k)
    tiny = np.abs(x) < 2.0 ** -100                   # the quotient itself is subnormal in float32
    assert np.all((np.abs(back - x) <= step / 2) | tiny)
