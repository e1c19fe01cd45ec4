"""MXFP8: blocks of 32 consecutive k with one power-of-two scale each (CPU oracle).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.

What is computed
----------------
Microscaling formats give each small block of consecutive elements its own
scale: blocks of 16 or 32 elements, the scale itself stored in 8 bits
("Quantization for LLM inference: FP8, INT4 (GPTQ, AWQ) and GGUF", blog.lo0.es
-- "Microscaling: NVFP4 and MXFP4"; its reference list names MXFP8).  For MXFP8 the blocks lie along the
reduction dimension ("Quantization: FP8 inference and KV-cache quantization" --
"Training in FP8 or lower": MXFP8 data must be contiguous along the reduction
dimension), and the scale byte is the OCP MX specification's E8M0 power of two,
the specification that page cites.

Readings (the pages do not spell out the MXFP8 scale rule):
* Block: 32 consecutive k of one row of A [M, K] or W [N, K].
* Scale byte e (E8M0): the value 2^(e - 127), e in 0..254; 255 (NaN) is never
  produced.
* Scale choice: the pages' dynamic rule s = amax / FMAX (the block's largest
  magnitude lands on the format's maximum), restricted to powers of two and
  rounded up, so that no element of the block saturates: s = 2^k with k the
  smallest integer such that amax <= FMAX * 2^k, clamped to [-127, 127]; a
  block of zeros gets 2^0 (the unit-scale reading used for every dynamic scale
  of this library).
* Codes: q = FMT(RN32(x / 2^k)) with the library's saturating round-to-
  nearest-even encoder (oracle/fp8.py).  Division by a power of two is exact
  except where the quotient is subnormal in float32; RN32 rounds it there.
* GEMM: the scales vary along k, so each 32-deep partial dot product is scaled
  on its own:
      y[m, n] = sum_b 2^(ka[m, b] + kw[n, b]) * P_b[m, n],
      P_b[m, n] = sum_{k = 32 b}^{32 b + 31} dec(a_q[m, k]) * dec(w_q[n, k]).
  A's element format is E4M3 or E5M2; W's is E4M3.

Reference arithmetic: for E4M3 x E4M3 every product is a multiple of 2^-18
below 2^18 in magnitude, so P_b (32 of them) is exact in float64; for
E5M2 x E4M3 the products are multiples of 2^-25 below 2^25, and the float64
sum of 32 may round, by at most 31 * 2^-53 * sum |p|.  The power-of-two scale
multiply is exact; the float64 sum over the K / 32 blocks adds at most
(K / 32) * 2^-53 of the sum of absolute terms.  Both are far below the float32
accumulator tolerance and a bf16 ulp.
"""

from __future__ import annotations

import numpy as np

from .fp8 import E4M3, Fp8Format, bf16_round_bits, decode, encode
from .w8a8 import f32_div

__all__ = ["BLOCK", "E8M0_BIAS", "e8m0_value", "scale_exponent", "block_amax", "quant_mx", "dequant_mx",
           "mx_partials", "gemm_mx_exact", "gemm_mx_abs", "gemm_mx_bf16"]

BLOCK = 32
E8M0_BIAS = 127


def e8m0_value(e) -> np.ndarray:
    """Value of E8M0 scale bytes (0..254): 2^(e - 127), float64."""
    e = np.asarray(e, np.int64)
    assert ((e >= 0) & (e <= 254)).all()
    return np.ldexp(1.0, (e - E8M0_BIAS).astype(np.int32))


def scale_exponent(amax, fmt: Fp8Format = E4M3) -> np.ndarray:
    """k per block: the smallest integer with amax <= FMAX * 2^k, clamped to
    [-127, 127]; 0 for amax == 0.  Every comparison is exact in float64
    (FMAX * 2^k is a float64 value; amax is a float32 value)."""
    a = np.asarray(amax, np.float64)
    fmax = float(fmt.max_finite)
    pos = a > 0
    # a first guess from the binary exponents, then the exact test decides
    ea = np.frexp(np.where(pos, a, 1.0))[1]
    ef = np.frexp(fmax)[1]
    k = (ea - ef).astype(np.int64) - 1
    for _ in range(3):
        k = np.where(a > fmax * np.ldexp(1.0, k.astype(np.int32)), k + 1, k)
    k = np.clip(k, -127, 127)
    return np.where(pos, k, 0).astype(np.int64)


def block_amax(x: np.ndarray) -> np.ndarray:
    """max |x| over each block of 32 consecutive k: [R, K] -> [R, K / 32] (float32, exact)."""
    x = np.asarray(x, np.float32)
    R, K = x.shape
    assert K % BLOCK == 0
    return np.abs(x).reshape(R, K // BLOCK, BLOCK).max(axis=-1)


def quant_mx(x: np.ndarray, fmt: Fp8Format = E4M3):
    """MX quantization of rows: returns (codes uint8 [R, K], scale bytes uint8 [R, K / 32])."""
    x = np.asarray(x, np.float32)
    k = scale_exponent(block_amax(x), fmt)
    s = np.ldexp(np.float32(1.0), k.astype(np.int32)).astype(np.float32)   # 2^k, exact in float32
    t = f32_div(x, np.repeat(s, BLOCK, axis=1))
    return encode(t, fmt), (k + E8M0_BIAS).astype(np.uint8)


def dequant_mx(q: np.ndarray, e8: np.ndarray, fmt: Fp8Format = E4M3) -> np.ndarray:
    """Exact values dec(q) * 2^(e - 127), float64 [R, K]."""
    return decode(q, fmt) * np.repeat(e8m0_value(e8), BLOCK, axis=1)


def mx_partials(a_q, w_q, a_fmt: Fp8Format = E4M3, absolute: bool = False) -> np.ndarray:
    """P [K / 32, M, N]: the 32-deep partial dot products of decoded codes (float64)."""
    a = decode(a_q, a_fmt)
    w = decode(w_q, E4M3)
    if absolute:
        a, w = np.abs(a), np.abs(w)
    nb = a.shape[1] // BLOCK
    return np.stack([a[:, b * BLOCK:(b + 1) * BLOCK] @ w[:, b * BLOCK:(b + 1) * BLOCK].T for b in range(nb)])


def _scale_grid(a_e8, w_e8) -> np.ndarray:
    """[K / 32, M, N] products 2^(ka[m, b] + kw[n, b]) (float64, exact)."""
    sa = e8m0_value(a_e8)   # [M, nb]
    sw = e8m0_value(w_e8)   # [N, nb]
    return sa.T[:, :, None] * sw.T[:, None, :]


def gemm_mx_exact(a_q, a_e8, w_q, w_e8, a_fmt: Fp8Format = E4M3) -> np.ndarray:
    """y [M, N] = sum_b 2^(ka + kw) P_b (float64)."""
    return (_scale_grid(a_e8, w_e8) * mx_partials(a_q, w_q, a_fmt)).sum(axis=0)


def gemm_mx_abs(a_q, a_e8, w_q, w_e8, a_fmt: Fp8Format = E4M3) -> np.ndarray:
    """sum_b 2^(ka + kw) sum_k |a w| -- the scale of the accumulator tolerance."""
    return (_scale_grid(a_e8, w_e8) * mx_partials(a_q, w_q, a_fmt, absolute=True)).sum(axis=0)


def gemm_mx_bf16(a_q, a_e8, w_q, w_e8, a_fmt: Fp8Format = E4M3):
    """Y = bf16(y_exact); returns (y_bits uint16 [M, N], y_exact float64)."""
    y = gemm_mx_exact(a_q, a_e8, w_q, w_e8, a_fmt)
    return bf16_round_bits(y), y

