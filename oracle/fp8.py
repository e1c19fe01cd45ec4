"""FP8 number formats, written out from their definitions (CPU oracle).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.

Formats
-------
E4M3 ("fn" variant): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
No infinities; the all-ones pattern S.1111.111 is NaN; the largest finite value
is 448 = 2^8 * 1.75, the smallest normal 2^-6, the smallest subnormal 2^-9.
(FP8 Inference Explained, in depth -- "The numbers in one byte"; FP8
Quantization notebook -- "FP8 Representation" and "E4M3 vs E5M2".)

E5M2: 1 sign bit, 5 exponent bits, 2 mantissa bits, largest finite 57,344.
The pages give only the bit split and the maximum; the bias 15, the infinities
at S.11111.00 and the NaNs at S.11111.{01,10,11} are the IEEE-style reading that
the maximum 57,344 = 2^15 * 1.75 implies (the E4M3 "fn" variant is described as
the one that "gives up infinities", so E5M2 keeps them).

Encoding rule
-------------
The encoder is the definition itself: the representable value nearest to the
input, ties going to the code whose mantissa is even (round half to even, as
the page's Python simulation states), saturating: every magnitude at or above
the largest finite value (including infinity) becomes that largest value (the
saturating mode of OCP FP8 conversion, described on the "Quantization: FP8
inference and KV-cache quantization" page under "Dynamic scales or static
scales").  The sign is kept, so -0 and negative values that round to zero give
the negative-zero code.  NaN gives the NaN code with the input's sign bit.

Everything here is computed in float64, where all the grid values and the
midpoints between neighbouring grid values are exact.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Fp8Format", "E4M3", "E5M2", "FORMATS", "decode", "encode", "bf16_round_bits",
           "bf16_bits_to_f64", "f32_from_bf16_bits"]


@dataclass(frozen=True)
class Fp8Format:
    name: str
    ebits: int
    mbits: int
    bias: int
    has_inf: bool
    values: np.ndarray = field(repr=False, compare=False)  # float64 [256], NaN where the code is NaN
    max_code: int = 0          # code of the largest finite positive value
    nan_code: int = 0x7F       # positive NaN code produced by the encoder

    @property
    def max_finite(self) -> float:
        return float(self.values[self.max_code])


def _decode_code(code: int, ebits: int, mbits: int, bias: int, has_inf: bool) -> float:
    """Value of one 8-bit code from the sign/exponent/mantissa fields."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    e_all_ones = (1 << ebits) - 1
    if has_inf:
        # IEEE-style: the all-ones exponent holds infinity (m == 0) and NaNs.
        if e == e_all_ones:
            return sign * np.inf if m == 0 else np.nan
    else:
        # "fn" variant: only all-ones exponent AND all-ones mantissa is NaN.
        if e == e_all_ones and m == (1 << mbits) - 1:
            return np.nan
    if e == 0:
        # subnormal: 0.m * 2^(1 - bias)
        return sign * (m / (1 << mbits)) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)


def _make_format(name: str, ebits: int, mbits: int, bias: int, has_inf: bool) -> Fp8Format:
    vals = np.array([_decode_code(c, ebits, mbits, bias, has_inf) for c in range(256)], dtype=np.float64)
    pos = vals[:128]
    finite = np.isfinite(pos)
    max_code = int(np.nonzero(finite)[0].max())
    return Fp8Format(name, ebits, mbits, bias, has_inf, vals, max_code, 0x7F)


E4M3 = _make_format("e4m3fn", 4, 3, 7, False)
E5M2 = _make_format("e5m2", 5, 2, 15, True)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2}


def decode(codes: np.ndarray, fmt: Fp8Format = E4M3) -> np.ndarray:
    """Codes (uint8) -> float64 values (exact)."""
    return fmt.values[np.asarray(codes, dtype=np.uint8)]


def _grid(fmt: Fp8Format):
    # Positive finite grid, codes 0 .. max_code, strictly increasing with the code.
    g = fmt.values[: fmt.max_code + 1].copy()
    assert np.all(np.diff(g) > 0)
    mids = (g[:-1] + g[1:]) / 2.0  # exact in float64 (grid values have <= 4 significant bits)
    return g, mids


_GRIDS = {id(E4M3): _grid(E4M3), id(E5M2): _grid(E5M2)}


def encode(t: np.ndarray, fmt: Fp8Format = E4M3) -> np.ndarray:
    """Saturating round-to-nearest-even encoding of float32 (or float64) values.

    Returns uint8 codes with the shape of ``t``.
    """
    t = np.asarray(t)
    grid, mids = _GRIDS[id(fmt)]
    with np.errstate(invalid="ignore"):
        a = np.abs(t.astype(np.float64))
    nan = np.isnan(a)
    a_safe = np.where(nan, 0.0, a)
    # index of the first midpoint >= a: candidates are grid[i] (below) and grid[i+1] (above)
    i = np.searchsorted(mids, a_safe, side="left")
    i = np.minimum(i, len(grid) - 1)
    # a < mids[i]  -> grid[i] is nearest;  a == mids[i] -> tie
    at_top = i >= len(mids)
    m_i = np.where(at_top, np.inf, mids[np.minimum(i, len(mids) - 1)])
    tie = (a_safe == m_i)
    code = i.astype(np.int64)
    # On a tie between codes i and i+1 the even one wins.
    code = np.where(tie & (code % 2 == 1), code + 1, code)
    # saturation: every magnitude >= the largest finite value
    code = np.where(a_safe >= fmt.max_finite, fmt.max_code, code)
    code = np.where(nan, fmt.nan_code, code)
    sign = np.signbit(t).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


# --------------------------------------------------------------------------- bf16

BF16_MAX = float.fromhex("0x1.fep+127")


def bf16_round_bits(v: np.ndarray) -> np.ndarray:
    """float64 (or float32) values -> bf16 bit patterns, round to nearest even.

    bf16 has 8 significant bits (1 implicit + 7 stored), exponent range as
    float32.  The rounding quantum of a normal value in [2^e, 2^(e+1)) is
    2^(e-7); below 2^-126 it is the subnormal quantum 2^-133.  A magnitude whose
    rounded value exceeds the largest finite bf16 overflows to infinity.
    NaN becomes the quiet NaN 0x7FC0 with the input's sign.
    """
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    inf = np.isinf(v)
    a = np.where(nan | inf, 0.0, np.abs(v))
    _, ex = np.frexp(a)               # a = f * 2^ex, f in [0.5, 1)
    e = ex - 1                        # a in [2^e, 2^(e+1))
    e = np.maximum(e, -126)           # subnormal range shares the 2^-126 binade's quantum
    quantum = np.ldexp(1.0, e - 7)
    r = np.rint(a / quantum) * quantum   # np.rint: round half to even; a/quantum is an exact scaling
    r = np.where(a == 0, 0.0, r)
    over = r > BF16_MAX
    with np.errstate(over="ignore"):
        r32 = np.where(over, 0.0, r).astype(np.float32)   # exact: r is a bf16 value
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint32)
    bits = np.where(over | inf, np.uint32(0x7F80), bits)
    bits = np.where(nan, np.uint32(0x7FC0), bits)
    sign = np.signbit(v).astype(np.uint32) << np.uint32(15)
    return (bits | sign).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(b).astype(np.float64)
