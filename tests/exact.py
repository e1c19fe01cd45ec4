"""Exact-rational helpers for the oracle pins (test code only)."""

import math
from fractions import Fraction

import numpy as np


def nearest_f32(q: Fraction) -> np.float32:
    """Nearest float32 to a rational, ties to even, by bracketing with nextafter.
    Magnitudes at or beyond the midpoint between FLT_MAX and 2^128 overflow."""
    if abs(q) >= Fraction(2) ** 128 - Fraction(2) ** 103:
        return np.float32(np.inf) if q > 0 else np.float32(-np.inf)
    c = np.float32(float(q))  # within one float32 step of q
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - q)
        key = (d, int(np.float32(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def nearest_bf16(v: Fraction) -> Fraction:
    """Nearest bf16 value to a rational (finite range), ties to even."""
    a = abs(v)
    if a == 0:
        return Fraction(0)
    e = math.floor(math.log2(a))
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    return -r if v < 0 else r
