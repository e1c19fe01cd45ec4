"""Pins for the oracle's FP8 formats, encoder and bf16 rounding (CPU only).

Each check ties the oracle to something other than itself: the pages' printed
facts (tests/golden), brute-force nearest-value enumeration, PyTorch's own
float8/bfloat16 conversions where they coincide with the saturating rule, and
exact rational arithmetic.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import parse_num, read_golden
from exact import nearest_bf16
from oracle import fp8, native
from oracle.fp8 import E4M3, E5M2

FMTS = {"e4m3": E4M3, "e5m2": E5M2}


def all_bf16_as_f32():
    b = np.arange(1 << 16, dtype=np.uint32)
    return (b << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ page facts

def test_golden_format_facts():
    for row in read_golden("e4m3_format_facts.txt"):
        if row[0] == "steps":
            fmt = FMTS[row[1]]
            per_binade = 1 << fmt.mbits
            assert per_binade == int(row[2])
            # codes sharing one normal exponent field, all distinct values, evenly spaced
            e_field = 1 << fmt.mbits  # exponent field 1
            vals = fmt.values[e_field: e_field + per_binade]
            assert np.allclose(np.diff(vals), vals[1] - vals[0])
            continue
        fmt = FMTS[row[0]]
        v = parse_num(row[1])
        code = int(row[2], 16)
        assert fp8.encode(np.float32([v]), fmt)[0] == code, row
        if v != 95:
            assert fp8.decode(np.uint8([code]), fmt)[0] == v, row


def test_96_bit_fields():
    # 96 = sign 0, exponent bits 1101, mantissa bits 100
    c = int(fp8.encode(np.float32([96.0]), E4M3)[0])
    assert c >> 7 == 0 and (c >> 3) & 0xF == 0b1101 and c & 7 == 0b100


def test_e4m3_has_no_infinity_and_two_nans():
    vals = E4M3.values
    assert not np.isinf(vals).any()
    nans = np.nonzero(np.isnan(vals))[0]
    assert list(nans) == [0x7F, 0xFF]
    assert np.isfinite(vals).sum() == 254
    assert E4M3.max_finite == 448.0
    assert vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9


def test_e5m2_specials():
    vals = E5M2.values
    assert vals[0x7B] == 57344.0 and vals[0x7C] == np.inf and vals[0xFC] == -np.inf
    assert np.isnan(vals[[0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]]).all()
    assert np.isfinite(vals).sum() == 248


def test_spacing_and_worst_relative_error():
    facts = {r[0]: float(r[1]) for r in read_golden("spacing_facts.txt")}
    # spacing within a binade relative to its start
    start = E4M3.values[0x38]  # 1.0
    assert (E4M3.values[0x39] - start) / start == facts["spacing_rel"]
    # worst-case relative rounding error over normal values, by a dense sweep
    x = np.float32(np.linspace(2.0 ** -6, 440.0, 2_000_001))
    r = fp8.decode(fp8.encode(x, E4M3), E4M3)
    rel = np.abs(r - x) / np.abs(x)
    assert rel.max() <= 1 / 16
    assert round(rel.max(), 2) == facts["worst_relerr_about"]


# ------------------------------------------------------------ decode vs torch

@pytest.mark.parametrize("name,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_decode_matches_torch_for_all_codes(name, tdt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(tdt).to(torch.float64).numpy()
    ours = fp8.decode(np.arange(256, dtype=np.uint8), FMTS[name])
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(np.where(both_nan, 0, ref), np.where(both_nan, 0, ours))


# ---------------------------------------------- encoder vs brute force / torch

def brute_force_encode(t, fmt):
    """Nearest finite value by scanning every code; ties to the even code."""
    vals = fmt.values[: fmt.max_code + 1]
    out = []
    for v in np.asarray(t, dtype=np.float64):
        if np.isnan(v):
            out.append(None)
            continue
        a = min(abs(v), fmt.max_finite)
        d = np.abs(vals - a)
        best = np.nonzero(d == d.min())[0]
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        if np.signbit(v):
            c |= 0x80
        out.append(c)
    return out


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_encoder_brute_force_all_bf16_patterns(name):
    fmt = FMTS[name]
    x = all_bf16_as_f32()
    ours = fp8.encode(x, fmt)
    ref = brute_force_encode(x, fmt)
    for i, (o, r) in enumerate(zip(ours, ref)):
        if r is None:
            assert o & 0x7F == 0x7F
        else:
            assert o == r, (hex(x.view(np.uint32)[i]), hex(o), hex(r))


@pytest.mark.parametrize("name,tdt,lim", [("e4m3", torch.float8_e4m3fn, 464.0),
                                          ("e5m2", torch.float8_e5m2, 61440.0)])
def test_encoder_matches_torch_inside_range(name, tdt, lim):
    """torch's float8 cast is round-to-nearest-even but not saturating; below the
    first out-of-range midpoint the two rules coincide."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < lim)]
    x = np.concatenate([x, all_bf16_as_f32()])
    x = x[np.isfinite(x) & (np.abs(x) < lim)]
    ref = torch.from_numpy(x).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(x, FMTS[name]), ref)


def test_encoder_saturates_and_keeps_sign():
    big = np.float32([448.0, 449.0, 463.99, 464.0, 672.0, 1e30, np.inf])
    assert (fp8.encode(big, E4M3) == 0x7E).all()
    assert (fp8.encode(-big, E4M3) == 0xFE).all()
    big5 = np.float32([57344.0, 59391.0, 59392.0, 61440.0, 1e38, np.inf])
    assert (fp8.encode(big5, E5M2) == 0x7B).all()
    assert fp8.encode(np.float32([-0.0]), E4M3)[0] == 0x80
    assert fp8.encode(np.float32([-1e-30]), E4M3)[0] == 0x80
    assert fp8.encode(np.float32([np.nan]), E4M3)[0] == 0x7F
    assert fp8.encode(-np.float32([np.nan]), E4M3)[0] == 0xFF


def test_ties_go_to_even():
    # midpoint between 1.0 (0x38) and 1.125 (0x39) -> 1.0 ; between 1.125 and 1.25 -> 1.25 (0x3A)
    assert fp8.encode(np.float32([1.0625, 1.1875]), E4M3).tolist() == [0x38, 0x3A]
    # subnormal/zero tie 2^-10 -> 0 ; 3*2^-10 between 2^-9 and 2^-8 -> 2^-8 (code 2)
    assert fp8.encode(np.float32([2.0 ** -10, 3 * 2.0 ** -10]), E4M3).tolist() == [0x00, 0x02]


def test_c_oracle_matches_numpy_oracle():
    x = all_bf16_as_f32()
    rng = np.random.default_rng(3)
    y = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    for name, fmt in FMTS.items():
        for arr in (x, y):
            assert np.array_equal(native.encode_f32(arr, name), fp8.encode(arr, fmt))
        start = 0x43E00000 - 5000
        pat = native.encode_bit_patterns(start, 10000, name)
        vals = (np.arange(start, start + 10000, dtype=np.uint64).astype(np.uint32)).view(np.float32)
        assert np.array_equal(pat, fp8.encode(vals, fmt))


# --------------------------------------------------------------------- bf16

def test_bf16_rounding_matches_torch_on_float32():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, size=3_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fp8.bf16_round_bits(x), ref)


def test_bf16_rounding_of_float64_is_single_rounding():
    # A float64 value just above a bf16 midpoint must round up, even though a
    # detour through float32 would land on the midpoint and round to even.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    b = fp8.bf16_round_bits(np.float64([v]))[0]
    assert fp8.f32_from_bf16_bits(np.uint16([b]))[0] == 1.0 + 2.0 ** -7
    rng = np.random.default_rng(5)
    vals = rng.standard_normal(20000) * np.exp2(rng.integers(-100, 100, 20000))
    ours = fp8.bf16_bits_to_f64(fp8.bf16_round_bits(vals))
    for v, o in zip(vals, ours):
        assert Fraction(float(o)) == nearest_bf16(Fraction(float(v)))


def test_bf16_overflow_and_specials():
    out = fp8.bf16_round_bits(np.float64([3.39e38, 3.4e38, -np.inf, np.nan, -0.0]))
    assert out.tolist() == [0x7F7F, 0x7F80, 0xFF80, 0x7FC0, 0x8000]
