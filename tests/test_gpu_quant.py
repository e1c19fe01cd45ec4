"""GPU parity of the FP8 quantizers against the CPU oracle (bit-exact codes and
scales), through the C ABI."""

import numpy as np
import pytest
import torch

from gpu_util import assert_codes_equal, dev, dev_bf16, host, require_gpu
from oracle import fp8, native, w8a8
from oracle.fp8 import E4M3, E5M2
from workloads import (bf16_bits_from_f32, decode_inputs, f32_from_bf16_bits, large_layer_inputs, prefill_inputs,
                       tiny_w8a8)

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def check_per_token_bf16(xb, what):
    x = f32_from_bf16_bits(xb)
    q_ref, s_ref = w8a8.quant_per_token(x)
    q, s = sg.fp8_quant_per_token(dev_bf16(xb))
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32)), f"{what}: scales differ"
    assert_codes_equal(host(q), q_ref, what)


def test_per_token_tiny_fp32():
    x, _ = tiny_w8a8(0)
    q_ref, s_ref = w8a8.quant_per_token(x)
    q, s = sg.fp8_quant_per_token(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert_codes_equal(host(q), q_ref, "tiny fp32 per-token")


@pytest.mark.parametrize("m", [1, 8, 32])
def test_per_token_decode_shapes(m):
    xb, _, _ = decode_inputs(m, with_weight=False)
    check_per_token_bf16(xb, f"decode M={m}")


@pytest.mark.parametrize("k", [16, 48, 256, 4096, 8192, 14336, 16384, 20480, 65536])
def test_per_token_row_lengths(k):
    """Row lengths covering every register-resident variant, a ragged last chunk
    set and the two-pass streaming kernel (k > 16384)."""
    rng = np.random.default_rng(k)
    m = 37
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.integers(0, k, 3)] *= 40
    check_per_token_bf16(bf16_bits_from_f32(x), f"K={k}")


def test_per_token_prefill_rows():
    xb, _, _ = prefill_inputs(4096, m=512, with_weight=False)
    check_per_token_bf16(xb, "prefill K=4096 (512 rows)")
    xb, _, _ = prefill_inputs(14336, m=256, with_weight=False)
    check_per_token_bf16(xb, "prefill K=14336 (256 rows)")


def test_per_token_student_t():
    xb, _ = large_layer_inputs(m=256, with_weight=False)
    check_per_token_bf16(xb, "student-t rows")


def test_per_token_edge_rows():
    """Zero rows (scale 1.0), signed zeros, rows so small that their scale leaves
    [2^-60, 2^60] (exact-division fallback), huge rows, a row whose maximum sits
    at the last element, and bf16 subnormals."""
    k = 64
    rows = []
    rows.append(np.zeros(k, np.float32))
    r = np.zeros(k, np.float32); r[::2] = -0.0; rows.append(r)
    rng = np.random.default_rng(3)
    for scale in (1e-30, 1e-38, 3e-39, 2.0 ** -120, 1e25, 3e38, 1.0, 448.0):
        rows.append((rng.standard_normal(k) * scale).astype(np.float32))
    r = rng.standard_normal(k).astype(np.float32); r[-1] = 1000.0; rows.append(r)
    r = np.float32([2.0 ** -133 * i for i in range(k)]); rows.append(r)
    r = np.float32([-(2.0 ** -130) * i for i in range(k)]); rows.append(r)
    x = np.stack(rows)
    xb = bf16_bits_from_f32(x)
    check_per_token_bf16(xb, "edge rows bf16")
    # fp32 inputs, including fp32 subnormals
    x32 = np.concatenate([f32_from_bf16_bits(xb), (rng.standard_normal((4, k)) * 1e-42).astype(np.float32)])
    q_ref, s_ref = w8a8.quant_per_token(x32)
    q, s = sg.fp8_quant_per_token(dev(x32))
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert_codes_equal(host(q), q_ref, "edge rows fp32")


def test_per_token_division_sweep():
    """Every finite bf16 magnitude below each row's maximum, against 96 row scales
    with random significands: exercises the exact-quotient scheme across
    (x, s) significand pairs."""
    allb = np.arange(1 << 15, dtype=np.uint16)  # non-negative bf16 patterns
    vals = f32_from_bf16_bits(allb)
    vals = vals[np.isfinite(vals)]
    rng = np.random.default_rng(12)
    rows = []
    for _ in range(96):
        amax = np.float32(np.exp2(rng.uniform(-20, 20)))
        amax = f32_from_bf16_bits(bf16_bits_from_f32(np.float32([amax])))[0]
        r = vals[(vals < amax) & (vals > amax * 2.0 ** -40)]
        r = np.resize(r, 16384)
        r[0] = amax
        sign = rng.integers(0, 2, r.size).astype(bool)
        r = np.where(sign, -r, r).astype(np.float32)
        rows.append(r)
    x = np.stack(rows)
    check_per_token_bf16(bf16_bits_from_f32(x), "division sweep")


def test_weight_per_channel_fp32():
    _, w = tiny_w8a8(0)
    q_ref, s_ref = w8a8.quant_weight_per_channel(w)
    q, s = sg.fp8_quant_weight_per_channel(dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert_codes_equal(host(q), q_ref, "tiny W")
    _, w, _ = decode_inputs(1, n=1024)
    q_ref, s_ref = w8a8.quant_weight_per_channel(w)
    q, s = sg.fp8_quant_weight_per_channel(dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert_codes_equal(host(q), q_ref, "W 1024x4096")


# --------------------------------------------------------------- static

SPECIALS = np.float32([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 1e38, -3e38, 1e-40, -1e-45, 448.0, 57344.0])


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("scale", [120.0 / 448.0, 1.0, 1e-3, 3.0, 1e-30, 1e25, 2.0 ** -100])
@pytest.mark.parametrize("numel", [16, 4099, 100000])
def test_static_bf16_and_fp32(fmt, scale, numel):
    rng = np.random.default_rng(numel)
    x = (rng.standard_t(3, numel) * np.float32(scale) * 200).astype(np.float32)
    x[: len(SPECIALS)] = SPECIALS[: min(len(SPECIALS), numel)]
    s = np.float32([scale])
    xb = bf16_bits_from_f32(np.where(np.isnan(x), 0, x).astype(np.float32))
    xb[: len(SPECIALS)] = bf16_bits_from_f32(np.nan_to_num(SPECIALS, nan=1.0))[: min(len(SPECIALS), numel)]
    if numel >= 6:
        xb[4] = 0x7FC0
        xb[5] = 0xFFC0
    name = "e4m3" if fmt is E4M3 else "e5m2"
    for inp, tensor in ((f32_from_bf16_bits(xb), dev_bf16(xb)), (x, dev(x))):
        want = w8a8.quant_static(inp, s[0], fmt)
        got = host(sg.fp8_quant_per_tensor_static(tensor, dev(s), fmt=name))
        torch.cuda.synchronize()
        assert_codes_equal(got, want, f"static {name} s={scale} n={numel}", nan_ok_mask=np.isnan(inp))
        if np.isnan(inp).any():
            assert (got[np.isnan(inp)] & 0x7F >= (0x7F if fmt is E4M3 else 0x7D)).all()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_static_all_bf16_patterns_many_scales(fmt):
    """All 65,536 bf16 patterns against 64 scales (C oracle)."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = f32_from_bf16_bits(allb)
    xt = dev_bf16(allb)
    rng = np.random.default_rng(21)
    scales = np.concatenate([np.float32([1.0, 120 / 448, 0.5, 1e-20, 1e20]),
                             np.exp2(rng.uniform(-50, 50, 59)).astype(np.float32)])
    nan = np.isnan(x)
    for s in scales:
        want = native.quant_given_scale_f32(x, float(s), fmt)
        got = host(sg.fp8_quant_per_tensor_static(xt, dev(np.float32([s])), fmt=fmt))
        assert_codes_equal(got, want, f"all bf16, s={s!r}", nan_ok_mask=nan)


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_static_unit_scale_every_float32_pattern(fmt):
    """With s = 1 the quotient is x itself, so this is the encoder on every one of
    the 2^32 float32 bit patterns (C oracle)."""
    chunk = 1 << 28
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    for start in range(0, 1 << 32, chunk):
        pat = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda")
        pat = torch.where(pat >= (1 << 31), pat - (1 << 32), pat).to(torch.int32)
        x = pat.view(torch.float32)
        got = host(sg.fp8_quant_per_tensor_static(x, one, fmt=fmt))
        want = native.encode_bit_patterns(start, chunk, fmt)
        nanmask = np.isnan(host(x))
        assert_codes_equal(got, want, f"float32 patterns from {start:#x}", nan_ok_mask=nanmask)
        del pat, x
