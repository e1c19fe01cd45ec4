"""GPU parity of the FP8 KV-cache calls against the CPU oracle (bit-exact),
through the C ABI."""

import numpy as np
import pytest
import torch

from gpu_util import assert_codes_equal, dev, dev_bf16, host, host_bits16, require_gpu
from oracle import kv as okv
from oracle import native
from oracle.fp8 import E4M3, E5M2
from workloads import f32_from_bf16_bits, kv_append_inputs, kv_inputs

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402

FMTS = {"e4m3": E4M3, "e5m2": E5M2}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def dequant_equal(got_bits, want_bits, codes, fmt, what):
    """bf16 bit-exact, except that any NaN is a correct dequantization of a NaN code."""
    nan_code = np.isnan(fmt.values[codes])
    diff = (got_bits != want_bits) & ~nan_code
    assert not diff.any(), f"{what}: {int(diff.sum())} bf16 values differ"
    if nan_code.any():
        g = got_bits[nan_code]
        assert (((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)).all(), f"{what}: NaN code not dequantized to NaN"


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(2, 48, 4, 32), (3, 257, 8, 128), (1, 5, 3, 16), (2, 64, 300, 16)])
def test_calibrate_quant_dequant_small(name, shape):
    fmt = FMTS[name]
    b, s, h, d = shape
    k, v, kc, vc = kv_inputs(sum(shape), b=b, s=s, h=h, d=d, n_out=max(1, (h * d) // 100))
    for t in (k, v):
        x = dev_bf16(t)
        sc = sg.fp8_kv_calibrate(x, name)
        sc_ref = okv.kv_calibrate(t, fmt)
        q = sg.fp8_kv_quant(x, sc, name)
        dq = sg.fp8_kv_dequant(q, sc, name)
        torch.cuda.synchronize()
        assert np.array_equal(host(sc).view(np.uint32), sc_ref.view(np.uint32)), f"{shape} {name} scales"
        q_ref = okv.kv_quant(t, sc_ref, fmt)
        assert_codes_equal(host(q), q_ref, f"{shape} {name} quant")
        dq_ref = okv.kv_dequant(q_ref, sc_ref, fmt)
        dequant_equal(host_bits16(dq), dq_ref, q_ref, fmt, f"{shape} {name} dequant")


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_quant_given_scales_with_specials(name):
    """Unit and tiny/huge per-head scales, saturation, infinities and NaN."""
    fmt = FMTS[name]
    b, s, h, d = 2, 40, 4, 32
    rng = np.random.default_rng(8)
    x = (rng.standard_t(2, (b, s, h, d)) * 30).astype(np.float32)
    from workloads import bf16_bits_from_f32
    t = bf16_bits_from_f32(x)
    t[0, 0, 0, :8] = [0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x0000, 0x8000, 0x0001, 0x8001]
    scales = np.float32([1.0, 1e-30, 3e20, 0.0123])
    q = sg.fp8_kv_quant(dev_bf16(t), dev(scales), name)
    torch.cuda.synchronize()
    q_ref = okv.kv_quant(t, scales, fmt)
    nan = np.isnan(f32_from_bf16_bits(t))
    assert_codes_equal(host(q), q_ref, f"{name} specials", nan_ok_mask=nan)
    dq = sg.fp8_kv_dequant(dev(q_ref), dev(scales), name)
    torch.cuda.synchronize()
    dequant_equal(host_bits16(dq), okv.kv_dequant(q_ref, scales, fmt), q_ref, fmt, f"{name} dequant specials")


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_dequant_every_code(name):
    fmt = FMTS[name]
    codes = np.tile(np.arange(256, dtype=np.uint8), 16).reshape(1, 16, 2, 128)
    scales = np.float32([0.0071428571, 3.5])
    dq = sg.fp8_kv_dequant(dev(codes), dev(scales), name)
    torch.cuda.synchronize()
    dequant_equal(host_bits16(dq), okv.kv_dequant(codes, scales, fmt), codes, fmt, f"{name} all codes")


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_full_size_sampled(name):
    """The full cache shape [8, 32768, 8, 128]: per-head scales checked in full
    (the oracle's maximum over the whole tensor), codes and dequantized values on
    512 sampled (b, s) rows of every head."""
    fmt = FMTS[name]
    k, v, kc, vc = kv_inputs(0)
    rng = np.random.default_rng(1)
    bs = rng.integers(0, 8, 512)
    ss = rng.integers(0, 32768, 512)
    for t in (k, v):
        x = dev_bf16(t)
        sc = sg.fp8_kv_calibrate(x, name)
        q = sg.fp8_kv_quant(x, sc, name)
        dq = sg.fp8_kv_dequant(q, sc, name)
        torch.cuda.synchronize()
        sc_ref = okv.kv_calibrate(t, fmt)
        assert np.array_equal(host(sc).view(np.uint32), sc_ref.view(np.uint32)), f"{name} scales"
        qs = host(q[torch.from_numpy(bs).cuda(), torch.from_numpy(ss).cuda()])
        sample = t[bs, ss]  # [512, H, D]
        q_ref = okv.kv_quant(sample[:, None], sc_ref, fmt)[:, 0]
        assert_codes_equal(qs, q_ref, f"{name} sampled codes")
        dqs = host_bits16(dq[torch.from_numpy(bs).cuda(), torch.from_numpy(ss).cuda()])
        dequant_equal(dqs, okv.kv_dequant(q_ref[:, None], sc_ref, fmt)[:, 0], q_ref, fmt, f"{name} sampled dequant")
        # saturation count over the whole tensor equals the oracle's rule (C oracle, all elements)
        del x, q, dq


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_full_size_quant_all_elements(name):
    """Every code of the full K tensor against the C oracle (per-head scales)."""
    fmt = FMTS[name]
    k, _, _, _ = kv_inputs(0)
    x = dev_bf16(k)
    sc = sg.fp8_kv_calibrate(x, name)
    q = host(sg.fp8_kv_quant(x, sc, name))
    sc_h = host(sc)
    want = native.quant_grouped_scale_f32(f32_from_bf16_bits(k).ravel(), sc_h, 128, name).reshape(k.shape)
    assert_codes_equal(q, want, f"{name} full K")


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_append(name):
    fmt = FMTS[name]
    b, s, h, d = 8, 64, 8, 128
    k, v, kc, vc = kv_inputs(3, b=b, s=s, h=h, d=d)
    kn, vn = kv_append_inputs(kc, vc, seed=3, b=b, h=h, d=d)
    sc = okv.kv_calibrate(k, fmt)
    cache = np.full((b, s + 1, h, d), 0xA5, np.uint8)
    cache[:, :s] = okv.kv_quant(k, sc, fmt)
    pos = np.int32([s, 0, 5, s, -1, s + 1, 63, 2 ** 30])  # the last three sequences are out of range or last
    cache_t = dev(cache)
    sg.fp8_kv_append(dev_bf16(kn), dev(pos), dev(sc), cache_t, name)
    torch.cuda.synchronize()
    valid = (pos >= 0) & (pos < s + 1)
    want = cache.copy()
    codes = okv.kv_quant(kn[:, None], sc, fmt)[:, 0]
    for i in range(b):
        if valid[i]:
            want[i, pos[i]] = codes[i]
    assert_codes_equal(host(cache_t), want, f"{name} append")


def test_append_full_shape_latency_path():
    """Config shape: 8 sequences, cache capacity 32769, append at 32768."""
    k, v, kc, vc = kv_inputs(0, s=64)
    kn, vn = kv_append_inputs(kc, vc)
    sc = okv.kv_calibrate(k, E4M3)
    cache_t = torch.zeros((8, 32769, 8, 128), dtype=torch.uint8, device="cuda")
    pos = np.full(8, 32768, np.int32)
    sg.fp8_kv_append(dev_bf16(kn), dev(pos), dev(sc), cache_t, "e4m3")
    torch.cuda.synchronize()
    got = host(cache_t[:, 32768])
    want = okv.kv_quant(kn[:, None], sc, E4M3)[:, 0]
    assert_codes_equal(got, want, "append at 32768")
    assert int(cache_t[:, :32768].count_nonzero()) == 0
