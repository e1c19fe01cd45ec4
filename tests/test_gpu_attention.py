"""GPU parity of fp8_kv_decode_attention against the CPU oracle
(oracle/attention.py), through the C ABI.

The cache is produced by the library's own calibrate + quantize calls (their
codes and scales are bit-exact with the oracle, tests/test_gpu_kv.py), so the
oracle and the kernel read the same codes.

Tolerance (derived from the kernel's arithmetic): every score is an fp32 sum of
128 exact products times two fp32 scale factors, the exponentials take
arguments up to ~90 in magnitude (relative error of exp ~ |x| 2^-24 plus one
ulp), and each output is an fp32 sum of at most 256 terms per wave, then 8 lane,
4 wave and chunk combinations; together under 5e-5 of W = sum_t p_t |V_t,d|.
The test allows |o - o_exact| <= 1e-4 W for the fp32 output, and one more bf16
ulp of o_exact for the bf16 output.
"""

import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, host_bits16, require_gpu
from oracle import attention as at
from oracle import fp8
from oracle.fp8 import E4M3, E5M2
from workloads import attention_queries, f32_from_bf16_bits, kv_inputs

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402

TOL = 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def bf16_ulp(y):
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e, -126) - 7)


def make_cache(b, s, h, fmt, seed=0):
    k, v, _, _ = kv_inputs(seed, b=b, s=s, h=h, d=128)
    kt, vt = dev_bf16(k), dev_bf16(v)
    sk = sg.fp8_kv_calibrate(kt, fmt)
    sv = sg.fp8_kv_calibrate(vt, fmt)
    kq = sg.fp8_kv_quant(kt, sk, fmt)
    vq = sg.fp8_kv_quant(vt, sv, fmt)
    torch.cuda.synchronize()
    del kt, vt
    return kq, vq, sk, sv


def check(q_bits, kq, vq, sk, sv, lengths, fmt, heads=None, scale=None, what=""):
    qt = dev_bf16(q_bits)
    Lt = dev(np.asarray(lengths, np.int32))
    o16 = sg.fp8_kv_decode_attention(qt, kq, vq, sk, sv, Lt, fmt, scale=scale)
    o32 = sg.fp8_kv_decode_attention(qt, kq, vq, sk, sv, Lt, fmt, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ofmt = E4M3 if fmt == "e4m3" else E5M2
    qf = f32_from_bf16_bits(q_bits)
    kqh, vqh, skh, svh = host(kq), host(vq), host(sk), host(sv)
    exact = at.attention_decode(qf, kqh, vqh, skh, svh, lengths, ofmt, scale, heads)
    W = at.attention_abs_weight(qf, kqh, vqh, skh, svh, lengths, ofmt, scale, heads)
    B, Hq, D = q_bits.shape
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    bi = np.array([p[0] for p in pairs])
    hi = np.array([p[1] for p in pairs])
    ex, w = exact[bi, hi], W[bi, hi]
    g32 = host(o32)[bi, hi].astype(np.float64)
    err = np.abs(g32 - ex)
    bad = err > TOL * w
    assert not bad.any(), f"{what}: fp32 output outside {TOL} W at {int(bad.sum())}; worst {np.max(err / np.maximum(w, 1e-30)):.3g} W"
    g16 = fp8.bf16_bits_to_f64(host_bits16(o16)[bi, hi])
    ref = fp8.bf16_bits_to_f64(fp8.bf16_round_bits(ex))
    d16 = np.abs(g16 - ex)
    bad = d16 > bf16_ulp(ref) + TOL * w
    assert not bad.any(), f"{what}: bf16 output beyond 1 ulp + {TOL} W at {int(bad.sum())}"
    empty = np.asarray(lengths)[bi] == 0
    assert (g32[empty] == 0).all() and (g16[empty] == 0).all()
    return o16, o32


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_small_ragged_lengths(fmt):
    kq, vq, sk, sv = make_cache(4, 2100, 8, fmt)
    q = attention_queries(1, b=4)
    check(q, kq, vq, sk, sv, np.array([2100, 1, 1024, 1025]), fmt, what=f"small {fmt}")
    check(q, kq, vq, sk, sv, np.array([0, 2049, 63, 64]), fmt, what=f"small {fmt} (2)")
    check(q, kq, vq, sk, sv, np.array([7, 1023, 2048, 2100 + 50]), fmt, what=f"small {fmt} (clamped)")


@pytest.mark.parametrize("G", [1, 2, 8])
def test_query_group_sizes(G):
    kq, vq, sk, sv = make_cache(2, 700, 4, "e4m3", seed=3)
    q = attention_queries(2, b=2, hq=4 * G)
    check(q, kq, vq, sk, sv, np.array([700, 333]), "e4m3", what=f"G={G}")


def test_explicit_softmax_scale():
    kq, vq, sk, sv = make_cache(2, 500, 8, "e4m3", seed=4)
    q = attention_queries(3, b=2)
    check(q, kq, vq, sk, sv, np.array([500, 200]), "e4m3", scale=0.02, what="scale 0.02")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_full_size_sampled(fmt):
    """The KV-cache workload's shape, [8, 32768, 8, 128], 32 query heads; sampled (b, h)."""
    kq, vq, sk, sv = make_cache(8, 32768, 8, fmt)
    q = attention_queries(0)
    rng = np.random.default_rng(7)
    heads = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, 8, 10), rng.integers(0, 32, 10))} | {(0, 0), (7, 31)})
    lengths = np.array([32768, 32768, 30000, 32768, 1, 32768, 16385, 32768])
    o16, _ = check(q, kq, vq, sk, sv, lengths, fmt, heads=heads, what=f"full {fmt}")
    # the same call again gives the same bits
    again = sg.fp8_kv_decode_attention(dev_bf16(q), kq, vq, sk, sv, dev(lengths.astype(np.int32)), fmt)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), o16.view(torch.int16))
