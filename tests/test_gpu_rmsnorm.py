"""GPU parity of fp8_rmsnorm_quant_per_token (RMSNorm with the per-token
quantization fused into it) against the CPU oracle, through the C ABI.

* The fp32 normalised rows (y_out) against the float64 definition
  (oracle/norm.py).  Tolerance from the kernel's arithmetic: the sum of
  squares takes 16 * ceil(K / 4096) sequential fused multiply-adds per thread
  (16-element units, 256 threads), then a 6-level wave tree and 2 levels across
  waves, all of positive terms, so its relative error is below
  (16 ceil(K / 4096) + 8) 2^-24; the square root halves it; the mean, the
  addition of eps, the square root, the reciprocal and the two products add one
  rounding each:
      |y - y_exact| <= ((16 ceil(K / 4096) + 8) / 2 + 6) 2^-24 |y_exact|.
* Codes and scales: the quantization is a decision taken on the kernel's fp32
  y, so it is checked in that precision: bit for bit equal to the oracle's
  per-token quantizer applied to y_out.  Without y_out the codes are the same.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_codes_equal, dev, dev_bf16, host, require_gpu
from oracle import norm, w8a8
from test_abi_host import pack_reference
from workloads import bf16_bits_from_f32, decode_inputs, f32_from_bf16_bits, prefill_inputs

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _gamma(K, seed=0):
    g = (1.0 + 0.1 * np.random.default_rng(seed).standard_normal(K)).astype(np.float32)
    return g


def check(x_host, g_host, eps, *, layout="row_major", what=""):
    is_bf16 = x_host.dtype == np.uint16
    if is_bf16:
        xt, gt = dev_bf16(x_host), dev_bf16(g_host)
        xf, gf = f32_from_bf16_bits(x_host), f32_from_bf16_bits(g_host)
    else:
        xt, gt = dev(x_host), dev(g_host)
        xf, gf = x_host, g_host
    M, K = xf.shape
    y = torch.empty((M, K), dtype=torch.float32, device="cuda")
    q, s = sg.fp8_rmsnorm_quant_per_token(xt, gt, eps, layout=layout, y_out=y)
    q2, s2 = sg.fp8_rmsnorm_quant_per_token(xt, gt, eps, layout=layout)
    torch.cuda.synchronize()
    yh = host(y)
    exact = norm.rmsnorm(xf, gf, eps)
    tol = ((16 * -(-K // 4096) + 8) / 2 + 6) * 2.0 ** -24
    err = np.abs(yh.astype(np.float64) - exact)
    bad = err > tol * np.abs(exact)
    assert not bad.any(), f"{what}: {int(bad.sum())} normalised values outside {tol:.3g} relative"
    want_q, want_s = w8a8.quant_per_token(yh)
    qh = host(q)
    if layout == "packed":
        want_q = pack_reference(want_q)[:qh.size].reshape(qh.shape)
        live = pack_reference(np.ones((M, K), np.uint8)).astype(bool)
        qh, want_q = qh[live], want_q[live]
    assert np.array_equal(host(s), want_s), f"{what}: scales differ"
    assert_codes_equal(qh, want_q, what)
    assert np.array_equal(host(q2), host(q)) and np.array_equal(host(s2), host(s)), f"{what}: y_out changed the codes"


@pytest.mark.parametrize("m", [1, 8, 32])
def test_decode_rows_bf16(m):
    xb, _, _ = decode_inputs(m, with_weight=False)
    check(xb, bf16_bits_from_f32(_gamma(4096)), 1e-6, what=f"decode M={m}")


def test_prefill_rows_bf16_both_layouts():
    xb, _, _ = prefill_inputs(4096, m=512, n=16, with_weight=False)
    g = bf16_bits_from_f32(_gamma(4096, 1))
    check(xb, g, 1e-5, what="prefill rows")
    check(xb, g, 1e-5, layout="packed", what="prefill rows packed")


@pytest.mark.parametrize("K", [16, 144, 2048, 4096, 16384])
def test_fp32_rows_of_every_length(K):
    rng = np.random.default_rng(K)
    x = rng.standard_normal((5, K)).astype(np.float32)
    x[:, rng.integers(0, K, 2)] *= 50
    x[4] = 0.0                                     # a zero row: y = 0, scale 1.0
    for eps in (0.0, 1e-6, 1e-2):
        if eps == 0.0:
            check(x[:4], _gamma(K, 2), eps, what=f"K={K} eps=0")
        else:
            check(x, _gamma(K, 2), eps, what=f"K={K} eps={eps}")


def test_errors():
    lib = sg.lib()
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    q = torch.empty((4, 128), dtype=torch.uint8, device="cuda")
    s = torch.empty(4, dtype=torch.float32, device="cuda")
    f = lib.fp8_rmsnorm_quant_per_token
    assert f(x.data_ptr(), sg.BF16, g.data_ptr(), 1e-6, 4, 20000, q.data_ptr(), s.data_ptr(), None, 0, None) == 2
    assert f(x.data_ptr(), sg.BF16, g.data_ptr(), -1.0, 4, 128, q.data_ptr(), s.data_ptr(), None, 0, None) == 2
    assert f(x.data_ptr(), sg.BF16, g.data_ptr(), float("nan"), 4, 128, q.data_ptr(), s.data_ptr(), None, 0, None) == 2
    assert f(x.data_ptr(), sg.BF16, None, 1e-6, 4, 128, q.data_ptr(), s.data_ptr(), None, 0, None) == 1
    assert f(x.data_ptr(), sg.E4M3, g.data_ptr(), 1e-6, 4, 128, q.data_ptr(), s.data_ptr(), None, 0, None) == 4
