"""GPU parity of the GEMM's FP8 output epilogue (fp8_scaled_gemm_fp8out).

The codes are a quantization decision taken on the kernel's fp32 result, so
the check takes that decision in the same precision: for every output,
code == E4M3(RN32(y32 / s_out)) bit for bit (the oracle's static quantizer,
oracle/w8a8.py), where y32 is what fp8_scaled_gemm writes with fp32 output for
the same arguments (same kernel, same accumulator).  That fp32 result is
itself checked here against the oracle's exact product of the same codes and
scales: within the accumulator tolerance times |s_a s_w| plus the epilogue's
two float32 roundings (exact mode: 1e-5 sum|a w|; FP8 matrix cores: the bound
derived from their group alignment).  Output scales cover a calibrated scale,
saturation of most outputs, and underflow of most outputs to subnormal codes
and zero.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_codes_equal, dev, dev_bf16, host, require_gpu
from oracle import w8a8
from test_gpu_gemm import fp8_mfma_bound
from workloads import bf16_bits_from_f32, decode_inputs, f32_from_bf16_bits, prefill_inputs, tiny_w8a8

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def check_f32_result(ys, xf_rows, w_cols, accum, s_static, what):
    """The kernel's fp32 result against the oracle's exact product of the same
    codes and scales (the oracle quantizes the rows and weight channels itself)."""
    if s_static is None:
        aq, sa = w8a8.quant_per_token(xf_rows)
    else:
        aq = w8a8.quant_static(xf_rows, s_static)
        sa = np.full(xf_rows.shape[0], s_static, np.float32)
    wq, sw = w8a8.quant_weight_per_channel(w_cols)
    acc = w8a8.gemm_acc_exact(aq, wq)
    y_ex = w8a8.scaled_gemm_f64(acc, sa, sw)
    bound = 1e-5 * w8a8.gemm_abs_sum(aq, wq) if accum == "exact" else fp8_mfma_bound(aq, wq)
    s_abs = np.abs(np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :])
    b = bound * s_abs * (1 + 2.0 ** -22) + 2.0 ** -22 * np.abs(y_ex)
    err = np.abs(ys.astype(np.float64) - y_ex)
    assert (err <= b).all(), (f"{what}: fp32 result outside the scaled accumulator bound at {int((err > b).sum())} "
                              f"outputs; worst err/bound {np.max(err / np.maximum(b, 1e-300)):.3g}")


def run(xt, wq, sw, *, accum, layout, mode="per_token", sa=None, rows=None, cols=None, what="", xf=None, wf=None,
        s_static=None):
    M = xt.shape[0]
    N = sw.shape[0]
    kw = dict(accum=accum, w_layout=layout, a_scale_mode=mode)
    y32 = sg.fp8_scaled_gemm(xt, sa, wq, sw, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    y = host(y32)
    rows = np.arange(M) if rows is None else rows
    cols = np.arange(N) if cols is None else cols
    ys = y[np.ix_(rows, cols)]
    check_f32_result(ys, xf[rows], wf[cols], accum, s_static, what)
    amax = float(np.max(np.abs(ys)))
    # the last two scales lie outside [2^-60, 2^60], where the kernels divide instead of
    # multiplying by the reciprocal with corrections
    for s_out in (np.float32(amax) / np.float32(448.0), np.float32(amax) / np.float32(2000.0), np.float32(1e-3),
                  np.float32(amax) * np.float32(8.0), np.float32(2.0 ** -70), np.float32(2.0 ** 70)):
        s_out = np.float32(s_out if s_out > 0 else 1.0)
        st = dev(np.array([s_out], np.float32))
        q = sg.fp8_scaled_gemm_fp8out(xt, sa, wq, sw, st, **kw)
        torch.cuda.synchronize()
        assert q.dtype == torch.uint8 and tuple(q.shape) == (M, N)
        want = w8a8.quant_static(ys, s_out)
        assert_codes_equal(host(q)[np.ix_(rows, cols)], want, f"{what} s_out={s_out!r}")


ACCUMS = ["exact", "mfma_fp8"]
LAYOUTS = ["row_major", "packed"]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("accum", ACCUMS)
def test_tiny_and_ragged(accum, layout):
    x, w = tiny_w8a8(0)
    shapes = [(x, w)]
    rng = np.random.default_rng(9)
    for m, n, k in ((300, 1000, 1024), (129, 1001, 256), (17, 515, 128), (5, 1, 384), (3, 77, 4096), (33, 130, 512)):
        xx = rng.standard_normal((m, k)).astype(np.float32)
        xx[:, rng.integers(0, k, 3)] *= 40
        shapes.append((bf16_bits_from_f32(xx), (rng.standard_normal((n, k)) * 0.02).astype(np.float32)))
    for xb, wf in shapes:
        xt = dev_bf16(xb) if xb.dtype == np.uint16 else dev(xb)
        xf = f32_from_bf16_bits(xb) if xb.dtype == np.uint16 else xb
        wq, sw = sg.fp8_quant_weight_per_channel(dev(wf))
        wg = sg.fp8_pack_weights(wq) if layout == "packed" else wq
        run(xt, wg, sw, accum=accum, layout=layout, what=f"{tuple(xt.shape)}x{wf.shape[0]} {accum} {layout}",
            xf=xf, wf=wf)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("m", [1, 8, 32])
def test_decode(m, accum):
    xb, w, _ = decode_inputs(m)
    wq, sw = sg.fp8_quant_weight_per_channel(dev(w))
    run(dev_bf16(xb), sg.fp8_pack_weights(wq), sw, accum=accum, layout="packed", what=f"decode M={m} {accum}",
        xf=f32_from_bf16_bits(xb), wf=w)


@pytest.mark.parametrize("accum", ACCUMS)
def test_prefill_static_activation_scale(accum):
    """A per-tensor static activation scale in, a per-tensor static output scale out."""
    xb, w, _ = prefill_inputs(4096, m=1024, n=2048)
    wq, sw = sg.fp8_quant_weight_per_channel(dev(w))
    s_static = np.float32(120.0) / np.float32(448.0)
    sa = dev(np.array([s_static], np.float32))
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, 1023], rng.choice(1024, 64, replace=False)]))
    run(dev_bf16(xb), sg.fp8_pack_weights(wq), sw, accum=accum, layout="packed", mode="per_tensor", sa=sa,
        rows=rows, what=f"prefill static {accum}", xf=f32_from_bf16_bits(xb), wf=w, s_static=s_static)


def test_errors():
    x = torch.zeros((40, 128), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    sw = torch.ones(8, dtype=torch.float32, device="cuda")
    lib = sg.lib()
    y = torch.empty((40, 8), dtype=torch.uint8, device="cuda")
    ws = torch.empty(sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", 40, 8, 128), dtype=torch.uint8,
                     device="cuda")
    st = lib.fp8_scaled_gemm_fp8out(x.data_ptr(), sg.BF16, None, sg.SCALE_PER_TOKEN, wq.data_ptr(), 0,
                                    sw.data_ptr(), None, y.data_ptr(), 40, 8, 128, sg.ACCUM_EXACT, ws.data_ptr(),
                                    ws.numel(), None)
    assert st == sg.fp8sg.E_NULL
