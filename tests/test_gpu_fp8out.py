"""GPU parity of the GEMM's FP8 output epilogue (fp8_scaled_gemm_fp8out).

The codes are a quantization decision taken on the kernel's fp32 result, so
the check takes that decision in the same precision: for every output,
code == E4M3(RN32(y32 / s_out)) bit for bit (the oracle's static quantizer,
oracle/w8a8.py), where y32 is what fp8_scaled_gemm writes with fp32 output for
the same arguments (same kernel, same accumulator).  That fp32 result itself
is checked against the exact product in tests/test_gpu_gemm.py.  Output
scales cover a calibrated scale, saturation of most outputs, and underflow of
most outputs to subnormal codes and zero.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_codes_equal, dev, dev_bf16, host, require_gpu
from oracle import w8a8
from workloads import bf16_bits_from_f32, decode_inputs, prefill_inputs, tiny_w8a8

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def run(xt, wq, sw, *, accum, layout, mode="per_token", sa=None, rows=None, cols=None, what=""):
    M = xt.shape[0]
    N = sw.shape[0]
    kw = dict(accum=accum, w_layout=layout, a_scale_mode=mode)
    y32 = sg.fp8_scaled_gemm(xt, sa, wq, sw, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    y = host(y32)
    rows = np.arange(M) if rows is None else rows
    cols = np.arange(N) if cols is None else cols
    ys = y[np.ix_(rows, cols)]
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
        wq, sw = sg.fp8_quant_weight_per_channel(dev(wf))
        wg = sg.fp8_pack_weights(wq) if layout == "packed" else wq
        run(xt, wg, sw, accum=accum, layout=layout, what=f"{tuple(xt.shape)}x{wf.shape[0]} {accum} {layout}")


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("m", [1, 8, 32])
def test_decode(m, accum):
    xb, w, _ = decode_inputs(m)
    wq, sw = sg.fp8_quant_weight_per_channel(dev(w))
    run(dev_bf16(xb), sg.fp8_pack_weights(wq), sw, accum=accum, layout="packed", what=f"decode M={m} {accum}")


@pytest.mark.parametrize("accum", ACCUMS)
def test_prefill_static_activation_scale(accum):
    """A per-tensor static activation scale in, a per-tensor static output scale out."""
    xb, w, _ = prefill_inputs(4096, m=1024, n=2048)
    wq, sw = sg.fp8_quant_weight_per_channel(dev(w))
    sa = dev(np.array([np.float32(120.0) / np.float32(448.0)], np.float32))
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, 1023], rng.choice(1024, 64, replace=False)]))
    run(dev_bf16(xb), sg.fp8_pack_weights(wq), sw, accum=accum, layout="packed", mode="per_tensor", sa=sa,
        rows=rows, what=f"prefill static {accum}")


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
