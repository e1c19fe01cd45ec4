"""fp8_scaled_gemm_noalloc, through the C ABI, against fp8_scaled_gemm with a
caller workspace.  Both run the same kernels on the same inputs, the first with
the library's static device scratch in place of the workspace, so the outputs
and the computed activation scales must be bit-identical.  Each case makes two
no-alloc calls in a row, the second smaller than the first (the scratch keeps
the first call's contents), and checks both."""

import numpy as np
import pytest
import torch

from gpu_util import dev_bf16, host, host_bits16, require_gpu
from workloads import decode_inputs

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _inputs(m, n, k, seed, fp32):
    rng = np.random.default_rng([seed, m, n, k])
    x = rng.standard_normal((m, k), dtype=np.float32)
    x[:, rng.choice(k, 2, replace=False)] *= 40.0
    w = (rng.standard_normal((n, k), dtype=np.float32) * 0.02).astype(np.float32)
    xt = torch.from_numpy(x).cuda() if fp32 else torch.from_numpy(x).to(torch.bfloat16).cuda()
    wq, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w).cuda())
    return xt, wq, sw


def _pair(xt, wq, sw, mode, accum, out_dtype, w_layout):
    """(noalloc result, workspace result) for one call's arguments."""
    m = xt.shape[0]
    n = sw.shape[0]
    w_in = sg.fp8_pack_weights(wq) if w_layout == "packed" else wq
    if mode == "per_token":
        sa_n = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda")
        sa_w = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda")
    else:
        sa_n = torch.tensor([0.07], dtype=torch.float32, device="cuda")
        sa_w = sa_n.clone()
    y_n = torch.full((m, n), float("nan"), dtype=out_dtype, device="cuda")
    y_w = torch.full((m, n), float("nan"), dtype=out_dtype, device="cuda")
    sg.fp8_scaled_gemm_noalloc(xt, sa_n, w_in, sw, y=y_n, a_scale_mode=mode, accum=accum, w_layout=w_layout,
                               out_dtype=out_dtype)
    torch.cuda.synchronize()
    got = (y_n.clone(), sa_n.clone())
    sg.fp8_scaled_gemm(xt, sa_w, w_in, sw, y=y_w, a_scale_mode=mode, accum=accum, w_layout=w_layout,
                       out_dtype=out_dtype)
    torch.cuda.synchronize()
    return got, (y_w, sa_w)


def _same(got, want, what):
    (y_n, sa_n), (y_w, sa_w) = got, want
    if y_n.dtype == torch.bfloat16:
        a, b = host_bits16(y_n), host_bits16(y_w)
    else:
        a, b = host(y_n).view(np.uint32), host(y_w).view(np.uint32)
    assert not np.isnan(host(y_n.float())).any(), f"{what}: an output was not written"
    assert np.array_equal(a, b), f"{what}: {int((a != b).sum())} outputs differ from fp8_scaled_gemm's"
    assert np.array_equal(host(sa_n).view(np.uint32), host(sa_w).view(np.uint32)), f"{what}: scales differ"


# (x dtype fp32?, scale mode, accumulation, output dtype, W layout, first (M, N, K), second (M, N, K))
CASES = [
    (False, "per_token", "exact", torch.bfloat16, "packed", (300, 520, 1024), (20, 200, 512)),
    (False, "per_token", "mfma_fp8", torch.float32, "row_major", (64, 256, 2048), (9, 130, 256)),
    (True, "per_token", "exact", torch.float32, "packed", (40, 384, 640), (5, 64, 128)),
    (False, "per_tensor", "exact", torch.bfloat16, "row_major", (257, 300, 768), (33, 48, 384)),
    (True, "per_tensor", "mfma_fp8", torch.bfloat16, "packed", (24, 1000, 1152), (3, 17, 128)),
]


@pytest.mark.parametrize("fp32,mode,accum,out_dtype,w_layout,first,second", CASES)
def test_noalloc_matches_workspace_call(fp32, mode, accum, out_dtype, w_layout, first, second):
    for i, (m, n, k) in enumerate((first, second)):
        print(f"noalloc case {mode} {accum} {w_layout} fp32={fp32} call {i}: M={m} N={n} K={k}", flush=True)
        xt, wq, sw = _inputs(m, n, k, i, fp32)
        got, want = _pair(xt, wq, sw, mode, accum, out_dtype, w_layout)
        _same(got, want, f"{mode}/{accum}/{w_layout} call {i} ({m}x{n}x{k})")


def test_noalloc_decode_full_size():
    # the decode workload's bf16 rows [M, 4096] against W [14336, 4096]: M = 32 and 8
    # quantize into the scratch, M = 1 inside the GEMM kernel (no scratch)
    _, w, _ = decode_inputs(1, with_weight=True)
    wq, sw = sg.fp8_quant_weight_per_channel(torch.from_numpy(w).cuda())
    wp = sg.fp8_pack_weights(wq)
    for m in (32, 8, 1):
        print(f"noalloc decode M={m}", flush=True)
        xb, _, _ = decode_inputs(m, with_weight=False)
        got, want = _decode_pair(dev_bf16(xb), wp, sw)
        _same(got, want, f"decode M={m}")


def _decode_pair(xt, wp, sw):
    m, n = xt.shape[0], sw.shape[0]
    sa_n = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda")
    sa_w = sa_n.clone()
    y_n = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    y_w = y_n.clone()
    sg.fp8_scaled_gemm_noalloc(xt, sa_n, wp, sw, y=y_n, w_layout="packed")
    torch.cuda.synchronize()
    sg.fp8_scaled_gemm(xt, sa_w, wp, sw, y=y_w, w_layout="packed")
    torch.cuda.synchronize()
    return (y_n, sa_n), (y_w, sa_w)


def test_noalloc_refuses_calls_beyond_the_scratch():
    # bf16 per-token X [4097, 4096]: 16 MiB + 4096 bytes of codes plus the scales
    m, n, k = 4097, 128, 4096
    need = sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", m, n, k)
    assert need > sg.fp8sg.SCRATCH_BYTES
    xt = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    sw = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sg.Fp8sgError) as e:
        sg.fp8_scaled_gemm_noalloc(xt, None, wq, sw, y=y)
    assert e.value.status == sg.fp8sg.E_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all(), "a refused call wrote its output"
    # the codes in the fragment order (rows padded to 16) and the scales: 4080 rows fit, 4081 do not
    assert sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", 4080, n, k) <= sg.fp8sg.SCRATCH_BYTES
    assert sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", 4081, n, k) > sg.fp8sg.SCRATCH_BYTES
