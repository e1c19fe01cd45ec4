"""A decode step captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: every call of the step -- the W8A8 GEMM on bf16 activations with the
per-token quantization inside the call (M = 1: inside the GEMM kernel; M = 8,
32: a quantization kernel into the workspace first), the MX decode call, the
FP8 KV append and the decode attention over the FP8 cache -- launches only
kernels on the caller's stream, with no allocation, host synchronisation or
memset inside a call, so the step can be captured.  Each replay runs on new
inputs written into the captured buffers, with eager work between replays, and
must give exactly the bits of the same calls run eagerly (every kernel is
deterministic)."""

import numpy as np
import pytest
import torch

from gpu_util import dev, require_gpu
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(bf16_bits_from_f32(x).view(np.int16)).view(torch.bfloat16).cuda()


def test_decode_step_replays_bit_exact():
    rng = np.random.default_rng(5)
    N, K = 2048, 1024
    w = dev((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, sw = sg.fp8_quant_weight_per_channel(w)
    wp = sg.fp8_pack_weights(wq)
    wmx, wsmx = sg.fp8_quant_mx(w, "e4m3", layout="packed", scale_layout="packed")
    B, S_cap, H, Hq, D = 2, 512, 2, 8, 128
    k_cache = torch.zeros((B, S_cap, H, D), dtype=torch.uint8, device="cuda")
    v_cache = torch.zeros_like(k_cache)
    k_fill, v_fill = _bf16(rng, (B, S_cap, H, D)), _bf16(rng, (B, S_cap, H, D))
    ks, vs = sg.fp8_kv_calibrate(k_fill), sg.fp8_kv_calibrate(v_fill)
    sg.fp8_kv_quant(k_fill, ks, out=k_cache)
    sg.fp8_kv_quant(v_fill, vs, out=v_cache)
    pos = torch.full((B,), 300, dtype=torch.int32, device="cuda")
    lengths = pos + 1

    Ms = (1, 8, 32)
    xs = {m: torch.empty((m, K), dtype=torch.bfloat16, device="cuda") for m in Ms}
    ws = {m: torch.empty((max(1, sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", m, N, K)),),
                         dtype=torch.uint8, device="cuda") for m in Ms}
    x_mx = torch.empty((8, K), dtype=torch.bfloat16, device="cuda")
    k_new = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    attn_ws = torch.empty((sg.fp8_kv_decode_attention_workspace_size(B, S_cap, Hq, H, D),), dtype=torch.uint8,
                          device="cuda")

    def fill(seed):
        r = np.random.default_rng(seed)
        for m in Ms:
            xs[m].copy_(_bf16(r, (m, K)))
        x_mx.copy_(_bf16(r, (8, K), 3.0))
        k_new.copy_(_bf16(r, (B, H, D)))
        v_new.copy_(_bf16(r, (B, H, D)))
        q.copy_(_bf16(r, (B, Hq, D)))

    def step(outs, kc, vc):
        for m in Ms:
            sg.fp8_scaled_gemm(xs[m], None, wp, sw, y=outs[f"y{m}"], workspace=ws[m], w_layout="packed")
        sg.fp8_scaled_gemm_mx_bf16(x_mx, wmx, wsmx, y=outs["ymx"], w_layout="packed", w_shape=(N, K))
        sg.fp8_kv_append(k_new, pos, ks, kc)
        sg.fp8_kv_append(v_new, pos, vs, vc)
        sg.fp8_kv_decode_attention(q, kc, vc, ks, vs, lengths, out=outs["attn"], workspace=attn_ws)

    def new_outs():
        o = {f"y{m}": torch.empty((m, N), dtype=torch.bfloat16, device="cuda") for m in Ms}
        o["ymx"] = torch.empty((8, N), dtype=torch.bfloat16, device="cuda")
        o["attn"] = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        return o

    # warm up on a side stream (library state is set up before capture), then capture
    g_outs = new_outs()
    fill(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(g_outs, k_cache, v_cache)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(g_outs, k_cache, v_cache)

    for rep in range(4):
        fill(100 + rep)
        g.replay()
        torch.cuda.synchronize()
        # the same calls eagerly, into fresh outputs and a copy of the caches as they were before the replay's
        # append (the appends write the same position each time, so re-appending to the replayed caches is
        # the identical state)
        e_outs = new_outs()
        kc, vc = k_cache.clone(), v_cache.clone()
        step(e_outs, kc, vc)
        torch.cuda.synchronize()
        for name in e_outs:
            assert torch.equal(g_outs[name].view(torch.int16), e_outs[name].view(torch.int16)), (rep, name)
        assert torch.equal(kc, k_cache) and torch.equal(vc, v_cache), rep


def test_prefill_calls_replay_bit_exact():
    """Prefill-sized calls captured and replayed: fp8_scaled_gemm on bf16
    activations with the per-token quantization inside the call (the 16-row-tile
    quantizer into the fragment order, then the large-tile exact GEMM) and with a
    given per-tensor scale, and the block-wise GEMM with exact partials on
    pre-quantized codes; every replay on new inputs equals the eager calls bit
    for bit."""
    rng = np.random.default_rng(6)
    M, N, K = 300, 1000, 1024
    w = dev((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, sw = sg.fp8_quant_weight_per_channel(w)
    wp = sg.fp8_pack_weights(wq)
    wbq, wbs = sg.fp8_quant_weight_blockwise(w)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    st = torch.tensor([0.011], dtype=torch.float32, device="cuda")
    ws_pt = torch.empty((sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", M, N, K),), dtype=torch.uint8,
                        device="cuda")
    ws_st = torch.empty((sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_tensor", M, N, K),),
                        dtype=torch.uint8, device="cuda")
    aq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")

    def step(o):
        sg.fp8_scaled_gemm(x, None, wp, sw, y=o["pt"], workspace=ws_pt, w_layout="packed")
        sg.fp8_scaled_gemm(x, st, wp, sw, y=o["st"], workspace=ws_st, a_scale_mode="per_tensor", w_layout="packed")
        sg.fp8_quant_per_token_group(x, q=aq, scales=sa)
        sg.fp8_scaled_gemm_blockwise(aq, sa, wbq, wbs, y=o["bw"], accum="exact")

    def new_outs():
        return {k: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for k in ("pt", "st", "bw")}

    g_outs = new_outs()
    x.copy_(_bf16(rng, (M, K)))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(g_outs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(g_outs)
    for rep in range(4):
        x.copy_(_bf16(np.random.default_rng(200 + rep), (M, K), 2.0))
        g.replay()
        torch.cuda.synchronize()
        e_outs = new_outs()
        step(e_outs)
        torch.cuda.synchronize()
        for name in e_outs:
            assert torch.equal(g_outs[name].view(torch.int16), e_outs[name].view(torch.int16)), (rep, name)
