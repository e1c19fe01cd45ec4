"""GPU parity of the block-wise scaled FP8 path (1 x 128 activation groups,
128 x 128 weight blocks) against the CPU oracle (oracle/blockwise.py), through
the C ABI.

Quantizers: codes and scales bit-exact.

GEMM, y = sum_g s_a[m, g] s_w[n // 128, g] P_g (read through the fp32 output):
  * exact mode (bf16 matrix cores, every M): |y - y_exact| <= 1e-5 * T, with
    T = sum_g |s_a s_w| sum_{k in g} |a_k w_k| -- the accumulator tolerance of
    the per-token GEMM applied to the block-scaled terms;
  * FP8 matrix-core mode: the bound derived from that hardware's summation
    (inside each 8-product group, truncation below 2^(e_max - 13), so a group
    loses less than 7 * 2^(e_max - 13)), scaled per block, plus one float32
    rounding per block partial, scale product and accumulation:
    |y - y_exact| <= sum_g |s_a s_w| sum_{groups in g} 7 * 2^(e_max - 13) + (G + 3) * 2^-24 * T.
The bf16 output must equal bf16_rne(fp32 output) bit for bit (same kernel,
same accumulator), and in exact mode lie within one bf16 ulp of the correctly
rounded exact value (outside that only where the tolerance itself exceeds an
ulp).
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_codes_equal, dev, dev_bf16, host, host_bits16, require_gpu
from oracle import blockwise as bw
from oracle import fp8
from workloads import bf16_bits_from_f32, decode_inputs, f32_from_bf16_bits, prefill_inputs, tiny_w8a8

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def bf16_ulp(y):
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e, -126) - 7)


def pack_reference(q):
    from test_abi_host import pack_reference as pr
    return pr(q)


def fp8_group_loss(a_rows, w_cols):
    """[r, c] sum over the 8-product groups of 7 * 2^(e_max - 13), per 128-deep block: [G, r, c]."""
    a = fp8.decode(a_rows)
    w = fp8.decode(w_cols)
    K = a.shape[1]
    G = K // 128
    out = np.zeros((G, a.shape[0], w.shape[0]))
    for i in range(a.shape[0]):
        p = np.abs(a[i][None, :] * w)                       # [c, K] exact products
        g = p.reshape(w.shape[0], K // 8, 8).max(axis=-1)    # [c, K / 8]
        e = np.floor(np.log2(np.where(g > 0, g, 1.0)))
        loss = np.where(g > 0, 7.0 * np.exp2(e - 13), 0.0)  # [c, K / 8]
        out[:, i, :] = loss.reshape(w.shape[0], G, 16).sum(axis=-1).T
    return out


def check_gemm(y_f32, y_bits, aq, sa, wq, sw, cols, accum, what):
    """aq/sa: the sampled rows; wq: all rows of W (for the block scales); cols: sampled columns."""
    sw_cols = sw                      # [NB, G]; indexed by column block below
    wq_c = wq[cols]
    # the oracle on the sampled columns: column n uses block n // 128 of s_w
    sw_rows = np.repeat(sw_cols, 128, axis=0)[cols]          # [c, G] scale of each sampled column
    P = bw.blockwise_partials(aq, wq_c)                       # [G, r, c] exact
    scale = sa.astype(np.float64).T[:, :, None] * sw_rows.astype(np.float64).T[:, None, :]  # [G, r, c]
    y_exact = (scale * P).sum(axis=0)
    a = np.abs(fp8.decode(aq))
    w = np.abs(fp8.decode(wq_c))
    G = aq.shape[1] // 128
    T = sum(np.abs(scale[g]) * (a[:, 128 * g:128 * g + 128] @ w[:, 128 * g:128 * g + 128].T) for g in range(G))
    err = np.abs(y_f32.astype(np.float64) - y_exact)
    if accum == "exact":
        bound = 1e-5 * T
    else:
        bound = (np.abs(scale) * fp8_group_loss(aq, wq_c)).sum(axis=0) + (G + 3) * 2.0 ** -24 * T
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs outside the bound; "
                           f"worst err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}")
    same = fp8.bf16_round_bits(y_f32.astype(np.float64)) == y_bits
    assert same.all(), f"{what}: {int((~same).sum())} bf16 outputs differ from the rounded fp32 output"
    if accum != "exact":
        return
    ref = fp8.bf16_bits_to_f64(fp8.bf16_round_bits(y_exact))
    d = np.abs(fp8.bf16_bits_to_f64(y_bits) - ref)
    ulp = bf16_ulp(ref)
    cancel = ulp < 1e-5 * T
    over = (d > ulp) & ~cancel
    assert not over.any(), f"{what}: {int(over.sum())} bf16 outputs beyond 1 ulp"
    assert (d[cancel] <= ulp[cancel] + 1e-5 * T[cancel]).all()


def run_case(x, w, *, accum, rows=None, cols=None, w_layout="row_major", a_layout="row_major", what="",
             kmajor=False):
    """Quantize X (1 x 128 groups) and W (128 x 128 blocks) on the GPU, check
    codes and scales against the oracle, run the GEMM, check its outputs.
    kmajor: the activation scales travel k-block-major ([K/128, M])."""
    is_bf16 = x.dtype == np.uint16
    xt = dev_bf16(x) if is_bf16 else dev(x)
    xf = f32_from_bf16_bits(x) if is_bf16 else x
    M, K = xf.shape
    N = w.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)

    sl = "kmajor" if kmajor else "row_major"
    aq_t, sa_t = sg.fp8_quant_per_token_group(xt, scale_layout=sl)
    wq_t, sw_t = sg.fp8_quant_weight_blockwise(dev(w))
    aq_ref, sa_ref = bw.quant_act_blockwise(xf[rows])
    sw_ref = bw.weight_block_scales(w)
    sa_host = host(sa_t).T if kmajor else host(sa_t)
    aq_got, sa_got, sw_got = host(aq_t)[rows], sa_host[rows], host(sw_t)
    assert np.array_equal(sa_got.view(np.uint32), sa_ref.view(np.uint32)), f"{what}: activation group scales"
    assert_codes_equal(aq_got, aq_ref, f"{what}: activation codes")
    assert np.array_equal(sw_got.view(np.uint32), sw_ref.view(np.uint32)), f"{what}: weight block scales"
    wq_all = host(wq_t)
    per_elem = np.repeat(np.repeat(sw_ref, 128, axis=0)[:N], 128, axis=1)[cols]
    from oracle.w8a8 import f32_div
    assert_codes_equal(wq_all[cols], fp8.encode(f32_div(w[cols], per_elem)), f"{what}: weight codes")

    a_in = aq_t if a_layout == "row_major" else sg.fp8_pack_weights(aq_t)
    w_in = wq_t if w_layout == "row_major" else sg.fp8_pack_weights(wq_t)
    kw = dict(accum=accum, w_layout=w_layout, a_layout=a_layout, a_shape=(M, K), w_shape=(N, K), a_scale_layout=sl)
    # outputs start as NaN: an output the kernels do not write stays NaN and fails below
    y32 = sg.fp8_scaled_gemm_blockwise(a_in, sa_t, w_in, sw_t, out_dtype=torch.float32,
                                       y=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"), **kw)
    y16 = sg.fp8_scaled_gemm_blockwise(a_in, sa_t, w_in, sw_t,
                                       y=torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda"), **kw)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(y32).any()) and not bool(torch.isnan(y16.float()).any()), f"{what}: unwritten outputs"
    check_gemm(host(y32)[np.ix_(rows, cols)], host_bits16(y16)[np.ix_(rows, cols)], aq_ref, sa_ref, wq_all, sw_ref,
               cols, accum, what)


def _sample(M, N, seed, nr=24, nc=256, tile=256, tile_n=128):
    """First and last rows / columns, one at random inside every 256-row and
    128-column tile (every output tile of both large-tile kernels: 256 x 256 in
    FP8 mode, 256 x 128 in exact mode), and more at random."""
    rng = np.random.default_rng(seed)
    per_r = [rng.integers(t, min(t + tile, M)) for t in range(0, M, tile)]
    per_c = [rng.integers(t, min(t + tile_n, N)) for t in range(0, N, tile_n)]
    rows = np.unique(np.concatenate([[0, M - 1], per_r, rng.choice(M, min(nr, M), replace=False)]).astype(np.int64))
    cols = np.unique(np.concatenate([[0, N - 1], per_c, rng.choice(N, min(nc, N), replace=False)]).astype(np.int64))
    return rows, cols


@pytest.mark.parametrize("layout", ["row_major", "packed"])
@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_tiny(accum, layout):
    x, w = tiny_w8a8(0)
    run_case(x, w, accum=accum, w_layout=layout, a_layout=layout, what=f"tiny {accum} {layout}")


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
@pytest.mark.parametrize("m", [1, 8, 32])
def test_decode(m, accum):
    xb, w, _ = decode_inputs(m)
    _, cols = _sample(m, w.shape[0], m, nc=1024)
    run_case(xb, w, accum=accum, cols=cols, w_layout="packed", a_layout="packed", what=f"decode M={m} {accum}",
             kmajor=(m == 8))


@pytest.mark.parametrize("kmajor", [False, True], ids=["scales_row_major", "scales_kmajor"])
@pytest.mark.parametrize("layout", ["row_major", "packed"])
@pytest.mark.parametrize("m,n,k", [(300, 1000, 1024), (129, 1001, 256), (33, 4100, 512), (17, 515, 128),
                                   (1, 7, 128), (5, 1, 384), (256, 384, 2048), (520, 130, 384), (300, 257, 128),
                                   (65, 1000, 256)])
def test_ragged(m, n, k, layout, kmajor):
    rng = np.random.default_rng(m * 7 + n + k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.integers(0, k, 3)] *= 40
    if k >= 256:
        x[m // 2, 128:256] = 0.0                                     # an all-zero group (scale 1.0)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[: min(n, 128), :128] *= 30                                     # one block with larger weights
    for accum in ("mfma_fp8", "exact"):
        run_case(bf16_bits_from_f32(x), w, accum=accum, w_layout=layout, a_layout=layout, kmajor=kmajor,
                 what=f"ragged {m}x{n}x{k} {accum} {layout} kmajor={kmajor}")


@pytest.mark.parametrize("accum", ["mfma_fp8", "exact"])
@pytest.mark.parametrize("kmajor", [False, True], ids=["scales_row_major", "scales_kmajor"])
@pytest.mark.parametrize("k", [4096, 14336])
def test_prefill_sampled(k, kmajor, accum):
    xb, w, _ = prefill_inputs(k)
    rows, cols = _sample(xb.shape[0], w.shape[0], k)
    run_case(xb, w, accum=accum, rows=rows, cols=cols, w_layout="packed", a_layout="row_major",
             what=f"prefill K={k} kmajor={kmajor} {accum}", kmajor=kmajor)


def test_fp32_input_and_packed_codes():
    """fp32 activations; the packed quantizer output equals the packed row-major output."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((37, 512)) * np.float32(3.0)).astype(np.float32)
    x[3, :128] *= 1e-30                                          # a group far down in float32
    xt = dev(x)
    q_rm, s_rm = sg.fp8_quant_per_token_group(xt)
    q_pk = torch.zeros(sg.fp8_packed_weight_bytes(37, 512), dtype=torch.uint8, device="cuda")
    q_pk, s_pk = sg.fp8_quant_per_token_group(xt, layout="packed", q=q_pk)
    torch.cuda.synchronize()
    q_ref, s_ref = bw.quant_act_blockwise(x)
    assert np.array_equal(host(s_rm).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(s_pk).view(np.uint32), s_ref.view(np.uint32))
    assert_codes_equal(host(q_rm), q_ref, "fp32 group codes")
    assert np.array_equal(host(q_pk), pack_reference(q_ref))


def test_deterministic_repeats():
    xb, w, _ = prefill_inputs(1024, m=600, n=700)
    aq, sa = sg.fp8_quant_per_token_group(dev_bf16(xb))
    wq, sw = sg.fp8_quant_weight_blockwise(dev(w))
    outs = [host_bits16(sg.fp8_scaled_gemm_blockwise(aq, sa, wq, sw)) for _ in range(8)]
    small = [host_bits16(sg.fp8_scaled_gemm_blockwise(aq[:24], sa[:24], wq, sw, accum=a)) for a in ("exact",) * 4]
    exact = [host_bits16(sg.fp8_scaled_gemm_blockwise(aq, sa, wq, sw, accum="exact")) for _ in range(4)]
    assert all(np.array_equal(o, outs[0]) for o in outs)
    assert all(np.array_equal(o, small[0]) for o in small)
    assert all(np.array_equal(o, exact[0]) for o in exact)


@pytest.mark.parametrize("m,n,k", [(600, 700, 1024), (257, 129, 384), (33, 4100, 256)])
def test_exact_layouts_agree_bit_for_bit(m, n, k):
    """Exact mode sums each block's products in one fixed k order whatever the
    operand layouts: row-major or packed A and W, row-major or k-block-major
    activation scales give the same bits, and so do repeated calls."""
    rng = np.random.default_rng(m + n + k)
    x = bf16_bits_from_f32(rng.standard_normal((m, k)).astype(np.float32) * 3)
    w = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    aq, sa = sg.fp8_quant_per_token_group(dev_bf16(x))
    sa_km = sa.t().contiguous()
    wq, sw = sg.fp8_quant_weight_blockwise(dev(w))
    ap, wp = sg.fp8_pack_weights(aq), sg.fp8_pack_weights(wq)
    outs = []
    for a_in, al in ((aq, "row_major"), (ap, "packed")):
        for w_in, wl in ((wq, "row_major"), (wp, "packed")):
            for s_in, sl in ((sa, "row_major"), (sa_km, "kmajor")):
                for dt in (torch.float32, torch.bfloat16):
                    y = sg.fp8_scaled_gemm_blockwise(a_in, s_in, w_in, sw, accum="exact", out_dtype=dt, a_layout=al,
                                                     w_layout=wl, a_shape=(m, k), w_shape=(n, k), a_scale_layout=sl)
                    outs.append((dt, host(y.view(torch.int32) if dt == torch.float32 else y.view(torch.int16))))
    again = host(sg.fp8_scaled_gemm_blockwise(aq, sa, wq, sw, accum="exact", out_dtype=torch.float32)
                 .view(torch.int32))
    torch.cuda.synchronize()
    f32 = [o for dt, o in outs if dt == torch.float32]
    b16 = [o for dt, o in outs if dt == torch.bfloat16]
    assert all(np.array_equal(o, f32[0]) for o in f32) and np.array_equal(again, f32[0])
    assert all(np.array_equal(o, b16[0]) for o in b16)


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_empty_k_writes_zeros(accum):
    """K = 0: every output is the empty sum, 0, at a large-tile M."""
    aq = torch.zeros((300, 0), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((300, 0), dtype=torch.float32, device="cuda")
    wq = torch.zeros((200, 0), dtype=torch.uint8, device="cuda")
    sw = torch.zeros((2, 0), dtype=torch.float32, device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        y = torch.full((300, 200), float("nan"), dtype=dt, device="cuda")
        sg.fp8_scaled_gemm_blockwise(aq, sa, wq, sw, accum=accum, out_dtype=dt, y=y)
        torch.cuda.synchronize()
        assert bool((y == 0).all()), f"K = 0 {accum} {dt}"
