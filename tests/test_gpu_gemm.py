"""GPU parity of fp8_scaled_gemm against the CPU oracle, through the C ABI.

Tolerances:
  * exact accumulation mode: |acc - acc_exact| <= 1e-5 * sum_k |a_k w_k| for
    every output (acc read through the fp32 output with unit scales), and the
    bf16 output within one bf16 ulp of the correctly rounded exact result;
  * FP8 matrix-core mode: the bound derived from that hardware's summation --
    within each group of 8 consecutive k the products are aligned to the group's
    largest and truncated below 2^(e_max - 13), so a group loses less than
    7 * 2^(e_max - 13); plus one float32 rounding per 128-deep instruction:
    |acc - acc_exact| <= sum_g 7 * 2^(e_max,g - 13) + (K / 128) * 2^-24 * sum|a w|.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_codes_equal, dev, dev_bf16, host, host_bits16, require_gpu
from oracle import fp8, w8a8
from oracle.fp8 import E4M3
from workloads import (STATIC_SCALE_DEN, STATIC_SCALE_NUM, decode_inputs, f32_from_bf16_bits, large_layer_inputs,
                       prefill_inputs, tiny_w8a8)

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def bf16_ulp(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e, -126) - 7)


def fp8_mfma_bound(aq_rows: np.ndarray, wq_rows: np.ndarray) -> np.ndarray:
    """Derived error bound of the FP8 matrix-core accumulation, per output."""
    a = fp8.decode(aq_rows)
    w = fp8.decode(wq_rows)
    K = a.shape[1]
    out = np.zeros((a.shape[0], w.shape[0]))
    for i in range(a.shape[0]):
        p = a[i][None, :] * w                       # [n, K] exact products
        g = np.abs(p).reshape(w.shape[0], K // 8, 8).max(axis=-1)
        e = np.floor(np.log2(np.where(g > 0, g, 1.0)))
        grp = np.where(g > 0, 7.0 * np.exp2(e - 13), 0.0).sum(axis=-1)
        out[i] = grp + (K / 128) * 2.0 ** -24 * np.abs(p).sum(axis=-1)
    return out


def check_outputs(y_bits, acc_gpu, aq_rows, sa_rows, wq_rows, sw_rows, accum, what, y_f32_fused=None):
    """y_bits: bf16 output [r, c]; acc_gpu: fp32 accumulator [r, c] (unit scales).

    y_f32_fused: when y_bits came from the decode kernel that quantizes the
    activations itself (its k order differs from the unit-scale call's), that
    kernel's fp32 output; its bf16 rounding must equal y_bits bit for bit, and
    it must lie within the accumulator bound (scaled) plus the epilogue's two
    float32 roundings of the exact result."""
    acc = w8a8.gemm_acc_exact(aq_rows, wq_rows)
    absum = w8a8.gemm_abs_sum(aq_rows, wq_rows)
    err = np.abs(acc_gpu.astype(np.float64) - acc)
    if accum == "exact":
        bound = 1e-5 * absum
    else:
        bound = fp8_mfma_bound(aq_rows, wq_rows)
    bad = err > bound
    assert not bad.any(), (f"{what}: accumulator outside tolerance at {int(bad.sum())} outputs; "
                           f"worst err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}")
    sa32 = np.asarray(sa_rows, np.float32).reshape(-1, 1)
    sw32 = np.asarray(sw_rows, np.float32).reshape(1, -1)
    if y_f32_fused is None:
        # the bf16 epilogue of the same accumulator: y = bf16_rne(RN32(RN32(acc * s_a) * s_w)), bit for bit
        # (the fp32 output with unit scales shares the bf16 kernel's main loop, so acc_gpu is its accumulator)
        y_epi = fp8.bf16_round_bits(((acc_gpu.astype(np.float32) * sa32) * sw32).astype(np.float64))
    else:
        y_epi = fp8.bf16_round_bits(y_f32_fused.astype(np.float64))
        s_abs = np.abs(sa32.astype(np.float64) * sw32.astype(np.float64))
        y_ex = w8a8.scaled_gemm_f64(acc, sa_rows, sw_rows)
        e_y = np.abs(y_f32_fused.astype(np.float64) - y_ex)
        b_y = bound * s_abs * (1 + 2.0 ** -22) + 2.0 ** -22 * np.abs(y_ex)
        assert (e_y <= b_y).all(), f"{what}: fused fp32 output outside the scaled bound at {int((e_y > b_y).sum())}"
    mism = y_epi != y_bits
    assert not mism.any(), f"{what}: {int(mism.sum())} bf16 outputs differ from the scaled accumulator"
    if accum != "exact":
        return
    y_ref_bits = fp8.bf16_round_bits(w8a8.scaled_gemm_f64(acc, sa_rows, sw_rows))
    y_ref = fp8.bf16_bits_to_f64(y_ref_bits)
    y = fp8.bf16_bits_to_f64(y_bits)
    d = np.abs(y - y_ref)
    ulp = bf16_ulp(y_ref)
    s_prod = np.abs(np.asarray(sa_rows, np.float64).reshape(-1, 1) * np.asarray(sw_rows, np.float64).reshape(1, -1))
    # an output may leave the 1-ulp band only where its exact value is so much
    # smaller than sum|a w| that the accumulator tolerance alone exceeds an ulp
    cancel = ulp < 1e-5 * absum * s_prod
    over = (d > ulp) & ~cancel
    assert not over.any(), (f"{what}: {int(over.sum())} bf16 outputs beyond 1 ulp; "
                            f"worst {np.max(d / ulp):.3g} ulp")
    assert (d[cancel] <= ulp[cancel] + 1e-5 * (absum * s_prod)[cancel]).all()


def gemm_case(x, w, *, rows=None, cols=None, accum="exact", static=None, what="", layout="row_major"):
    """Quantize W (per channel) and run the GEMM with the activation quantized
    inside the call; check W codes, activation scales and outputs on the sampled
    rows/cols against the oracle."""
    is_bf16 = x.dtype == np.uint16
    xt = dev_bf16(x) if is_bf16 else dev(x)
    xf = f32_from_bf16_bits(x) if is_bf16 else x
    M, K = xf.shape
    N = w.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)

    wq_t, sw_t = sg.fp8_quant_weight_per_channel(dev(w))
    wg = sg.fp8_pack_weights(wq_t) if layout == "packed" else wq_t
    wq_ref, sw_ref = w8a8.quant_weight_per_channel(w[cols])
    wq_got = host(wq_t)[cols]
    sw_got = host(sw_t)[cols]
    assert np.array_equal(sw_got.view(np.uint32), sw_ref.view(np.uint32)), f"{what}: weight scales"
    assert_codes_equal(wq_got, wq_ref, f"{what}: weight codes")

    # every output buffer starts as NaN: a tile the kernels skip (or a row or
    # column they drop) leaves NaN behind, which the full-size check below finds
    def nan_out(dtype):
        return torch.full((M, N), float("nan"), dtype=dtype, device="cuda")

    y32_fused = None
    if static is None:
        sa_t = torch.empty(M, dtype=torch.float32, device="cuda")
        y_t = sg.fp8_scaled_gemm(xt, sa_t, wg, sw_t, a_scale_mode="per_token", accum=accum, w_layout=layout,
                                 y=nan_out(torch.bfloat16))
        if is_bf16 and sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", M, N, K) == 0:
            # quantized inside the decode kernel: the same kernel's fp32 output checks its epilogue
            y32_fused = sg.fp8_scaled_gemm(xt, None, wg, sw_t, out_dtype=torch.float32, accum=accum,
                                           w_layout=layout, y=nan_out(torch.float32))
        aq_ref, sa_ref = w8a8.quant_per_token(xf[rows])
        assert np.array_equal(host(sa_t)[rows].view(np.uint32), sa_ref.view(np.uint32)), f"{what}: act scales"
        # the accumulator through the same kernel: pre-quantized codes, unit scales, fp32 out
        aq_t, _ = sg.fp8_quant_per_token(xt)
        assert_codes_equal(host(aq_t)[rows], aq_ref, f"{what}: act codes")
    else:
        s = np.float32(static)
        sa_t = dev(np.float32([s]))
        y_t = sg.fp8_scaled_gemm(xt, sa_t, wg, sw_t, a_scale_mode="per_tensor", accum=accum, w_layout=layout,
                                 y=nan_out(torch.bfloat16))
        aq_ref = w8a8.quant_static(xf[rows], s)
        sa_ref = np.full(len(rows), s, np.float32)
        aq_t = sg.fp8_quant_per_tensor_static(xt, sa_t)
        assert_codes_equal(host(aq_t)[rows], aq_ref, f"{what}: act codes")
    ones_m = torch.ones(M, dtype=torch.float32, device="cuda")
    ones_n = torch.ones(N, dtype=torch.float32, device="cuda")
    acc_t = sg.fp8_scaled_gemm(aq_t, ones_m, wg, ones_n, out_dtype=torch.float32, accum=accum, w_layout=layout,
                               y=nan_out(torch.float32))
    # the same codes in the fragment order (FP8SG_A_PACKED): the kernels give each
    # lane the same k, so the accumulators must agree bit for bit
    ap_t = sg.fp8_pack_weights(aq_t)
    acc_p = sg.fp8_scaled_gemm(ap_t, ones_m, wg, ones_n, out_dtype=torch.float32, accum=accum, w_layout=layout,
                               a_layout="packed", a_shape=(M, K), y=nan_out(torch.float32))
    torch.cuda.synchronize()
    # every output of every call was written (finite inputs give finite outputs)
    for name, t in (("bf16 output", y_t), ("fp32 accumulator", acc_t), ("packed-A accumulator", acc_p),
                    ("fused fp32 output", y32_fused)):
        if t is not None:
            assert not bool(torch.isnan(t.float()).any()), f"{what}: {name} has unwritten (NaN) outputs"
    y_bits = host_bits16(y_t)[np.ix_(rows, cols)]
    acc_gpu = host(acc_t)[np.ix_(rows, cols)]
    acc_pk = host(acc_p)[np.ix_(rows, cols)]
    assert np.array_equal(acc_pk.view(np.uint32), acc_gpu.view(np.uint32)), f"{what}: packed-A accumulator differs"
    del ap_t, acc_p
    y32f = None if y32_fused is None else host(y32_fused)[np.ix_(rows, cols)]
    check_outputs(y_bits, acc_gpu, aq_ref, sa_ref, wq_ref, sw_ref, accum, what, y_f32_fused=y32f)


ACCUMS = ["exact", "mfma_fp8"]
LAYOUTS = ["row_major", "packed"]


def test_pack_weights_is_the_documented_permutation():
    from test_abi_host import pack_reference
    rng = np.random.default_rng(1)
    for n, k in ((37, 384), (16, 128), (1, 256), (300, 1024)):
        wq = rng.integers(0, 256, (n, k), dtype=np.uint8)
        got = host(sg.fp8_pack_weights(dev(wq)))
        assert np.array_equal(got, pack_reference(wq)), (n, k)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("accum", ACCUMS)
def test_tiny_w8a8(accum, layout):
    x, w = tiny_w8a8(0)
    gemm_case(x, w, accum=accum, what=f"tiny {accum} {layout}", layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("m", [1, 8, 32])
def test_decode_full_size(m, accum, layout):
    xb, w, _ = decode_inputs(m)
    gemm_case(xb, w, accum=accum, what=f"decode M={m} {accum} {layout}", layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("m,n,k", [(300, 1000, 1024), (129, 1001, 256), (17, 515, 128), (33, 4100, 512),
                                   (256, 384, 2048), (1, 7, 128), (5, 1, 384)])
def test_ragged_tiles(m, n, k, accum, layout):
    rng = np.random.default_rng(m * 7 + n + k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.integers(0, k, 2)] *= 40
    from workloads import bf16_bits_from_f32
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    gemm_case(bf16_bits_from_f32(x), w, accum=accum, what=f"ragged {m}x{n}x{k} {accum} {layout}", layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("m,n,k", [(1, 7, 128), (5, 1000, 384), (16, 515, 4096), (17, 130, 1152), (32, 14336, 4096)])
def test_decode_static_scale_in_call(m, n, k, accum, layout):
    """A given per-tensor activation scale with M <= 32: the call quantizes X
    straight into the fragment order (rows padded to 16) before the decode
    GEMM, so the codes, the accumulator and the bf16 output all go through that
    quantizer; scales cover a calibrated one, heavy saturation and underflow."""
    from workloads import bf16_bits_from_f32
    rng = np.random.default_rng(m * 31 + n + k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.integers(0, k, 3)] *= 40
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    xb = bf16_bits_from_f32(x)
    amax = float(np.max(np.abs(f32_from_bf16_bits(xb))))
    for s in (np.float32(amax) / np.float32(448.0), np.float32(amax) / np.float32(4000.0), np.float32(amax)):
        gemm_case(xb, w, accum=accum, static=np.float32(s), layout=layout,
                  what=f"decode static {m}x{n}x{k} s={s!r} {accum} {layout}")


@pytest.mark.parametrize("m,k,dt", [(33, 128, "bf16"), (129, 8192, "bf16"), (300, 1024, "bf16"), (50, 4096, "f32"),
                                    (1000, 2944, "bf16"), (40, 8320, "bf16")])
def test_per_token_codes_in_the_call_workspace(m, k, dt):
    """The codes and scales a per-token call leaves in its workspace against the
    oracle's per-token quantizer, byte for byte on every live row: the fragment
    order (rows padded to 16) written by the 16-row-tile quantizer where its
    registers hold a tile's rows (bf16 K <= 8192, fp32 K <= 4096), row-major
    codes beyond that (K = 8320); the scales follow at the next 256 bytes."""
    rng = np.random.default_rng(m * 13 + k)
    x = (rng.standard_t(3, (m, k)) * 2).astype(np.float32)
    x[rng.integers(0, m, 3)] = 0.0                      # zero rows: unit scales
    x[:, rng.integers(0, k, 2)] *= 30
    _check_call_workspace(x, dt, f"{m}x{k} {dt}")


def test_per_token_edge_rows_in_the_call():
    """The edge rows of the standalone per-token quantizer's test (zero and
    signed-zero rows, rows whose scale leaves [2^-60, 2^60], huge rows, a
    maximum at the last element, subnormals) quantized inside fp8_scaled_gemm
    by the 16-row-tile quantizer (M > 32, K = 128), bf16 and fp32."""
    k = 128
    rng = np.random.default_rng(31)
    rows = [np.zeros(k, np.float32)]
    r = np.zeros(k, np.float32); r[::2] = -0.0; rows.append(r)
    for scale in (1e-30, 1e-38, 3e-39, 2.0 ** -120, 1e25, 3e38, 1.0, 448.0):
        rows.append((rng.standard_normal(k) * scale).astype(np.float32))
    r = rng.standard_normal(k).astype(np.float32); r[-1] = 1000.0; rows.append(r)
    rows.append(np.float32([2.0 ** -133 * i for i in range(k)]))
    rows.append(np.float32([-(2.0 ** -130) * i for i in range(k)]))
    rows += [(rng.standard_normal(k) * 1e-42).astype(np.float32) for _ in range(4)]   # fp32 subnormals
    x = np.stack(rows + [rng.standard_normal(k).astype(np.float32) for _ in range(40 - len(rows))])
    _check_call_workspace(x, "bf16", "edge rows bf16")
    _check_call_workspace(x, "f32", "edge rows fp32")


def _check_call_workspace(x, dt, what):
    """Run a per-token fp8_scaled_gemm on x (quantized inside the call) and compare
    the codes and scales its workspace holds with the oracle's, byte for byte."""
    from test_abi_host import pack_reference
    from workloads import bf16_bits_from_f32
    m, k = x.shape
    if dt == "bf16":
        xb = bf16_bits_from_f32(x)
        xt, xf = dev_bf16(xb), f32_from_bf16_bits(xb)
    else:
        xt, xf = dev(x), x
    n = 16
    rng = np.random.default_rng(k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    wq_t, sw_t = sg.fp8_quant_weight_per_channel(dev(w))
    nbytes = sg.fp8_scaled_gemm_workspace_size(xt.dtype, "per_token", m, n, k)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    sg.fp8_scaled_gemm(xt, None, wq_t, sw_t, workspace=ws)
    torch.cuda.synchronize()
    wsh = host(ws)
    want_q, want_s = w8a8.quant_per_token(xf)
    packed = k <= (8192 if dt == "bf16" else 4096)
    rows = (m + 15) // 16 * 16 if packed else m
    codes = wsh[:rows * k]
    if packed:
        live = pack_reference(np.ones((m, k), np.uint8)).astype(bool)
        assert_codes_equal(codes[live], pack_reference(want_q)[live], f"{what} packed codes")
    else:
        assert_codes_equal(codes.reshape(m, k), want_q, f"{what} row-major codes")
    off = (rows * k + 255) // 256 * 256
    got_s = wsh[off:off + 4 * m].view(np.float32)
    assert np.array_equal(got_s.view(np.uint32), np.asarray(want_s, np.float32).view(np.uint32)), f"{what} scales"


def _sample(M, N, seed, nr=40, nc=384, tile=256):
    """Rows and columns to compare at full size: the first and last, one at random
    inside every 256-row and every 256-column tile (so every output tile of the
    large-tile kernels, and every tile of its per-XCD order, is compared at
    least once), and nr / nc more at random."""
    rng = np.random.default_rng(seed)
    per_r = [rng.integers(t, min(t + tile, M)) for t in range(0, M, tile)]
    per_c = [rng.integers(t, min(t + tile, N)) for t in range(0, N, tile)]
    rows = np.unique(np.concatenate([[0, M - 1], per_r, rng.choice(M, nr, replace=False)]).astype(np.int64))
    cols = np.unique(np.concatenate([[0, N - 1], per_c, rng.choice(N, nc, replace=False)]).astype(np.int64))
    return rows, cols


def test_sample_covers_every_output_tile():
    for M, N in ((8192, 4096), (4096, 28672), (300, 1000)):
        rows, cols = _sample(M, N, 3)
        assert set(np.unique(rows // 256)) == set(range((M + 255) // 256))
        assert set(np.unique(cols // 256)) == set(range((N + 255) // 256))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("k", [4096, 14336])
def test_prefill_full_size_sampled(k, accum, layout):
    xb, w, _ = prefill_inputs(k)
    rows, cols = _sample(xb.shape[0], w.shape[0], k)
    gemm_case(xb, w, rows=rows, cols=cols, accum=accum, what=f"prefill K={k} {accum} {layout}", layout=layout)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("static,layout", [(True, "packed"), (False, "packed"), (False, "row_major")],
                         ids=["static-packed", "dynamic-packed", "dynamic-row_major"])
def test_large_layer_sampled(static, layout, accum):
    """The large layer in the calls the benchmark times (bf16 X quantized inside
    the call into the fragment order, packed W; per-token and static arms), and
    the per-token arm on row-major W."""
    xb, w = large_layer_inputs()
    rows, cols = _sample(xb.shape[0], w.shape[0], 4, nr=24, nc=256)
    s = np.float32(STATIC_SCALE_NUM) / np.float32(STATIC_SCALE_DEN) if static else None
    gemm_case(xb, w, rows=rows, cols=cols, accum=accum, static=s, layout=layout,
              what=f"large {'static' if static else 'dyn'} {layout}")


def test_prequantized_input_and_per_tensor_scale():
    x, w = tiny_w8a8(0)
    aq, sa = w8a8.quant_per_token(x)
    wq, sw = w8a8.quant_weight_per_channel(w)
    y = sg.fp8_scaled_gemm(dev(aq), dev(sa), dev(wq), dev(sw))
    s = np.float32([0.0371])
    y2 = sg.fp8_scaled_gemm(dev(aq), dev(s), dev(wq), dev(sw), a_scale_mode="per_tensor")
    torch.cuda.synchronize()
    acc = w8a8.gemm_acc_exact(aq, wq)
    for got, sc in ((y, sa), (y2, s)):
        ref = fp8.bf16_bits_to_f64(fp8.bf16_round_bits(w8a8.scaled_gemm_f64(acc, sc, sw)))
        d = np.abs(fp8.bf16_bits_to_f64(host_bits16(got)) - ref)
        assert (d <= bf16_ulp(ref)).all()


def test_deterministic_repeats():
    xb, w, _ = decode_inputs(32, n=2048)
    wq, sw = sg.fp8_quant_weight_per_channel(dev(w))
    xt = dev_bf16(xb)
    outs = [host_bits16(sg.fp8_scaled_gemm(xt, None, wq, sw)) for _ in range(20)]
    wp = sg.fp8_pack_weights(wq)
    outs += [host_bits16(sg.fp8_scaled_gemm(xt, None, wp, sw, w_layout="packed")) for _ in range(20)]
    xb2, w2, _ = prefill_inputs(1024, m=512, n=512)
    wq2, sw2 = sg.fp8_quant_weight_per_channel(dev(w2))
    xt2 = dev_bf16(xb2)
    outs2 = [host_bits16(sg.fp8_scaled_gemm(xt2, None, wq2, sw2, accum=a)) for a in ACCUMS for _ in range(10)]
    assert all(np.array_equal(o, outs[0]) for o in outs)
    assert all(np.array_equal(o, outs2[0]) for o in outs2[:10])
    assert all(np.array_equal(o, outs2[10]) for o in outs2[10:])


def test_fp8_matrix_core_group_alignment_is_what_exact_mode_avoids():
    """One output, K = 128: a = [256, 2^-9 x 127], w = 1.  Exact mode returns
    256 + 127 * 2^-9; the FP8 matrix cores drop the seven small products that
    share the first 8-product group with 256 (they sit more than 13 bits below
    it), giving 256 + 120 * 2^-9."""
    a = np.full((1, 128), 0x01, np.uint8)
    a[0, 0] = 0x78  # 256
    wq = np.full((1, 128), 0x38, np.uint8)  # 1.0
    one = dev(np.float32([1.0]))
    ex = sg.fp8_scaled_gemm(dev(a), one, dev(wq), one, out_dtype=torch.float32, accum="exact")
    f8 = sg.fp8_scaled_gemm(dev(a), one, dev(wq), one, out_dtype=torch.float32, accum="mfma_fp8")
    torch.cuda.synchronize()
    assert float(host(ex)[0, 0]) == 256 + 127 * 2.0 ** -9
    assert float(host(f8)[0, 0]) == 256 + 120 * 2.0 ** -9


def test_workspace_and_errors():
    # decode-sized (M <= 4) per-token activations are quantized inside the GEMM kernel: no workspace
    assert sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", 4, 8, 128) == 0
    assert sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_tensor", 4, 8, 128) >= 4 * 128
    x = torch.zeros((40, 128), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    sw = torch.ones(8, dtype=torch.float32, device="cuda")
    need = sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", 40, 8, 128)
    assert need >= 40 * 128
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(sg.Fp8sgError) as e:
        sg.fp8_scaled_gemm(x, None, wq, sw, workspace=small)
    assert e.value.status == sg.fp8sg.E_WORKSPACE
    y = sg.fp8_scaled_gemm(x, None, wq, sw)
    torch.cuda.synchronize()
    assert (host_bits16(y) == 0).all()

@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_fused_decode_quant(accum, layout):
    """For bf16 activations with M <= 4 and K <= 4096 the per-token quantization
    runs inside the GEMM kernel.  Its scales must equal fp8_quant_per_token's
    bit for bit; its output must not depend on whether the scales are returned;
    and its output must meet the oracle checks (the 1-ulp / accumulator bounds),
    also at K = 4224 (past the limit: the two-kernel path) and for fp32
    activations (always the two-kernel path)."""
    rng = np.random.default_rng(5)
    from workloads import bf16_bits_from_f32
    for m, n, k in ((1, 300, 4096), (3, 1000, 128), (4, 4100, 4096), (4, 77, 4224), (2, 33, 1152), (5, 64, 256)):
        x = rng.standard_normal((m, k)).astype(np.float32)
        x[:, rng.integers(0, k, 3)] *= 40
        xb = bf16_bits_from_f32(x)
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        what = f"fused {m}x{n}x{k} {accum} {layout}"
        gemm_case(xb, w, accum=accum, what=what, layout=layout)
        wq, sw = sg.fp8_quant_weight_per_channel(dev(w))
        wg = sg.fp8_pack_weights(wq) if layout == "packed" else wq
        xt = dev_bf16(xb)
        sa = torch.empty(m, dtype=torch.float32, device="cuda")
        y1 = sg.fp8_scaled_gemm(xt, sa, wg, sw, accum=accum, w_layout=layout)
        y0 = sg.fp8_scaled_gemm(xt, None, wg, sw, accum=accum, w_layout=layout)
        _, sa2 = sg.fp8_quant_per_token(xt)
        torch.cuda.synchronize()
        assert np.array_equal(host(sa).view(np.uint32), host(sa2).view(np.uint32)), what
        assert np.array_equal(host_bits16(y1), host_bits16(y0)), what
    x = rng.standard_normal((4, 512)).astype(np.float32)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    gemm_case(x, w, accum=accum, what=f"fp32 activations {accum} {layout}", layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("m", [1, 4, 32, 300])
def test_exact_mode_widens_every_code(m, layout):
    """One-hot weights (code 0x38 = 1.0 at k = n) against activation rows that
    hold every one of the 254 finite E4M3 codes: in exact mode each output is
    exactly the decoded activation code, so the FP8 -> bf16 widening of every
    code, both signs, subnormals and the maximum included, is checked bit for
    bit (skinny kernels for M <= 32, the large-tile kernel above)."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert finite.size == 254
    K = 256
    rng = np.random.default_rng(m)
    a = np.zeros((m, K), np.uint8)
    for i in range(m):
        a[i, :254] = rng.permutation(finite)
    n = K
    w = np.zeros((n, K), np.uint8)
    w[np.arange(n), np.arange(n)] = 0x38
    wt = dev(w)
    wg = sg.fp8_pack_weights(wt) if layout == "packed" else wt
    one_m = torch.ones(m, dtype=torch.float32, device="cuda")
    one_n = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    sg.fp8_scaled_gemm(dev(a), one_m, wg, one_n, y=y, out_dtype=torch.float32, accum="exact", w_layout=layout)
    torch.cuda.synchronize()
    got = host(y).astype(np.float64)
    want = fp8.decode(a)
    assert np.array_equal(got, want), f"{int((got != want).sum())} outputs differ"
    # the sign of zero is not asked for: the accumulator starts at +0


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("m", [1, 4, 20, 300])
def test_empty_reduction(m, accum):
    """K = 0: an empty sum.  bf16 per-token activations with M <= 4 take the
    two-kernel path (the row quantizer writes the unit scales), never the
    decode kernel that quantizes inside the GEMM; M = 20 runs the two-m-tile
    decode kernel and M = 300 the large-tile kernels; every output is 0."""
    n = 40
    x = torch.empty((m, 0), dtype=torch.bfloat16, device="cuda")
    wq = torch.empty((n, 0), dtype=torch.uint8, device="cuda")
    sw = torch.full((n,), 3.0, dtype=torch.float32, device="cuda")
    assert sg.fp8_scaled_gemm_workspace_size(torch.bfloat16, "per_token", m, n, 0) > 0
    for out_dtype in (torch.bfloat16, torch.float32):
        sa = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda")
        y = torch.full((m, n), float("nan"), dtype=out_dtype, device="cuda")
        sg.fp8_scaled_gemm(x, sa, wq, sw, y=y, out_dtype=out_dtype, accum=accum)
        torch.cuda.synchronize()
        assert (host(sa) == 1.0).all()
        assert (host(y.float()) == 0.0).all()
    so = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    q = torch.full((m, n), 0x7F, dtype=torch.uint8, device="cuda")
    sg.fp8_scaled_gemm_fp8out(x, None, wq, sw, so, y=q, accum=accum)
    torch.cuda.synchronize()
    assert (host(q) == 0).all()
