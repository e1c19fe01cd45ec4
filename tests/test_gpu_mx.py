"""GPU parity of the MXFP8 path (fp8_quant_mx, fp8_pack_mx_scales,
fp8_scaled_gemm_mx) against the CPU oracle (oracle/mx.py), through the C ABI.

* Quantization: codes and E8M0 scale bytes bit for bit, in every layout.
* GEMM: the scaled FP8 matrix cores sum each group of 8 consecutive products
  aligned to the group's largest and truncated below 2^(e_max - 13) (the
  behaviour pinned for the unscaled instruction in tests/test_gpu_gemm.py);
  the group's products share one pair of block scales, so with p the scaled
  products, |acc - exact| <= sum_g 7 * 2^(e_max,g - 13) + (K / 32) * 2^-24 *
  sum |p| per output (one float32 rounding per 32-deep block at most).  The
  bf16 output is the float32 output of the same kernel rounded to nearest
  even, bit for bit.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_codes_equal, dev, dev_bf16, host, host_bits16, require_gpu
from oracle import fp8, mx
from oracle.fp8 import E4M3, E5M2
from test_abi_host import pack_mx_codes_reference, pack_mx_scales_reference
from workloads import bf16_bits_from_f32, decode_inputs, f32_from_bf16_bits, prefill_inputs, tiny_w8a8

pytestmark = pytest.mark.gpu

import scaled_gemm_amd as sg  # noqa: E402

FMTS = {"e4m3": E4M3, "e5m2": E5M2}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def unpack_codes(buf: np.ndarray, R: int, K: int) -> np.ndarray:
    """Inverse of the MX fragment order (include/fp8sg.h) for rows < R."""
    nkb = K // 128
    T = (R + 15) // 16
    b = buf.reshape(T, nkb, 2, 4, 16, 16)              # tile, k block, half, k group, row, byte
    out = b.transpose(0, 4, 1, 2, 3, 5).reshape(T * 16, K)   # row-major k = 128 kb + 64 h + 16 g + byte
    return out[:R]


def unpack_scales(buf: np.ndarray, R: int, K: int) -> np.ndarray:
    """Inverse of the packed MX scale layout (include/fp8sg.h) for rows < R."""
    T4 = (R + 63) // 64
    p = buf.reshape(K // 128, T4, 64, 4)                # kb, group, lane, j
    out = np.zeros((T4 * 64, K // 32), np.uint8)
    for lane in range(64):
        for j in range(4):
            rows = (4 * np.arange(T4) + j) * 16 + lane % 16
            for kb in range(K // 128):
                out[rows, 4 * kb + lane // 16] = p[kb, :, lane, j]
    return out[:R]


def special_rows(K=256):
    x = np.random.default_rng(4).standard_normal((8, K)).astype(np.float32)
    x[0, :32] = 0.0                                   # zero block: scale 2^0, +0 codes
    x[0, 32:64] = -0.0                                 # negative zeros keep their sign
    x[1, :32] = 448.0                                  # maximum exactly at the format maximum
    x[1, 32:64] = np.float32(1e-39)                    # subnormal block maximum: scale clamps at 2^-127
    x[2, :32] *= np.float32(3e37)                      # large: scale exponent near 120
    x[3, :32] *= np.float32(2.0 ** -120)               # small normal values
    x[4, 64:96] = np.float32(2.0 ** -149)              # smallest subnormal
    x[5, :] *= 60.0
    x[6, ::7] = np.float32(57344.0)
    return x


def quant_inputs():
    x, _ = tiny_w8a8(0)
    xb, _, _ = decode_inputs(32, with_weight=False)
    rng = np.random.default_rng(8)
    rag = rng.standard_normal((37, 384)).astype(np.float32)
    rag[:, rng.integers(0, 384, 4)] *= 40
    return [("tiny fp32", x), ("decode bf16", xb), ("ragged fp32", rag), ("special fp32", special_rows())]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quant_bit_exact_every_layout(fmt):
    for what, x in quant_inputs():
        is_bf16 = x.dtype == np.uint16
        xt = dev_bf16(x) if is_bf16 else dev(x)
        xf = f32_from_bf16_bits(x) if is_bf16 else x
        R, K = xf.shape
        want_q, want_s = mx.quant_mx(xf, FMTS[fmt])
        for layout in ("row_major", "packed"):
            for sl in ("row_major", "packed"):
                q, s = sg.fp8_quant_mx(xt, fmt, layout=layout, scale_layout=sl)
                torch.cuda.synchronize()
                qh, sh = host(q), host(s)
                if layout == "packed":
                    qh = unpack_codes(qh, R, K)
                if sl == "packed":
                    sh = unpack_scales(sh, R, K)
                tag = f"{what} {fmt} codes={layout} scales={sl}"
                assert np.array_equal(sh, want_s), f"{tag}: {int((sh != want_s).sum())} scale bytes differ"
                assert_codes_equal(qh, want_q, tag)


def test_quant_full_decode_row_bf16_and_large_rows():
    xb, _, _ = prefill_inputs(4096, m=512, n=16, with_weight=False)
    want_q, want_s = mx.quant_mx(f32_from_bf16_bits(xb), E4M3)
    q, s = sg.fp8_quant_mx(dev_bf16(xb), "e4m3")
    torch.cuda.synchronize()
    assert np.array_equal(host(s), want_s)
    assert_codes_equal(host(q), want_q, "prefill rows bf16")


def test_pack_mx_scales_matches_the_documented_layout():
    rng = np.random.default_rng(2)
    for R, K in ((1, 128), (16, 256), (70, 384), (130, 1024)):
        s = rng.integers(0, 255, (R, K // 32), dtype=np.uint8)
        got = host(sg.fp8_pack_mx_scales(dev(s)))
        assert np.array_equal(got, pack_mx_scales_reference(s)), (R, K)


def mx_bound(a_vals: np.ndarray, w_vals: np.ndarray) -> np.ndarray:
    """Error bound of the scaled FP8 matrix-core accumulation per output, from
    the exactly scaled operand values (float64 [r, K] and [c, K])."""
    K = a_vals.shape[1]
    out = np.zeros((a_vals.shape[0], w_vals.shape[0]))
    for i in range(a_vals.shape[0]):
        p = a_vals[i][None, :] * w_vals
        g = np.abs(p).reshape(w_vals.shape[0], K // 8, 8).max(axis=-1)
        e = np.floor(np.log2(np.where(g > 0, g, 1.0)))
        grp = np.where(g > 0, 7.0 * np.exp2(e - 13), 0.0).sum(axis=-1)
        out[i] = grp + (K / 32) * 2.0 ** -24 * np.abs(p).sum(axis=-1)
    return out


_WCACHE = {}


def _quant_w(w):
    key = (w.shape, float(w[0, 0]), float(w[-1, -1]))
    if key not in _WCACHE:
        _WCACHE.clear()
        _WCACHE[key] = mx.quant_mx(w, E4M3)
    return _WCACHE[key]


def run_gemm(x, w, *, a_fmt="e4m3", w_layout="row_major", a_layout="row_major", rows=None, cols=None, what=""):
    """Quantize x and w with the oracle (codes bit-exact with the GPU
    quantizer, tested above), run the GPU GEMM with fp32 and bf16 output and
    check the sampled outputs."""
    fa = FMTS[a_fmt]
    aq, ae = mx.quant_mx(x, fa)
    wq, we = _quant_w(w)
    M, K = aq.shape
    N = wq.shape[0]
    a_t, w_t = dev(aq), dev(wq)
    a_in = dev(pack_mx_codes_reference(aq)) if a_layout == "packed" else a_t
    w_in = dev(pack_mx_codes_reference(wq)) if w_layout == "packed" else w_t
    as_p, ws_p = sg.fp8_pack_mx_scales(dev(ae)), sg.fp8_pack_mx_scales(dev(we))
    kw = dict(a_fmt=a_fmt, w_layout=w_layout, a_layout=a_layout, a_shape=(M, K), w_shape=(N, K))
    y32 = sg.fp8_scaled_gemm_mx(a_in, as_p, w_in, ws_p, out_dtype=torch.float32, **kw)
    y16 = sg.fp8_scaled_gemm_mx(a_in, as_p, w_in, ws_p, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    cols = np.arange(N) if cols is None else cols
    y32h = host(y32)[np.ix_(rows, cols)].astype(np.float64)
    y16h = host_bits16(y16)[np.ix_(rows, cols)]
    exact = mx.gemm_mx_exact(aq[rows], ae[rows], wq[cols], we[cols], fa)
    bound = mx_bound(mx.dequant_mx(aq[rows], ae[rows], fa), mx.dequant_mx(wq[cols], we[cols]))
    err = np.abs(y32h - exact)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs outside the bound; worst err/bound "
                           f"{np.max(err / np.maximum(bound, 1e-300)):.3g}")
    mism = fp8.bf16_round_bits(y32h) != y16h
    assert not mism.any(), f"{what}: {int(mism.sum())} bf16 outputs differ from the rounded fp32 output"


def _gemm_shapes():
    rng = np.random.default_rng(9)
    out = []
    for m, n, k in ((16, 512, 256), (5, 77, 384), (33, 130, 512), (300, 1000, 1024), (1, 1, 128), (64, 64, 128)):
        x = rng.standard_normal((m, k)).astype(np.float32)
        x[:, rng.integers(0, k, 3)] *= 40
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        w[rng.integers(0, n, 2), :64] *= 300.0
        out.append((x, w))
    return out


@pytest.mark.parametrize("a_fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("layout", ["row_major", "packed"])
def test_gemm_tiny_and_ragged(a_fmt, layout):
    for x, w in _gemm_shapes():
        run_gemm(x, w, a_fmt=a_fmt, w_layout=layout, a_layout=layout,
                 what=f"{x.shape[0]}x{w.shape[0]}x{x.shape[1]} {a_fmt} {layout}")
    x, w = _gemm_shapes()[3]
    run_gemm(x, w, a_fmt=a_fmt, w_layout=layout, a_layout="row_major" if layout == "packed" else "packed",
             what=f"mixed layouts {a_fmt} {layout}")


@pytest.mark.parametrize("m", [1, 8, 32])
def test_gemm_decode_full_size(m):
    xb, w, _ = decode_inputs(m)
    cols = np.unique(np.concatenate([np.arange(64), np.random.default_rng(m).choice(14336, 1024, replace=False),
                                     np.arange(14336 - 64, 14336)]))
    run_gemm(f32_from_bf16_bits(xb), w, w_layout="packed", a_layout="packed", cols=cols, what=f"decode M={m}")


@pytest.mark.parametrize("a_fmt", ["e4m3", "e5m2"])
def test_gemm_prefill_sampled(a_fmt):
    xb, w, _ = prefill_inputs(4096, m=2048)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 255, 256, 2047], rng.choice(2048, 24, replace=False)]))
    cols = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 256, replace=False)]))
    run_gemm(f32_from_bf16_bits(xb), w, a_fmt=a_fmt, w_layout="packed", a_layout="packed", rows=rows, cols=cols,
             what=f"prefill {a_fmt}")


def test_decode_path_quantized_on_the_gpu():
    """The decode usage: activations quantized on the GPU straight into the
    packed codes and scales the GEMM reads."""
    xb, w, _ = decode_inputs(8)
    wq, we = mx.quant_mx(w, E4M3)
    w_in, ws_p = sg.fp8_quant_mx(dev(w), "e4m3", layout="packed", scale_layout="packed")
    q, s = sg.fp8_quant_mx(dev_bf16(xb), "e4m3", layout="packed", scale_layout="packed")
    y = sg.fp8_scaled_gemm_mx(q, s, w_in, ws_p, out_dtype=torch.float32, w_layout="packed", a_layout="packed",
                              a_shape=(8, 4096), w_shape=(14336, 4096))
    torch.cuda.synchronize()
    aq, ae = mx.quant_mx(f32_from_bf16_bits(xb), E4M3)
    cols = np.arange(0, 14336, 7)
    exact = mx.gemm_mx_exact(aq, ae, wq[cols], we[cols])
    bound = mx_bound(mx.dequant_mx(aq, ae), mx.dequant_mx(wq[cols], we[cols]))
    assert (np.abs(host(y)[:, cols].astype(np.float64) - exact) <= bound).all()


@pytest.mark.parametrize("m", [3, 300], ids=["decode_kernel", "large_tile_kernel"])
def test_zero_depth_and_empty(m):
    a = torch.zeros((m, 0), dtype=torch.uint8, device="cuda")
    w = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    e = torch.zeros((0,), dtype=torch.uint8, device="cuda")
    y = torch.full((m, 5), 7.0, dtype=torch.float32, device="cuda")
    lib = sg.lib()
    st = lib.fp8_scaled_gemm_mx(a.data_ptr(), e.data_ptr(), sg.E4M3, w.data_ptr(), e.data_ptr(), 0, y.data_ptr(),
                                sg.F32, m, 5, 0, None)
    torch.cuda.synchronize()
    assert st == 0 and (host(y) == 0).all()


def test_deterministic_repeats():
    x, w = _gemm_shapes()[3]
    aq, ae = mx.quant_mx(x, E4M3)
    wq, we = mx.quant_mx(w, E4M3)
    args = (dev(aq), sg.fp8_pack_mx_scales(dev(ae)), dev(wq), sg.fp8_pack_mx_scales(dev(we)))
    y0 = host(sg.fp8_scaled_gemm_mx(*args, out_dtype=torch.float32))
    for _ in range(3):
        assert np.array_equal(host(sg.fp8_scaled_gemm_mx(*args, out_dtype=torch.float32)), y0)


# ---------------------------------------------------------------------------
# fp8_scaled_gemm_mx_bf16: the decode MX GEMM on bf16 activations quantized inside the kernel.

def _bf16x_cases():
    rng = np.random.default_rng(21)
    out = []
    for m, n, k in ((1, 77, 128), (5, 130, 384), (16, 512, 256), (9, 96, 512), (16, 1000, 1024)):
        x = rng.standard_normal((m, k)).astype(np.float32)
        x[:, rng.integers(0, k, 3)] *= 40
        x[0, :32] = 0.0                               # a zero block
        if m > 1:
            x[1, 32:64] *= np.float32(2.0 ** -120)    # a block of tiny values
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        w[rng.integers(0, n, 2), :64] *= 300.0
        out.append((bf16_bits_from_f32(x), w))
    return out


@pytest.mark.parametrize("a_fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("w_layout", ["row_major", "packed"])
def test_bf16x_equals_quantize_then_gemm(a_fmt, w_layout):
    """One launch on bf16 X gives the same bits as fp8_quant_mx followed by
    fp8_scaled_gemm_mx: the same codes, scales and products in the same order."""
    for xb, w in _bf16x_cases():
        M, K = xb.shape
        N = w.shape[0]
        x = dev_bf16(xb)
        wq, ws = sg.fp8_quant_mx(dev(w), "e4m3", layout=w_layout, scale_layout="packed")
        q, s = sg.fp8_quant_mx(x, a_fmt, layout="packed", scale_layout="packed")
        kw = dict(a_fmt=a_fmt, w_layout=w_layout, w_shape=(N, K))
        for out in (torch.float32, torch.bfloat16):
            y2 = sg.fp8_scaled_gemm_mx(q, s, wq, ws, out_dtype=out, a_layout="packed", a_shape=(M, K), **kw)
            y1 = sg.fp8_scaled_gemm_mx_bf16(x, wq, ws, out_dtype=out, **kw)
            torch.cuda.synchronize()
            assert torch.equal(y1.view(torch.int16 if out == torch.bfloat16 else torch.int32),
                               y2.view(torch.int16 if out == torch.bfloat16 else torch.int32)), \
                f"{M}x{N}x{K} {a_fmt} {w_layout} {out}"


@pytest.mark.parametrize("m", [1, 8, 16])
def test_bf16x_decode_against_the_oracle(m):
    """Full decode shape, sampled columns: within the scaled matrix cores' bound
    of the exact sum over the oracle's MX codes of the same bf16 X."""
    xb, w, _ = decode_inputs(m)
    wq, we = _quant_w(w)
    w_in, ws_p = sg.fp8_quant_mx(dev(w), "e4m3", layout="packed", scale_layout="packed")
    y = sg.fp8_scaled_gemm_mx_bf16(dev_bf16(xb), w_in, ws_p, out_dtype=torch.float32, w_layout="packed",
                                   w_shape=(14336, 4096))
    torch.cuda.synchronize()
    aq, ae = mx.quant_mx(f32_from_bf16_bits(xb), E4M3)
    cols = np.unique(np.concatenate([np.arange(32), np.arange(0, 14336, 37), np.arange(14336 - 32, 14336)]))
    exact = mx.gemm_mx_exact(aq, ae, wq[cols], we[cols])
    bound = mx_bound(mx.dequant_mx(aq, ae), mx.dequant_mx(wq[cols], we[cols]))
    err = np.abs(host(y)[:, cols].astype(np.float64) - exact)
    assert (err <= bound).all(), f"M={m}: worst err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"


def test_bf16x_zero_depth_and_shape_limit():
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    e = torch.zeros((0,), dtype=torch.uint8, device="cuda")
    y = torch.full((3, 5), 7.0, dtype=torch.float32, device="cuda")
    lib = sg.lib()
    st = lib.fp8_scaled_gemm_mx_bf16(x.data_ptr(), sg.E4M3, w.data_ptr(), e.data_ptr(), 0, y.data_ptr(), sg.F32,
                                     3, 5, 0, None)
    torch.cuda.synchronize()
    assert st == 0 and (host(y) == 0).all()
    xb = torch.zeros((17, 128), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((sg.fp8_mx_packed_scale_bytes(8, 128),), dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        sg.fp8_scaled_gemm_mx_bf16(xb, wq, ws)
