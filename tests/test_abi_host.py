"""The C-ABI library without a GPU: it loads, exports every entry point that
include/fp8sg.h declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import subprocess

import pytest

import scaled_gemm_amd as sg
from scaled_gemm_amd import fp8sg as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    names = sg.declared_symbols()
    assert len(names) == 26
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = sg.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings_and_version():
    assert sg.lib().fp8sg_version() == 9
    for st in range(9):
        assert sg.status_string(st)
    assert sg.status_string(99) == "unknown status"


def test_binding_names_match_the_header():
    py = {n for n in dir(sg) if n.startswith("fp8_")}
    declared = {n for n in sg.declared_symbols() if n.startswith("fp8_")}
    assert declared <= py


L = None


@pytest.fixture(scope="module")
def lib():
    return sg.lib()


A = 4096  # a 16-byte-aligned fake device address: never dereferenced, validation fails first


def test_blockwise_validation(lib):
    # group quantizer: K % 128, dtype, layout bits, nulls, alignment, empty work
    assert lib.fp8_quant_per_token_group(A, b.BF16, 4, 64, A, A, 0, None) == b.E_SHAPE
    assert lib.fp8_quant_per_token_group(A, b.E4M3, 4, 128, A, A, 0, None) == b.E_DTYPE
    assert lib.fp8_quant_per_token_group(A, b.BF16, 4, 128, A, A, b.W_PACKED, None) == b.E_DTYPE
    assert lib.fp8_quant_per_token_group(A, b.BF16, 4, 128, A, A, b.MX_SCALES_PACKED, None) == b.E_DTYPE
    # the k-block-major scale layout is accepted (it fails later only for lack of a device)
    assert lib.fp8_quant_per_token_group(None, b.BF16, 0, 128, None, None, b.SCALES_KMAJOR | b.A_PACKED, None) == b.OK
    assert lib.fp8_quant_per_token_group(A, b.BF16, 4, 128, A, None, 0, None) == b.E_NULL
    assert lib.fp8_quant_per_token_group(A + 4, b.BF16, 4, 128, A, A, 0, None) == b.E_ALIGN
    assert lib.fp8_quant_per_token_group(None, b.BF16, 0, 128, None, None, 0, None) == b.OK
    # weight blocks
    assert lib.fp8_quant_weight_blockwise(A, b.F32, 4, 100, A, A, None) == b.E_SHAPE
    assert lib.fp8_quant_weight_blockwise(A, b.E5M2, 4, 128, A, A, None) == b.E_DTYPE
    assert lib.fp8_quant_weight_blockwise(A, b.F32, 4, 128, None, A, None) == b.E_NULL
    assert lib.fp8_quant_weight_blockwise(None, b.F32, 0, 128, None, None, None) == b.OK
    # GEMM: accumulation mode; K % 128; layout bits; nulls; alignment
    g = lib.fp8_scaled_gemm_blockwise
    assert g(A, A, A, 0, A, A, b.BF16, 33, 8, 128, 7, None) == b.E_DTYPE
    # exact accumulation at every M (an empty call succeeds without a device)
    assert g(None, None, None, 0, None, None, b.BF16, 0, 8, 128, b.ACCUM_EXACT, None) == b.OK
    assert g(A, A, A, 0, A, A, b.BF16, 4, 8, 100, b.ACCUM_MFMA_FP8, None) == b.E_SHAPE
    assert g(A, A, A, 4, A, A, b.BF16, 4, 8, 128, b.ACCUM_MFMA_FP8, None) == b.E_DTYPE
    assert g(A, A, A, 16, A, A, b.BF16, 4, 8, 128, b.ACCUM_MFMA_FP8, None) == b.E_DTYPE
    assert g(None, None, None, b.SCALES_KMAJOR, None, None, b.BF16, 0, 8, 128, b.ACCUM_MFMA_FP8, None) == b.OK
    assert g(A, A, A, 0, A, A, b.E4M3, 4, 8, 128, b.ACCUM_MFMA_FP8, None) == b.E_DTYPE
    assert g(A, None, A, 0, A, A, b.BF16, 4, 8, 128, b.ACCUM_MFMA_FP8, None) == b.E_NULL
    assert g(A, A, A, 0, A + 2, A, b.BF16, 4, 8, 128, b.ACCUM_MFMA_FP8, None) == b.E_ALIGN
    assert g(None, None, None, 0, None, None, b.BF16, 0, 8, 128, b.ACCUM_MFMA_FP8, None) == b.OK


def test_attention_validation(lib):
    f = lib.fp8_kv_decode_attention
    ws = lib.fp8_kv_decode_attention_workspace_size(8, 32768, 32, 8, 128)
    assert ws == 8 * 8 * 32 * 4 * 130 * 4
    assert lib.fp8_kv_decode_attention_workspace_size(8, 32768, 32, 8, 64) == 0   # D must be 128

    def call(**kw):
        d = dict(q=A, k=A, v=A, sk=A, sv=A, fmt=b.E4M3, L=A, B=8, S=32768, Hq=32, Hkv=8, D=128, scale=0.0, out=A,
                 odt=b.BF16, ws=A, wsb=ws)
        d.update(kw)
        return f(d["q"], d["k"], d["v"], d["sk"], d["sv"], d["fmt"], d["L"], d["B"], d["S"], d["Hq"], d["Hkv"],
                 d["D"], d["scale"], d["out"], d["odt"], d["ws"], d["wsb"], None)

    assert call(fmt=b.BF16) == b.E_DTYPE
    assert call(odt=b.E4M3) == b.E_DTYPE
    assert call(D=64) == b.E_SHAPE
    assert call(Hq=30) == b.E_SHAPE           # not a multiple of Hkv
    assert call(Hq=24) == b.E_SHAPE           # G = 3
    assert call(Hq=128) == b.E_SHAPE          # G = 16
    assert call(scale=float("nan")) == b.E_SHAPE
    assert call(L=None) == b.E_NULL
    assert call(v=None) == b.E_NULL
    assert call(q=A + 8) == b.E_ALIGN
    assert call(wsb=ws - 1) == b.E_WORKSPACE
    assert call(ws=None) == b.E_WORKSPACE
    assert call(B=0, q=None, k=None, v=None, out=None) == b.OK


def test_quant_validation(lib):
    assert lib.fp8_quant_per_token(A, 7, 4, 16, A, A, None) == b.E_DTYPE
    assert lib.fp8_quant_per_token(A, b.BF16, 4, 17, A, A, None) == b.E_SHAPE
    assert lib.fp8_quant_per_token(A, b.BF16, -1, 16, A, A, None) == b.E_SHAPE
    assert lib.fp8_quant_per_token(None, b.BF16, 4, 16, A, A, None) == b.E_NULL
    assert lib.fp8_quant_per_token(A, b.BF16, 4, 16, A, None, None) == b.E_NULL
    assert lib.fp8_quant_per_token(A + 8, b.BF16, 4, 16, A, A, None) == b.E_ALIGN
    assert lib.fp8_quant_per_token(A, b.BF16, 4, 16, A, A + 2, None) == b.E_ALIGN
    assert lib.fp8_quant_per_token(A, b.BF16, 0, 16, None, None, None) == b.OK
    assert lib.fp8_quant_weight_per_channel(A, b.E4M3, 4, 16, A, A, None) == b.E_DTYPE
    assert lib.fp8_quant_per_tensor_static(A, b.F32, 100, A, 9, A, None) == b.E_DTYPE
    assert lib.fp8_quant_per_tensor_static(A, b.E4M3, 100, A, b.E4M3, A, None) == b.E_DTYPE
    assert lib.fp8_quant_per_tensor_static(A, b.F32, 100, None, b.E4M3, A, None) == b.E_NULL
    assert lib.fp8_quant_per_tensor_static(A, b.F32, 0, None, b.E4M3, None, None) == b.OK


def test_gemm_validation(lib):
    g = lib.fp8_scaled_gemm
    ok = dict(a=A, a_dt=b.E4M3, sa=A, mode=b.SCALE_PER_TOKEN, wq=A, lay=b.W_ROW_MAJOR, sw=A, y=A, y_dt=b.BF16, M=4,
              N=8, K=128, accum=b.ACCUM_EXACT, ws=None, wsb=0)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return g(d["a"], d["a_dt"], d["sa"], d["mode"], d["wq"], d["lay"], d["sw"], d["y"], d["y_dt"], d["M"], d["N"],
                 d["K"], d["accum"], d["ws"], d["wsb"], None)

    assert call(lay=4) == b.E_DTYPE
    assert call(lay=b.W_PACKED | 4) == b.E_DTYPE
    # packed activation codes only: high-precision activations are row-major
    assert call(lay=b.A_PACKED, a_dt=b.BF16) == b.E_DTYPE
    assert call(K=100) == b.E_SHAPE
    assert call(a_dt=b.E5M2) == b.E_DTYPE
    assert call(y_dt=b.E4M3) == b.E_DTYPE
    assert call(mode=5) == b.E_DTYPE
    assert call(accum=2) == b.E_DTYPE
    assert call(sa=None) == b.E_NULL
    assert call(wq=None) == b.E_NULL
    assert call(y=A + 4) == b.E_ALIGN
    assert call(M=0) == b.OK
    # a bf16 activation needs the workspace the size query reports: the codes
    # (fragment order, rows padded to 16, for M <= 32, for every per-tensor
    # scale and for per-token rows when K <= 8192 bf16 / 4096 fp32; other
    # per-token rows above 32 row-major), then
    # the per-token scales -- except bf16 per-token with M <= 4 and K <= 4096,
    # which the decode kernel quantizes itself (no workspace)
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 4, 8, 128) == 0
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 1, 8, 4096) == 0
    assert lib.fp8_scaled_gemm_workspace_size(b.F32, b.SCALE_PER_TOKEN, 1, 8, 4096) == 16 * 4096 + 256
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 4, 8, 4224) == 16 * 4224 + 256
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 5, 8, 128) == 16 * 128 + 256
    need = lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 12, 8, 128)
    assert need == 16 * 128 + 256
    assert lib.fp8_scaled_gemm_workspace_size(b.E4M3, b.SCALE_PER_TOKEN, 4, 8, 128) == 0
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TENSOR, 4, 8, 128) == 16 * 128
    assert lib.fp8_scaled_gemm_workspace_size(b.F32, b.SCALE_PER_TENSOR, 17, 8, 256) == 32 * 256
    assert lib.fp8_scaled_gemm_workspace_size(b.F32, b.SCALE_PER_TENSOR, 33, 8, 256) == 48 * 256
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TENSOR, 4096, 8, 8192) == 4096 * 8192
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 33, 8, 128) == 48 * 128 + 256
    al = lambda v: (v + 255) // 256 * 256
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 4100, 8, 8192) == al(4112 * 8192) + al(4100 * 4)
    # past the tile quantizer's register budget: row-major codes
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 33, 8, 8320) == al(33 * 8320) + al(33 * 4)
    assert lib.fp8_scaled_gemm_workspace_size(b.F32, b.SCALE_PER_TOKEN, 33, 8, 4224) == al(33 * 4224) + al(33 * 4)
    assert call(a_dt=b.BF16, sa=None, M=12) == b.E_WORKSPACE
    assert call(a_dt=b.BF16, sa=None, M=12, ws=A, wsb=need - 1) == b.E_WORKSPACE
    assert call(a_dt=b.BF16, sa=None, M=12, ws=A + 16, wsb=need) == b.E_ALIGN
    assert call(a_dt=b.BF16, mode=b.SCALE_PER_TENSOR, sa=None, ws=A, wsb=need) == b.E_NULL


def test_gemm_empty_reduction_takes_the_row_quantizer(lib):
    # K == 0 never reaches the decode kernel that quantizes inside the GEMM (its
    # loads assume at least one k block): a bf16 per-token call with K == 0 asks
    # for the workspace of the two-kernel path (no codes, the unit scales)
    for m in (1, 4):
        assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, m, 8, 0) == 256
        assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, m, 8, 128) == 0
    g = lib.fp8_scaled_gemm
    # without that workspace the call is refused before any HIP call
    assert g(None, b.BF16, None, b.SCALE_PER_TOKEN, None, 0, A, A, b.BF16, 4, 8, 0, b.ACCUM_EXACT, None, 0,
             None) == b.E_WORKSPACE
    assert g(None, b.BF16, A, b.SCALE_PER_TOKEN, None, 0, A, A, b.BF16, 1, 8, 0, b.ACCUM_EXACT, None, 0,
             None) == b.E_WORKSPACE


def test_gemm_reduction_length_limit(lib):
    # per-lane tile offsets are 32-bit: K < 2^24 on every GEMM entry point
    big = 1 << 24
    g = lib.fp8_scaled_gemm
    assert g(A, b.E4M3, A, b.SCALE_PER_TOKEN, A, 0, A, A, b.BF16, 64, 8, big, b.ACCUM_EXACT, None, 0,
             None) == b.E_SHAPE
    import torch
    if not torch.cuda.is_available():  # with a device these fake addresses would reach a kernel
        assert g(A, b.E4M3, A, b.SCALE_PER_TOKEN, A, 0, A, A, b.BF16, 64, 8, big - 128, b.ACCUM_EXACT, None, 0,
                 None) == b.E_DEVICE
    assert lib.fp8_scaled_gemm_fp8out(A, b.E4M3, A, b.SCALE_PER_TOKEN, A, 0, A, A, A, 64, 8, big, b.ACCUM_EXACT,
                                      None, 0, None) == b.E_SHAPE
    assert lib.fp8_scaled_gemm_blockwise(A, A, A, 0, A, A, b.BF16, 64, 8, big, b.ACCUM_MFMA_FP8,
                                         None) == b.E_SHAPE
    assert lib.fp8_scaled_gemm_mx(A, A, b.E4M3, A, A, 0, A, b.BF16, 64, 8, big, None) == b.E_SHAPE
    assert lib.fp8_scaled_gemm_mx_bf16(A, b.E4M3, A, A, 0, A, b.BF16, 4, 8, big, None) == b.E_SHAPE


def test_pack_validation(lib):
    assert lib.fp8_packed_weight_bytes(17, 256) == 32 * 256
    assert lib.fp8_packed_weight_bytes(0, 256) == 0
    assert lib.fp8_pack_weights(A, 17, 100, A, None) == b.E_SHAPE
    assert lib.fp8_pack_weights(None, 17, 128, A, None) == b.E_NULL
    assert lib.fp8_pack_weights(A, 17, 128, A + 4, None) == b.E_ALIGN
    assert lib.fp8_pack_weights(A, 0, 128, None, None) == b.OK


def pack_reference(wq):
    """The packed layout written out from its definition in include/fp8sg.h."""
    import numpy as np
    N, K = wq.shape
    rows = (N + 15) // 16 * 16
    w = np.zeros((rows, K), np.uint8)
    w[:N] = wq
    nkb = K // 128
    out = np.zeros(rows * K, np.uint8)
    for t in range(rows // 16):
        for kb in range(nkb):
            base = (t * nkb + kb) * 2048
            for lane in range(64):
                r = 16 * t + lane % 16
                k0 = kb * 128 + 32 * (lane // 16)
                out[base + lane * 16: base + lane * 16 + 16] = w[r, k0:k0 + 16]
                out[base + 1024 + lane * 16: base + 1024 + lane * 16 + 16] = w[r, k0 + 16:k0 + 32]
    return out


def test_pack_reference_is_a_permutation():
    import numpy as np
    rng = np.random.default_rng(0)
    wq = rng.integers(0, 256, (37, 384), dtype=np.uint8)
    p = pack_reference(wq)
    assert p.size == 48 * 384
    # every original byte appears exactly once, the padding rows are zero
    padded = np.zeros((48, 384), np.uint8)
    padded[:37] = wq
    assert np.array_equal(np.sort(p), np.sort(padded.ravel()))


def test_kv_validation(lib):
    assert lib.fp8_kv_quant(A, 2, 4, 8, 24, A, b.E4M3, A, None) == b.E_SHAPE
    assert lib.fp8_kv_quant(A, 2, 4, 8, 32, A, b.BF16, A, None) == b.E_DTYPE
    assert lib.fp8_kv_quant(None, 2, 4, 8, 32, A, b.E4M3, A, None) == b.E_NULL
    assert lib.fp8_kv_dequant(A, 2, 4, 8, 32, None, b.E5M2, A, None) == b.E_NULL
    assert lib.fp8_kv_dequant(A + 1, 2, 4, 8, 32, A, b.E5M2, A, None) == b.E_ALIGN
    assert lib.fp8_kv_calibrate(A, 2, 4, 8, 32, b.E4M3, None, None) == b.E_NULL
    assert lib.fp8_kv_append(A, None, 2, 4, 8, 32, A, b.E4M3, A, None) == b.E_NULL
    assert lib.fp8_kv_append(A, A + 2, 2, 4, 8, 32, A, b.E4M3, A, None) == b.E_ALIGN
    assert lib.fp8_kv_quant(A, 0, 4, 8, 32, A, b.E4M3, A, None) == b.OK


def test_no_device_is_reported_not_faked(lib):
    """Valid arguments on a machine without a gfx950 device: FP8SG_E_DEVICE, never
    a silent fallback."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a HIP device is present")
    assert lib.fp8_quant_per_token(A, b.BF16, 4, 16, A, A, None) == b.E_DEVICE
    assert lib.fp8_kv_quant(A, 2, 4, 8, 32, A, b.E4M3, A, None) == b.E_DEVICE


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        sg.fp8_quant_per_token(torch.zeros((2, 16), dtype=torch.bfloat16))


def pack_mx_scales_reference(s):
    """The packed MX scale layout written out from its definition in include/fp8sg.h:
    s [rows, K / 32] E8M0 bytes -> ceil(rows / 64) * 256 * (K / 128) bytes, rows past
    the end 127."""
    import numpy as np
    R, nb = s.shape
    K = 32 * nb
    T4 = (R + 63) // 64
    out = np.zeros((K // 128) * T4 * 256, np.uint8)
    for kb in range(K // 128):
        for g in range(T4):
            for lane in range(64):
                for j in range(4):
                    r = 16 * (4 * g + j) + lane % 16
                    b = 4 * kb + lane // 16
                    out[(kb * T4 + g) * 256 + 4 * lane + j] = s[r, b] if r < R else 127
    return out


def test_mx_packed_scale_bytes_and_reference_layout():
    import numpy as np
    assert sg.fp8_mx_packed_scale_bytes(1, 128) == 256
    assert sg.fp8_mx_packed_scale_bytes(64, 4096) == 256 * 32
    assert sg.fp8_mx_packed_scale_bytes(65, 256) == 2 * 256 * 2
    assert sg.fp8_mx_packed_scale_bytes(0, 128) == 0
    # the reference is a bijection of the real rows' bytes onto their slots, padding 127
    rng = np.random.default_rng(0)
    s = rng.integers(0, 255, (70, 8), dtype=np.uint8)
    p = pack_mx_scales_reference(s)
    assert p.size == sg.fp8_mx_packed_scale_bytes(70, 256)
    assert np.array_equal(np.sort(p[p != 127]), np.sort(s[s != 127].ravel()))
    assert (p == 127).sum() == (s == 127).sum() + (128 - 70) * 8


def test_mx_validation(lib):
    # quantizer: dtype, format, layout bits, K multiple, nulls, alignment, empty work
    assert lib.fp8_quant_mx(A, b.E4M3, 4, 128, b.E4M3, A, A, 0, None) == b.E_DTYPE
    assert lib.fp8_quant_mx(A, b.BF16, 4, 128, b.BF16, A, A, 0, None) == b.E_DTYPE
    assert lib.fp8_quant_mx(A, b.BF16, 4, 128, b.E4M3, A, A, 8, None) == b.E_DTYPE
    assert lib.fp8_quant_mx(A, b.BF16, 4, 48, b.E4M3, A, A, 0, None) == b.E_SHAPE
    assert lib.fp8_quant_mx(A, b.BF16, 4, 96, b.E4M3, A, A, b.MX_SCALES_PACKED, None) == b.E_SHAPE
    assert lib.fp8_quant_mx(A, b.BF16, 4, 128, b.E4M3, A, None, 0, None) == b.E_NULL
    assert lib.fp8_quant_mx(A + 4, b.BF16, 4, 128, b.E4M3, A, A, 0, None) == b.E_ALIGN
    assert lib.fp8_quant_mx(None, b.BF16, 0, 128, b.E5M2, None, None, 0, None) == b.OK
    # scale packing
    assert lib.fp8_pack_mx_scales(A, 4, 96, A, None) == b.E_SHAPE
    assert lib.fp8_pack_mx_scales(None, 4, 128, A, None) == b.E_NULL
    assert lib.fp8_pack_mx_scales(None, 0, 128, None, None) == b.OK
    # GEMM: output dtype, activation format, layout bits, K multiple, nulls, alignment, empty work
    assert lib.fp8_scaled_gemm_mx(A, A, b.E4M3, A, A, 0, A, b.E4M3, 4, 8, 128, None) == b.E_DTYPE
    assert lib.fp8_scaled_gemm_mx(A, A, b.BF16, A, A, 0, A, b.BF16, 4, 8, 128, None) == b.E_DTYPE
    assert lib.fp8_scaled_gemm_mx(A, A, b.E4M3, A, A, 4, A, b.BF16, 4, 8, 128, None) == b.E_DTYPE
    assert lib.fp8_scaled_gemm_mx(A, A, b.E4M3, A, A, 0, A, b.BF16, 4, 8, 96, None) == b.E_SHAPE
    assert lib.fp8_scaled_gemm_mx(A, None, b.E4M3, A, A, 0, A, b.BF16, 4, 8, 128, None) == b.E_NULL
    assert lib.fp8_scaled_gemm_mx(A, A, b.E4M3, A, A, 0, None, b.BF16, 4, 8, 128, None) == b.E_NULL
    assert lib.fp8_scaled_gemm_mx(A + 8, A, b.E4M3, A, A, 0, A, b.BF16, 4, 8, 128, None) == b.E_ALIGN
    assert lib.fp8_scaled_gemm_mx(A, A + 2, b.E4M3, A, A, 0, A, b.BF16, 4, 8, 128, None) == b.E_ALIGN
    assert lib.fp8_scaled_gemm_mx(None, None, b.E5M2, None, None, 0, None, b.F32, 0, 8, 128, None) == b.OK
    # GEMM on bf16 activations quantized inside the kernel: as above, plus M <= 16 and W-only layout bits
    g = lib.fp8_scaled_gemm_mx_bf16
    assert g(A, b.E4M3, A, A, 0, A, b.E4M3, 4, 8, 128, None) == b.E_DTYPE          # output dtype
    assert g(A, b.BF16, A, A, 0, A, b.BF16, 4, 8, 128, None) == b.E_DTYPE          # activation format
    assert g(A, b.E4M3, A, A, b.A_PACKED, A, b.BF16, 4, 8, 128, None) == b.E_DTYPE  # x is row-major bf16
    assert g(A, b.E4M3, A, A, 0, A, b.BF16, 4, 8, 96, None) == b.E_SHAPE
    assert g(A, b.E4M3, A, A, 0, A, b.BF16, 17, 8, 128, None) == b.E_SHAPE         # one 16-row m-tile only
    assert g(None, b.E4M3, A, A, 0, A, b.BF16, 4, 8, 128, None) == b.E_NULL
    assert g(A, b.E4M3, A, None, 0, A, b.BF16, 4, 8, 128, None) == b.E_NULL
    assert g(A, b.E4M3, A, A, 0, None, b.BF16, 4, 8, 128, None) == b.E_NULL
    assert g(A + 8, b.E4M3, A, A, 0, A, b.BF16, 4, 8, 128, None) == b.E_ALIGN
    assert g(A, b.E4M3, A, A + 2, 0, A, b.BF16, 4, 8, 128, None) == b.E_ALIGN
    assert g(None, b.E5M2, None, None, 0, None, b.F32, 0, 8, 128, None) == b.OK


def pack_mx_codes_reference(q):
    """The MX fragment order written out from its definition in include/fp8sg.h:
    codes [R, K] -> ceil(R / 16) * 16 * K bytes; lane l of the 2048-byte block of
    (16-row tile t, 128-k block kb) holds row 16 t + l % 16, k 128 kb + 16 (l / 16)
    + [0, 16) at 16 l and k 128 kb + 64 + 16 (l / 16) + [0, 16) at 1024 + 16 l;
    padding rows 0."""
    import numpy as np
    R, K = q.shape
    rows = (R + 15) // 16 * 16
    w = np.zeros((rows, K), np.uint8)
    w[:R] = q
    nkb = K // 128
    out = np.zeros(rows * K, np.uint8)
    for t in range(rows // 16):
        for kb in range(nkb):
            base = (t * nkb + kb) * 2048
            for lane in range(64):
                r = 16 * t + lane % 16
                k0 = kb * 128 + 16 * (lane // 16)
                out[base + lane * 16: base + lane * 16 + 16] = w[r, k0:k0 + 16]
                out[base + 1024 + lane * 16: base + 1024 + lane * 16 + 16] = w[r, k0 + 64:k0 + 80]
    return out


def test_mx_code_order_is_a_permutation():
    import numpy as np
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, (32, 256), dtype=np.uint8)
    p = pack_mx_codes_reference(q)
    assert np.array_equal(np.sort(p), np.sort(q.ravel()))
    assert np.array_equal(p[:16], q[0, :16]) and np.array_equal(p[1024:1040], q[0, 64:80])
    assert np.array_equal(p[16 * 17:16 * 18], q[1, 16:32])


def test_rmsnorm_quant_validation(lib):
    f = lib.fp8_rmsnorm_quant_per_token
    assert f(A, b.E4M3, A, 1e-6, 4, 128, A, A, None, 0, None) == b.E_DTYPE
    assert f(A, b.BF16, A, 1e-6, 4, 128, A, A, None, b.W_PACKED, None) == b.E_DTYPE
    assert f(A, b.BF16, A, 1e-6, 4, 20000, A, A, None, 0, None) == b.E_SHAPE       # K beyond 16384
    assert f(A, b.BF16, A, 1e-6, 4, 24, A, A, None, 0, None) == b.E_SHAPE          # K % 16
    assert f(A, b.BF16, A, 1e-6, 4, 144, A, A, None, b.A_PACKED, None) == b.E_SHAPE  # K % 128 when packed
    assert f(A, b.BF16, A, -1.0, 4, 128, A, A, None, 0, None) == b.E_SHAPE         # eps < 0
    assert f(A, b.BF16, A, float("inf"), 4, 128, A, A, None, 0, None) == b.E_SHAPE
    assert f(A, b.BF16, A, 1e-6, 4, 0, A, A, None, 0, None) == b.E_SHAPE           # empty rows
    assert f(A, b.BF16, None, 1e-6, 4, 128, A, A, None, 0, None) == b.E_NULL
    assert f(A, b.BF16, A, 1e-6, 4, 128, A, A, A + 4, 0, None) == b.E_ALIGN
    assert f(None, b.BF16, None, 1e-6, 0, 128, None, None, None, 0, None) == b.OK


def test_noalloc_gemm_validation(lib):
    """fp8_scaled_gemm_noalloc: the fp8_scaled_gemm checks, and a call whose
    workspace would exceed the static scratch is refused before any HIP call."""
    g = lib.fp8_scaled_gemm_noalloc
    cap = b.SCRATCH_BYTES
    # bf16 per-token codes in the fragment order (rows padded to 16) + the scales: 4080 rows fit, 4081 do not
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 4080, 8, 4096) <= cap
    assert lib.fp8_scaled_gemm_workspace_size(b.BF16, b.SCALE_PER_TOKEN, 4081, 8, 4096) > cap
    assert g(A, b.BF16, None, b.SCALE_PER_TOKEN, A, 0, A, A, b.BF16, 4081, 8, 4096, b.ACCUM_EXACT,
             None) == b.E_SCRATCH
    assert g(A, b.F32, A, b.SCALE_PER_TENSOR, A, 0, A, A, b.BF16, 8193, 8, 2048, b.ACCUM_EXACT,
             None) == b.E_SCRATCH
    assert g(A, b.BF16, None, b.SCALE_PER_TOKEN, A, 0, A, A, b.E4M3, 4, 8, 128, b.ACCUM_EXACT, None) == b.E_DTYPE
    assert g(A, b.BF16, None, b.SCALE_PER_TOKEN, A, 0, A, A, b.BF16, 4, 8, 100, b.ACCUM_EXACT, None) == b.E_SHAPE
    assert g(A, b.BF16, None, b.SCALE_PER_TOKEN, None, 0, A, A, b.BF16, 4, 8, 128, b.ACCUM_EXACT,
             None) == b.E_NULL
    assert g(None, b.BF16, None, b.SCALE_PER_TOKEN, None, 0, A, A, b.BF16, 0, 8, 128, b.ACCUM_EXACT,
             None) == b.OK
    assert "scratch" in sg.status_string(b.E_SCRATCH)
