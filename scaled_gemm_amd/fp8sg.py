"""Thin Python binding of libfp8sg (include/fp8sg.h) for torch tensors.

Argument marshalling only: each function checks devices, dtypes and
contiguity, allocates outputs with torch when the caller does not pass them,
and calls the C entry point of the same name on the current HIP stream.  All
arithmetic happens in the library's HIP kernels.  If the library is not built
the import of a function fails loudly (there is no fallback path).

FP8 codes travel as torch.uint8 tensors; bf16 data as torch.bfloat16.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libfp8sg.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fp8sg.h")

# enums of include/fp8sg.h
OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_DEVICE, E_LAUNCH, E_WORKSPACE, E_SCRATCH = range(9)
SCRATCH_BYTES = 16 << 20  # FP8SG_SCRATCH_BYTES
F32, BF16, E4M3, E5M2 = 0, 1, 2, 3
SCALE_PER_TOKEN, SCALE_PER_TENSOR = 0, 1
W_ROW_MAJOR, W_PACKED, A_PACKED, MX_SCALES_PACKED, SCALES_KMAJOR = 0, 1, 2, 4, 8
ACCUM_EXACT, ACCUM_MFMA_FP8 = 0, 1

_FMT = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2}
_ACCUM = {"exact": ACCUM_EXACT, "mfma_fp8": ACCUM_MFMA_FP8, ACCUM_EXACT: ACCUM_EXACT,
          ACCUM_MFMA_FP8: ACCUM_MFMA_FP8}
_LAYOUT = {"row_major": W_ROW_MAJOR, "packed": W_PACKED, W_ROW_MAJOR: W_ROW_MAJOR, W_PACKED: W_PACKED}
_SCALE = {"per_token": SCALE_PER_TOKEN, "per_tensor": SCALE_PER_TENSOR, SCALE_PER_TOKEN: SCALE_PER_TOKEN,
          SCALE_PER_TENSOR: SCALE_PER_TENSOR}


class Fp8sgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t

_SIGS = {
    "fp8sg_status_string": (ctypes.c_char_p, [_i32]),
    "fp8sg_version": (_i32, []),
    "fp8_quant_per_token": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _vp]),
    "fp8_quant_per_tensor_static": (_i32, [_vp, _i32, _i64, _vp, _i32, _vp, _vp]),
    "fp8_quant_weight_per_channel": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _vp]),
    "fp8_scaled_gemm_workspace_size": (_sz, [_i32, _i32, _i64, _i64, _i64]),
    "fp8_packed_weight_bytes": (_sz, [_i64, _i64]),
    "fp8_pack_weights": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm": (_i32, [_vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _sz,
                               _vp]),
    "fp8_scaled_gemm_noalloc": (_i32, [_vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _i64, _i32,
                                       _vp]),
    "fp8_scaled_gemm_fp8out": (_i32, [_vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp,
                                      _sz, _vp]),
    "fp8_quant_per_token_group": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _i32, _vp]),
    "fp8_quant_weight_blockwise": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _vp]),
    "fp8_scaled_gemm_blockwise": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp]),
    "fp8_rmsnorm_quant_per_token": (_i32, [_vp, _i32, _vp, ctypes.c_float, _i64, _i64, _vp, _vp, _vp, _i32, _vp]),
    "fp8_mx_packed_scale_bytes": (_sz, [_i64, _i64]),
    "fp8_quant_mx": (_i32, [_vp, _i32, _i64, _i64, _i32, _vp, _vp, _i32, _vp]),
    "fp8_pack_mx_scales": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_mx": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp]),
    "fp8_scaled_gemm_mx_bf16": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp]),
    "fp8_kv_decode_attention_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "fp8_kv_decode_attention": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _i64, _i64,
                                       ctypes.c_float, _vp, _i32, _vp, _sz, _vp]),
    "fp8_kv_calibrate": (_i32, [_vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp]),
    "fp8_kv_quant": (_i32, [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp]),
    "fp8_kv_dequant": (_i32, [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp]),
    "fp8_kv_append": (_i32, [_vp, _vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp]),
}


def lib():
    """The loaded library with argument types set; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libfp8sg is not built ({LIB_PATH} missing): run `python -m scaled_gemm_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def declared_symbols(header: str = HEADER_PATH):
    """Function names declared in include/fp8sg.h."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8\w*)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().fp8sg_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise Fp8sgError(status, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _hp_code(t: torch.Tensor) -> int:
    return BF16 if t.dtype == torch.bfloat16 else F32


_HP = (torch.float32, torch.bfloat16)


def fp8_quant_per_token(x: torch.Tensor, q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """x [M, K] (bf16/fp32) -> (q [M, K] uint8 E4M3, scales [M] fp32)."""
    _need(x, "x", _HP)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if q is None else q
    scales = torch.empty((M,), dtype=torch.float32, device=x.device) if scales is None else scales
    _need(q, "q", (torch.uint8,), (M, K))
    _need(scales, "scales", (torch.float32,), (M,))
    _check(lib().fp8_quant_per_token(_ptr(x), _hp_code(x), M, K, _ptr(q), _ptr(scales), _stream(stream)),
           "fp8_quant_per_token")
    return q, scales


def fp8_quant_weight_per_channel(w: torch.Tensor, wq: Optional[torch.Tensor] = None,
                                 w_scales: Optional[torch.Tensor] = None, stream=None):
    """w [N, K] (fp32/bf16) -> (wq [N, K] uint8 E4M3, w_scales [N] fp32)."""
    _need(w, "w", _HP)
    N, K = w.shape
    wq = torch.empty((N, K), dtype=torch.uint8, device=w.device) if wq is None else wq
    w_scales = torch.empty((N,), dtype=torch.float32, device=w.device) if w_scales is None else w_scales
    _need(wq, "wq", (torch.uint8,), (N, K))
    _need(w_scales, "w_scales", (torch.float32,), (N,))
    _check(lib().fp8_quant_weight_per_channel(_ptr(w), _hp_code(w), N, K, _ptr(wq), _ptr(w_scales),
                                              _stream(stream)), "fp8_quant_weight_per_channel")
    return wq, w_scales


def fp8_quant_per_tensor_static(x: torch.Tensor, scale: torch.Tensor, fmt="e4m3", q: Optional[torch.Tensor] = None,
                                stream=None) -> torch.Tensor:
    """x (bf16/fp32, any shape) with a device scale [1] -> codes uint8 of x's shape."""
    _need(x, "x", _HP)
    _need(scale, "scale", (torch.float32,), (1,))
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    _need(q, "q", (torch.uint8,), tuple(x.shape))
    _check(lib().fp8_quant_per_tensor_static(_ptr(x), _hp_code(x), x.numel(), _ptr(scale), _FMT[fmt], _ptr(q),
                                             _stream(stream)), "fp8_quant_per_tensor_static")
    return q


def fp8_packed_weight_bytes(N: int, K: int) -> int:
    return int(lib().fp8_packed_weight_bytes(N, K))


def fp8_pack_weights(wq: torch.Tensor, wp: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Row-major E4M3 codes [N, K] -> the packed fragment-order buffer (uint8, 1-D)."""
    _need(wq, "wq", (torch.uint8,))
    N, K = wq.shape
    nbytes = fp8_packed_weight_bytes(N, K)
    wp = torch.empty(nbytes, dtype=torch.uint8, device=wq.device) if wp is None else wp
    _need(wp, "wp", (torch.uint8,), (nbytes,))
    _check(lib().fp8_pack_weights(_ptr(wq), N, K, _ptr(wp), _stream(stream)), "fp8_pack_weights")
    return wp


def fp8_scaled_gemm_workspace_size(a_dtype, a_scale_mode, M: int, N: int, K: int) -> int:
    code = {torch.uint8: E4M3, torch.bfloat16: BF16, torch.float32: F32}.get(a_dtype, a_dtype)
    return int(lib().fp8_scaled_gemm_workspace_size(code, _SCALE[a_scale_mode], M, N, K))


def fp8_scaled_gemm(a: torch.Tensor, a_scales: Optional[torch.Tensor], wq: torch.Tensor, w_scales: torch.Tensor,
                    **kw) -> torch.Tensor:
    """Y [M, N] = diag(s_a) (A_q W_q^T) diag(s_w).

    a: uint8 E4M3 codes [M, K] (a_scales is then an input), or bf16/fp32
    activations that the call quantizes first (per token: a_scales, if given,
    receives the computed scales; per tensor: a_scales [1] is the given scale).
    a_layout="packed": a is the 1-D fragment-order buffer of fp8_pack_weights
    applied to the [M, K] codes, and a_shape=(M, K) gives the shape.
    wq: [N, K] row-major codes, or (w_layout="packed") the 1-D buffer of
    fp8_pack_weights; N is taken from w_scales.  Keywords: a_scale_mode,
    out_dtype, accum, w_layout, a_layout, a_shape, y, workspace, stream.
    """
    return _scaled_gemm(a, a_scales, wq, w_scales, **kw)


def _scaled_gemm(a: torch.Tensor, a_scales: Optional[torch.Tensor], wq: torch.Tensor, w_scales: torch.Tensor, *,
                 a_scale_mode="per_token", out_dtype=torch.bfloat16, accum="exact", w_layout="row_major",
                 a_layout="row_major", a_shape: Optional[tuple] = None, y: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, out_scale: Optional[torch.Tensor] = None,
                 noalloc: bool = False, stream=None) -> torch.Tensor:
    """Shared body of fp8_scaled_gemm and fp8_scaled_gemm_fp8out (out_scale given)."""
    _need(a, "a", (torch.uint8, torch.bfloat16, torch.float32))
    _need(wq, "wq", (torch.uint8,))
    _need(w_scales, "w_scales", (torch.float32,))
    a_packed = _LAYOUT[a_layout] == W_PACKED
    if a_packed:
        if a.dtype != torch.uint8 or a_shape is None:
            raise ValueError("a_layout='packed' takes E4M3 codes and a_shape=(M, K)")
        M, K = (int(v) for v in a_shape)
        if a.numel() != fp8_packed_weight_bytes(M, K):
            raise ValueError(f"packed a has {a.numel()} bytes, expected {fp8_packed_weight_bytes(M, K)}")
    else:
        M, K = a.shape
    N = w_scales.shape[0]
    layout = _LAYOUT[w_layout] | (A_PACKED if a_packed else 0)
    if _LAYOUT[w_layout] == W_ROW_MAJOR:
        if tuple(wq.shape) != (N, K):
            raise ValueError(f"wq has shape {tuple(wq.shape)}, expected {(N, K)}")
    elif wq.numel() != fp8_packed_weight_bytes(N, K):
        raise ValueError(f"packed wq has {wq.numel()} bytes, expected {fp8_packed_weight_bytes(N, K)}")
    mode = _SCALE[a_scale_mode]
    if a_scales is not None:
        _need(a_scales, "a_scales", (torch.float32,), (M,) if mode == SCALE_PER_TOKEN else (1,))
    a_code = {torch.uint8: E4M3, torch.bfloat16: BF16, torch.float32: F32}[a.dtype]
    if out_scale is not None:
        out_dtype = torch.uint8
    y_code = {torch.bfloat16: BF16, torch.float32: F32, torch.uint8: E4M3}[out_dtype]
    y = torch.empty((M, N), dtype=out_dtype, device=a.device) if y is None else y
    _need(y, "y", (out_dtype,), (M, N))
    if noalloc:
        _check(lib().fp8_scaled_gemm_noalloc(_ptr(a), a_code, _ptr(a_scales), mode, _ptr(wq), layout,
                                             _ptr(w_scales), _ptr(y), y_code, M, N, K, _ACCUM[accum],
                                             _stream(stream)), "fp8_scaled_gemm_noalloc")
        return y
    need = int(lib().fp8_scaled_gemm_workspace_size(a_code, mode, M, N, K))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out_scale is not None:
        _need(out_scale, "out_scale", (torch.float32,), (1,))
        _check(lib().fp8_scaled_gemm_fp8out(_ptr(a), a_code, _ptr(a_scales), mode, _ptr(wq), layout, _ptr(w_scales),
                                            _ptr(out_scale), _ptr(y), M, N, K, _ACCUM[accum], _ptr(workspace),
                                            ws_bytes, _stream(stream)), "fp8_scaled_gemm_fp8out")
        return y
    _check(lib().fp8_scaled_gemm(_ptr(a), a_code, _ptr(a_scales), mode, _ptr(wq), layout, _ptr(w_scales), _ptr(y),
                                 y_code, M, N, K, _ACCUM[accum], _ptr(workspace), ws_bytes, _stream(stream)),
           "fp8_scaled_gemm")
    return y


def fp8_scaled_gemm_noalloc(a: torch.Tensor, a_scales: Optional[torch.Tensor], wq: torch.Tensor,
                            w_scales: torch.Tensor, **kw) -> torch.Tensor:
    """fp8_scaled_gemm with the library's static device scratch in place of a
    workspace (the C call allocates nothing; pass y to allocate nothing here
    either).  Keywords as for fp8_scaled_gemm, without workspace."""
    if "workspace" in kw:
        raise TypeError("fp8_scaled_gemm_noalloc takes no workspace")
    return _scaled_gemm(a, a_scales, wq, w_scales, noalloc=True, **kw)


def fp8_scaled_gemm_fp8out(a: torch.Tensor, a_scales: Optional[torch.Tensor], wq: torch.Tensor,
                           w_scales: torch.Tensor, out_scale: torch.Tensor, **kw) -> torch.Tensor:
    """fp8_scaled_gemm with E4M3 output codes [M, N] (uint8) under the per-tensor
    output scale out_scale [1]: code = E4M3(RN32(y32 / out_scale)), saturating."""
    return _scaled_gemm(a, a_scales, wq, w_scales, out_scale=out_scale, **kw)


def fp8_quant_per_token_group(x: torch.Tensor, layout="row_major", q: Optional[torch.Tensor] = None,
                              scales: Optional[torch.Tensor] = None, scale_layout="row_major", stream=None):
    """x [M, K] (bf16/fp32) -> (codes, scales [M, K / 128] fp32): one scale per
    token and 128-element group.  layout="packed": the codes in the fragment
    order (1-D, fp8_packed_weight_bytes(M, K) bytes).  scale_layout="kmajor":
    the scales as [K / 128, M]."""
    _need(x, "x", _HP)
    M, K = x.shape
    packed = _LAYOUT[layout] == W_PACKED
    kmajor = scale_layout == "kmajor"
    qshape = (fp8_packed_weight_bytes(M, K),) if packed else (M, K)
    sshape = (K // 128, M) if kmajor else (M, K // 128)
    q = torch.empty(qshape, dtype=torch.uint8, device=x.device) if q is None else q
    scales = torch.empty(sshape, dtype=torch.float32, device=x.device) if scales is None else scales
    _need(q, "q", (torch.uint8,), qshape)
    _need(scales, "scales", (torch.float32,), sshape)
    _check(lib().fp8_quant_per_token_group(_ptr(x), _hp_code(x), M, K, _ptr(q), _ptr(scales),
                                           (A_PACKED if packed else 0) | (SCALES_KMAJOR if kmajor else 0),
                                           _stream(stream)), "fp8_quant_per_token_group")
    return q, scales


def fp8_quant_weight_blockwise(w: torch.Tensor, wq: Optional[torch.Tensor] = None,
                               w_scales: Optional[torch.Tensor] = None, stream=None):
    """w [N, K] (fp32/bf16) -> (wq [N, K] uint8, w_scales [ceil(N/128), K/128] fp32)."""
    _need(w, "w", _HP)
    N, K = w.shape
    sshape = ((N + 127) // 128, K // 128)
    wq = torch.empty((N, K), dtype=torch.uint8, device=w.device) if wq is None else wq
    w_scales = torch.empty(sshape, dtype=torch.float32, device=w.device) if w_scales is None else w_scales
    _need(wq, "wq", (torch.uint8,), (N, K))
    _need(w_scales, "w_scales", (torch.float32,), sshape)
    _check(lib().fp8_quant_weight_blockwise(_ptr(w), _hp_code(w), N, K, _ptr(wq), _ptr(w_scales), _stream(stream)),
           "fp8_quant_weight_blockwise")
    return wq, w_scales


def fp8_scaled_gemm_blockwise(a: torch.Tensor, a_scales: torch.Tensor, wq: torch.Tensor, w_scales: torch.Tensor, *,
                              out_dtype=torch.bfloat16, accum="mfma_fp8", w_layout="row_major", a_layout="row_major",
                              a_shape: Optional[tuple] = None, w_shape: Optional[tuple] = None,
                              y: Optional[torch.Tensor] = None, a_scale_layout="row_major",
                              stream=None) -> torch.Tensor:
    """Y [M, N] = sum_g diag(s_a[:, g]) (A_q W_q^T)_g diag(s_w[n // 128, g]).

    a: E4M3 codes [M, K] (or the packed 1-D buffer with a_shape=(M, K));
    a_scales [M, K/128]; wq [N, K] (or packed with w_shape=(N, K));
    w_scales [ceil(N/128), K/128].  accum: "mfma_fp8" or "exact".
    a_scale_layout="kmajor": a_scales is [K/128, M]."""
    _need(a, "a", (torch.uint8,))
    _need(wq, "wq", (torch.uint8,))
    a_packed = _LAYOUT[a_layout] == W_PACKED
    w_packed = _LAYOUT[w_layout] == W_PACKED
    M, K = (int(v) for v in a_shape) if a_packed else a.shape
    N = int(w_shape[0]) if w_packed else wq.shape[0]
    if a_packed and a.numel() != fp8_packed_weight_bytes(M, K):
        raise ValueError(f"packed a has {a.numel()} bytes, expected {fp8_packed_weight_bytes(M, K)}")
    if w_packed and (w_shape is None or int(w_shape[1]) != K or wq.numel() != fp8_packed_weight_bytes(N, K)):
        raise ValueError("w_layout='packed' takes w_shape=(N, K) and fp8_packed_weight_bytes(N, K) bytes")
    if not w_packed and wq.shape[1] != K:
        raise ValueError(f"wq has shape {tuple(wq.shape)}, expected K = {K}")
    kmajor = a_scale_layout == "kmajor"
    _need(a_scales, "a_scales", (torch.float32,), (K // 128, M) if kmajor else (M, K // 128))
    _need(w_scales, "w_scales", (torch.float32,), ((N + 127) // 128, K // 128))
    y_code = {torch.bfloat16: BF16, torch.float32: F32}[out_dtype]
    y = torch.empty((M, N), dtype=out_dtype, device=a.device) if y is None else y
    _need(y, "y", (out_dtype,), (M, N))
    layout = (W_PACKED if w_packed else 0) | (A_PACKED if a_packed else 0) | (SCALES_KMAJOR if kmajor else 0)
    _check(lib().fp8_scaled_gemm_blockwise(_ptr(a), _ptr(a_scales), _ptr(wq), layout, _ptr(w_scales), _ptr(y), y_code,
                                           M, N, K, _ACCUM[accum], _stream(stream)), "fp8_scaled_gemm_blockwise")
    return y


def fp8_rmsnorm_quant_per_token(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, layout="row_major",
                                q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                                y_out: Optional[torch.Tensor] = None, stream=None):
    """RMSNorm(x) * gamma quantized per token in one pass: x [M, K] (bf16/fp32),
    gamma [K] (same dtype) -> (codes, scales [M] fp32).  layout="packed": the
    codes in the fragment order (1-D).  y_out: optional [M, K] fp32 tensor that
    receives the normalised rows."""
    _need(x, "x", _HP)
    M, K = x.shape
    _need(gamma, "gamma", (x.dtype,), (K,))
    packed = _LAYOUT[layout] == W_PACKED
    qshape = (fp8_packed_weight_bytes(M, K),) if packed else (M, K)
    q = torch.empty(qshape, dtype=torch.uint8, device=x.device) if q is None else q
    scales = torch.empty(M, dtype=torch.float32, device=x.device) if scales is None else scales
    _need(q, "q", (torch.uint8,), qshape)
    _need(scales, "scales", (torch.float32,), (M,))
    if y_out is not None:
        _need(y_out, "y_out", (torch.float32,), (M, K))
    _check(lib().fp8_rmsnorm_quant_per_token(_ptr(x), _hp_code(x), _ptr(gamma), float(eps), M, K, _ptr(q),
                                             _ptr(scales), _ptr(y_out), A_PACKED if packed else 0, _stream(stream)),
           "fp8_rmsnorm_quant_per_token")
    return q, scales


def fp8_mx_packed_scale_bytes(rows: int, K: int) -> int:
    return int(lib().fp8_mx_packed_scale_bytes(rows, K))


def fp8_quant_mx(x: torch.Tensor, fmt="e4m3", layout="row_major", scale_layout="row_major",
                 q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None, stream=None):
    """x [rows, K] (bf16/fp32) -> (codes, E8M0 scale bytes): one power-of-two
    scale per 32 consecutive k.  layout="packed": codes in the MX fragment
    order (1-D, fp8_packed_weight_bytes(rows, K) bytes); scale_layout="packed": the
    scales in the layout fp8_scaled_gemm_mx reads (1-D,
    fp8_mx_packed_scale_bytes(rows, K) bytes), else [rows, K / 32]."""
    _need(x, "x", _HP)
    R, K = x.shape
    pc = _LAYOUT[layout] == W_PACKED
    ps = _LAYOUT[scale_layout] == W_PACKED
    qshape = (fp8_packed_weight_bytes(R, K),) if pc else (R, K)
    sshape = (fp8_mx_packed_scale_bytes(R, K),) if ps else (R, K // 32)
    q = torch.empty(qshape, dtype=torch.uint8, device=x.device) if q is None else q
    scales = torch.empty(sshape, dtype=torch.uint8, device=x.device) if scales is None else scales
    _need(q, "q", (torch.uint8,), qshape)
    _need(scales, "scales", (torch.uint8,), sshape)
    flags = (A_PACKED if pc else 0) | (MX_SCALES_PACKED if ps else 0)
    _check(lib().fp8_quant_mx(_ptr(x), _hp_code(x), R, K, _FMT[fmt], _ptr(q), _ptr(scales), flags, _stream(stream)),
           "fp8_quant_mx")
    return q, scales


def fp8_pack_mx_scales(scales: torch.Tensor, packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Row-major E8M0 scales [rows, K / 32] -> the packed layout (1-D)."""
    _need(scales, "scales", (torch.uint8,))
    R, nb = scales.shape
    K = 32 * nb
    n = fp8_mx_packed_scale_bytes(R, K)
    packed = torch.empty((n,), dtype=torch.uint8, device=scales.device) if packed is None else packed
    _need(packed, "packed", (torch.uint8,), (n,))
    _check(lib().fp8_pack_mx_scales(_ptr(scales), R, K, _ptr(packed), _stream(stream)), "fp8_pack_mx_scales")
    return packed


def fp8_scaled_gemm_mx(a: torch.Tensor, a_scales: torch.Tensor, wq: torch.Tensor, w_scales: torch.Tensor, *,
                       a_fmt="e4m3", out_dtype=torch.bfloat16, w_layout="row_major", a_layout="row_major",
                       a_shape: Optional[tuple] = None, w_shape: Optional[tuple] = None,
                       y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y [M, N] = sum_b 2^(ka + kw) (A_q W_q^T)_b over the 32-deep blocks b.

    a: codes [M, K] of format a_fmt (or the MX-packed 1-D buffer of
    fp8_quant_mx with a_shape=(M, K)); wq: E4M3 [N, K] (or MX-packed with
    w_shape=(N, K));
    a_scales / w_scales: packed E8M0 scales (fp8_quant_mx with
    scale_layout="packed", or fp8_pack_mx_scales)."""
    _need(a, "a", (torch.uint8,))
    _need(wq, "wq", (torch.uint8,))
    a_packed = _LAYOUT[a_layout] == W_PACKED
    w_packed = _LAYOUT[w_layout] == W_PACKED
    M, K = (int(v) for v in a_shape) if a_packed else a.shape
    N = int(w_shape[0]) if w_packed else wq.shape[0]
    if a_packed and a.numel() != fp8_packed_weight_bytes(M, K):
        raise ValueError(f"packed a has {a.numel()} bytes, expected {fp8_packed_weight_bytes(M, K)}")
    if w_packed and (w_shape is None or int(w_shape[1]) != K or wq.numel() != fp8_packed_weight_bytes(N, K)):
        raise ValueError("w_layout='packed' takes w_shape=(N, K) and fp8_packed_weight_bytes(N, K) bytes")
    if not w_packed and wq.shape[1] != K:
        raise ValueError(f"wq has shape {tuple(wq.shape)}, expected K = {K}")
    _need(a_scales, "a_scales", (torch.uint8,), (fp8_mx_packed_scale_bytes(M, K),))
    _need(w_scales, "w_scales", (torch.uint8,), (fp8_mx_packed_scale_bytes(N, K),))
    y_code = {torch.bfloat16: BF16, torch.float32: F32}[out_dtype]
    y = torch.empty((M, N), dtype=out_dtype, device=a.device) if y is None else y
    _need(y, "y", (out_dtype,), (M, N))
    layout = (W_PACKED if w_packed else 0) | (A_PACKED if a_packed else 0)
    _check(lib().fp8_scaled_gemm_mx(_ptr(a), _ptr(a_scales), _FMT[a_fmt], _ptr(wq), _ptr(w_scales), layout, _ptr(y),
                                    y_code, M, N, K, _stream(stream)), "fp8_scaled_gemm_mx")
    return y


def fp8_scaled_gemm_mx_bf16(x: torch.Tensor, wq: torch.Tensor, w_scales: torch.Tensor, *, a_fmt="e4m3",
                            out_dtype=torch.bfloat16, w_layout="row_major", w_shape: Optional[tuple] = None,
                            y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The MX decode GEMM on bf16 x [M, K] (M <= 16): each 32-element block of x
    is quantized to format a_fmt inside the kernel (the codes and scales of
    fp8_quant_mx), then multiplied as fp8_scaled_gemm_mx does."""
    _need(x, "x", (torch.bfloat16,))
    _need(wq, "wq", (torch.uint8,))
    if x.dim() != 2:
        raise ValueError(f"x must be [M, K], got {tuple(x.shape)}")
    M, K = x.shape
    w_packed = _LAYOUT[w_layout] == W_PACKED
    N = int(w_shape[0]) if w_packed else wq.shape[0]
    if w_packed and (w_shape is None or int(w_shape[1]) != K or wq.numel() != fp8_packed_weight_bytes(N, K)):
        raise ValueError("w_layout='packed' takes w_shape=(N, K) and fp8_packed_weight_bytes(N, K) bytes")
    if not w_packed and wq.shape[1] != K:
        raise ValueError(f"wq has shape {tuple(wq.shape)}, expected K = {K}")
    _need(w_scales, "w_scales", (torch.uint8,), (fp8_mx_packed_scale_bytes(N, K),))
    y_code = {torch.bfloat16: BF16, torch.float32: F32}[out_dtype]
    y = torch.empty((M, N), dtype=out_dtype, device=x.device) if y is None else y
    _need(y, "y", (out_dtype,), (M, N))
    _check(lib().fp8_scaled_gemm_mx_bf16(_ptr(x), _FMT[a_fmt], _ptr(wq), _ptr(w_scales), W_PACKED if w_packed else 0,
                                         _ptr(y), y_code, M, N, K, _stream(stream)), "fp8_scaled_gemm_mx_bf16")
    return y


def _kv_dims(t: torch.Tensor):
    if t.dim() != 4:
        raise ValueError("KV tensors are [B, S, H, D]")
    return tuple(int(v) for v in t.shape)


def fp8_kv_calibrate(kv: torch.Tensor, fmt="e4m3", head_scales: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """kv [B, S, H, D] bf16 -> head_scales [H] fp32."""
    _need(kv, "kv", (torch.bfloat16,))
    B, S, H, D = _kv_dims(kv)
    head_scales = torch.empty((H,), dtype=torch.float32, device=kv.device) if head_scales is None else head_scales
    _need(head_scales, "head_scales", (torch.float32,), (H,))
    _check(lib().fp8_kv_calibrate(_ptr(kv), B, S, H, D, _FMT[fmt], _ptr(head_scales), _stream(stream)),
           "fp8_kv_calibrate")
    return head_scales


def fp8_kv_quant(kv: torch.Tensor, head_scales: torch.Tensor, fmt="e4m3", out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """kv [B, S, H, D] bf16 -> codes uint8 [B, S, H, D]."""
    _need(kv, "kv", (torch.bfloat16,))
    B, S, H, D = _kv_dims(kv)
    _need(head_scales, "head_scales", (torch.float32,), (H,))
    out = torch.empty(kv.shape, dtype=torch.uint8, device=kv.device) if out is None else out
    _need(out, "out", (torch.uint8,), tuple(kv.shape))
    _check(lib().fp8_kv_quant(_ptr(kv), B, S, H, D, _ptr(head_scales), _FMT[fmt], _ptr(out), _stream(stream)),
           "fp8_kv_quant")
    return out


def fp8_kv_dequant(kvq: torch.Tensor, head_scales: torch.Tensor, fmt="e4m3", out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """codes uint8 [B, S, H, D] -> bf16 [B, S, H, D]."""
    _need(kvq, "kvq", (torch.uint8,))
    B, S, H, D = _kv_dims(kvq)
    _need(head_scales, "head_scales", (torch.float32,), (H,))
    out = torch.empty(kvq.shape, dtype=torch.bfloat16, device=kvq.device) if out is None else out
    _need(out, "out", (torch.bfloat16,), tuple(kvq.shape))
    _check(lib().fp8_kv_dequant(_ptr(kvq), B, S, H, D, _ptr(head_scales), _FMT[fmt], _ptr(out), _stream(stream)),
           "fp8_kv_dequant")
    return out


def fp8_kv_append(kv_new: torch.Tensor, pos: torch.Tensor, head_scales: torch.Tensor, cache: torch.Tensor,
                  fmt="e4m3", stream=None) -> torch.Tensor:
    """kv_new [B, H, D] bf16, pos [B] int32, cache [B, S_cap, H, D] uint8 (updated in place)."""
    _need(kv_new, "kv_new", (torch.bfloat16,))
    _need(cache, "cache", (torch.uint8,))
    B, S_cap, H, D = _kv_dims(cache)
    if tuple(kv_new.shape) != (B, H, D):
        raise ValueError(f"kv_new has shape {tuple(kv_new.shape)}, expected {(B, H, D)}")
    _need(pos, "pos", (torch.int32,), (B,))
    _need(head_scales, "head_scales", (torch.float32,), (H,))
    _check(lib().fp8_kv_append(_ptr(kv_new), _ptr(pos), B, S_cap, H, D, _ptr(head_scales), _FMT[fmt], _ptr(cache),
                               _stream(stream)), "fp8_kv_append")
    return cache


def fp8_kv_decode_attention_workspace_size(B: int, S_cap: int, Hq: int, Hkv: int, D: int) -> int:
    return int(lib().fp8_kv_decode_attention_workspace_size(B, S_cap, Hq, Hkv, D))


def fp8_kv_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scales: torch.Tensor,
                            v_scales: torch.Tensor, lengths: torch.Tensor, fmt="e4m3", scale: Optional[float] = None,
                            out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q [B, Hq, D] bf16; caches [B, S_cap, Hkv, D] uint8 codes; per-head scales
    [Hkv] fp32; lengths [B] int32 -> out [B, Hq, D] (bf16 or fp32)."""
    _need(q, "q", (torch.bfloat16,))
    _need(k_cache, "k_cache", (torch.uint8,))
    B, S_cap, Hkv, D = _kv_dims(k_cache)
    _need(v_cache, "v_cache", (torch.uint8,), (B, S_cap, Hkv, D))
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != D:
        raise ValueError(f"q has shape {tuple(q.shape)}, expected (B, Hq, D) = ({B}, Hq, {D})")
    Hq = int(q.shape[1])
    _need(k_scales, "k_scales", (torch.float32,), (Hkv,))
    _need(v_scales, "v_scales", (torch.float32,), (Hkv,))
    _need(lengths, "lengths", (torch.int32,), (B,))
    o_code = {torch.bfloat16: BF16, torch.float32: F32}[out_dtype]
    out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device) if out is None else out
    _need(out, "out", (out_dtype,), (B, Hq, D))
    need = fp8_kv_decode_attention_workspace_size(B, S_cap, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().fp8_kv_decode_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
                                         _FMT[fmt], _ptr(lengths), B, S_cap, Hq, Hkv, D,
                                         0.0 if scale is None else float(scale), _ptr(out), o_code, _ptr(workspace),
                                         ws_bytes, _stream(stream)), "fp8_kv_decode_attention")
    return out
