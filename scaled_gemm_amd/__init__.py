"""scaled_gemm_amd: FP8 W8A8 scaled GEMM, FP8 quantizers and FP8 KV-cache passes
for AMD Instinct MI355X (gfx950), as hand-written HIP kernels behind a C ABI
(include/fp8sg.h, built into scaled_gemm_amd/lib/libfp8sg.so).

The Python functions here are the thin torch binding of that library.
"""

from .fp8sg import (  # noqa: F401
    ACCUM_EXACT,
    ACCUM_MFMA_FP8,
    BF16,
    E4M3,
    E5M2,
    F32,
    Fp8sgError,
    SCALE_PER_TENSOR,
    SCALE_PER_TOKEN,
    A_PACKED,
    MX_SCALES_PACKED,
    W_PACKED,
    W_ROW_MAJOR,
    declared_symbols,
    fp8_kv_append,
    fp8_kv_calibrate,
    fp8_kv_decode_attention,
    fp8_kv_decode_attention_workspace_size,
    fp8_kv_dequant,
    fp8_kv_quant,
    fp8_mx_packed_scale_bytes,
    fp8_pack_mx_scales,
    fp8_pack_weights,
    fp8_packed_weight_bytes,
    fp8_quant_mx,
    fp8_rmsnorm_quant_per_token,
    fp8_quant_per_tensor_static,
    fp8_quant_per_token_group,
    fp8_quant_weight_blockwise,
    fp8_quant_per_token,
    fp8_quant_weight_per_channel,
    fp8_scaled_gemm,
    fp8_scaled_gemm_blockwise,
    fp8_scaled_gemm_fp8out,
    fp8_scaled_gemm_mx,
    fp8_scaled_gemm_mx_bf16,
    fp8_scaled_gemm_noalloc,
    fp8_scaled_gemm_workspace_size,
    lib,
    status_string,
)
