// Internal launchers (host side).  Each enqueues kernels on `stream` and returns
// hipGetLastError(); arguments are already validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8sg {

// What the GEMM kernels write: fp32, bf16, or E4M3 codes of the fp32 result
// under a given per-tensor output scale.
constexpr int kOutF32 = 0, kOutBF16 = 1, kOutE4M3 = 2;

// packed: write the codes in the GEMM fragment order (K % 128 == 0) instead of [M, K].
hipError_t launch_row_quant(const void* x, bool x_is_bf16, int64_t M, int64_t K, uint8_t* q, float* scales,
                            bool packed, hipStream_t stream);

// Per-token quantization of [M, K] straight into the fragment order (rows padded
// to 16), one workgroup per 16-row tile, for the K that row_quant_tiles_fit accepts.
bool row_quant_tiles_fit(bool x_is_bf16, int64_t K);
hipError_t launch_row_quant_tiles(const void* x, bool x_is_bf16, int64_t M, int64_t K, uint8_t* q, float* scales,
                                  hipStream_t stream);

// RMSNorm fused with per-token E4M3 quantization of its output (K <= 16384);
// gamma has x's dtype; y_out (optional) receives the fp32 normalised rows.
hipError_t launch_rmsnorm_quant(const void* x, bool x_is_bf16, const void* gamma, float eps, int64_t M, int64_t K,
                                uint8_t* q, float* scales, float* y_out, bool packed, hipStream_t stream);

// Block-wise dynamic quantization: activations in 1 x 128 groups (scales [M, K/128],
// or [K/128, M] with scales_kmajor), weights in 128 x 128 blocks (scales
// [ceil(N/128), K/128]); K % 128 == 0.
hipError_t launch_group_quant(const void* x, bool x_is_bf16, int64_t M, int64_t K, uint8_t* q, float* scales,
                              bool packed, bool scales_kmajor, hipStream_t stream);
hipError_t launch_block_quant_weight(const void* w, bool w_is_bf16, int64_t N, int64_t K, uint8_t* q, float* scales,
                                     hipStream_t stream);

// Static per-tensor E4M3 quantization of [M, K] (K % 128 == 0) into the fragment order.
hipError_t launch_static_quant_packed(const void* x, bool x_is_bf16, int64_t M, int64_t K, const float* scale,
                                      uint8_t* q, hipStream_t stream);

hipError_t launch_grouped_quant(const void* x, bool x_is_bf16, int64_t numel, const float* scales,
                                int64_t inner_units, int nscales, int fmt, uint8_t* q, hipStream_t stream);

hipError_t launch_gemm(const uint8_t* aq, bool a_packed, const float* a_scales, bool a_per_token, const uint8_t* wq,
                       bool w_packed, const float* w_scales, void* y, int out_kind, const float* out_scale, int64_t M,
                       int64_t N, int64_t K, bool fp8_mfma, hipStream_t stream);

// Decode GEMM with the per-token activation quantization inside the same
// kernel (bf16 X), for the shapes gemm_fused_quant_fits accepts.  sa_out may be NULL.
bool gemm_fused_quant_fits(bool x_is_bf16, int64_t M, int64_t K);
hipError_t launch_gemm_fused_quant(const uint16_t* x, float* sa_out, const uint8_t* wq, bool w_packed,
                                   const float* w_scales, void* y, int out_kind, const float* out_scale, int64_t M,
                                   int64_t N, int64_t K, bool fp8_mfma, hipStream_t stream);

// Block-wise scaled GEMM: a_scales [M, K/128] (or [K/128, M] with sa_kmajor),
// w_scales [ceil(N/128), K/128].
hipError_t launch_gemm_blockwise(const uint8_t* aq, bool a_packed, const float* a_scales, bool sa_kmajor,
                                 const uint8_t* wq, bool w_packed, const float* w_scales, void* y, bool y_bf16,
                                 int64_t M, int64_t N, int64_t K, bool fp8_mfma, hipStream_t stream);

// MXFP8: E8M0 scale bytes per 32 consecutive k (fmt 0 = E4M3, 1 = E5M2).  Scales
// row-major [R, K / 32] or in the GEMM's packed layout; codes row-major or in
// the fragment order; K % 32 == 0 (K % 128 == 0 for either packed form).
hipError_t launch_mx_quant(const void* x, bool x_is_bf16, int64_t R, int64_t K, int fmt, uint8_t* q,
                           bool packed_codes, uint8_t* scales, bool packed_scales, hipStream_t stream);
hipError_t launch_pack_mx_scales(const uint8_t* s, int64_t R, int64_t K, uint8_t* p, hipStream_t stream);
// MXFP8 GEMM: W E4M3, A E4M3 (a_fmt 0) or E5M2 (1), both scale arrays packed;
// out_kind kOutF32 or kOutBF16.
hipError_t launch_gemm_mx(const uint8_t* aq, bool a_packed, const uint8_t* a_scales, int a_fmt, const uint8_t* wq,
                          bool w_packed, const uint8_t* w_scales, void* y, int out_kind, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream);
// The same on bf16 activations X [M, K] (M <= 16), quantized to MX blocks of
// format a_fmt inside the kernel.
hipError_t launch_gemm_mx_bf16x(const uint16_t* x, int a_fmt, const uint8_t* wq, bool w_packed,
                                const uint8_t* w_scales, void* y, int out_kind, int64_t M, int64_t N, int64_t K,
                                hipStream_t stream);

hipError_t launch_pack_weights(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wp, hipStream_t stream);

hipError_t launch_kv_calibrate(const uint16_t* kv, int64_t B, int64_t S, int64_t H, int64_t D, int fmt,
                               float* head_scales, hipStream_t stream);

hipError_t launch_kv_dequant(const uint8_t* kvq, int64_t numel, int64_t H, int64_t D, const float* head_scales,
                             int fmt, uint16_t* out, hipStream_t stream);

hipError_t launch_kv_append(const uint16_t* kv_new, const int32_t* pos, int64_t B, int64_t S_cap, int64_t H,
                            int64_t D, const float* head_scales, int fmt, uint8_t* cache, hipStream_t stream);

// Decode attention over an FP8 KV cache (head dim 128; G = Hq / Hkv in {1, 2, 4, 8}).
size_t attn_workspace_bytes(int64_t B, int64_t S_cap, int64_t Hq, int64_t Hkv);
hipError_t launch_kv_decode_attention(const uint16_t* q, const uint8_t* kc, const uint8_t* vc, const float* k_scales,
                                      const float* v_scales, int fmt, const int32_t* lengths, int64_t B,
                                      int64_t S_cap, int64_t Hq, int64_t Hkv, float scale, void* out, bool out_bf16,
                                      float* part, hipStream_t stream);

}  // namespace fp8sg
