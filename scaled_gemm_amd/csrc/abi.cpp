// C-ABI entry points of libfp8sg: argument validation (always before any HIP
// call), device check, workspace layout and dispatch to the kernel launchers.
// The declarations, with the meaning, layout and ownership of every argument,
// are in include/fp8sg.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/fp8sg.h"
#include "launch.h"

namespace {

constexpr int kAbiVersion = 9;
constexpr int64_t kMaxDim = (int64_t)1 << 31;  // grid / int32 index limit per dimension
// The GEMM kernels keep per-lane operand offsets within a tile in 32 bits:
// rows x K bytes of a 256-row tile must stay below 2^32.
constexpr int64_t kMaxGemmK = (int64_t)1 << 24;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// 0 = unknown, 1 = gfx950, 2 = not usable.  One slot per device ordinal.
std::atomic<int> g_dev_state[64];

fp8sg_status device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return FP8SG_E_DEVICE;
    }
    if (dev >= 64) return FP8SG_E_DEVICE;
    int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return FP8SG_E_DEVICE;
        }
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? FP8SG_OK : FP8SG_E_DEVICE;
}

fp8sg_status launched(hipError_t e) { return e == hipSuccess ? FP8SG_OK : FP8SG_E_LAUNCH; }

bool is_hp(int dt) { return dt == FP8SG_F32 || dt == FP8SG_BF16; }
bool is_fp8(int dt) { return dt == FP8SG_E4M3 || dt == FP8SG_E5M2; }

// Row-wise dynamic quantization shared by the per-token and per-channel calls.
fp8sg_status row_quant(const void* x, int dt, int64_t R, int64_t K, uint8_t* q, float* scales, void* stream) {
    if (!is_hp(dt)) return FP8SG_E_DTYPE;
    if (R < 0 || K < 0 || R >= kMaxDim || K >= kMaxDim || (K % 16) != 0) return FP8SG_E_SHAPE;
    if (R == 0) return FP8SG_OK;
    if (!scales || (K > 0 && (!x || !q))) return FP8SG_E_NULL;
    if ((x && !aligned(x, 16)) || (q && !aligned(q, 16)) || !aligned(scales, 4)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    // K == 0 still writes the scales: the maximum of an empty row is 0, so s = 1.0
    return launched(fp8sg::launch_row_quant(x, dt == FP8SG_BF16, R, K, q, scales, false, (hipStream_t)stream));
}

// Common checks for the [B, S, H, D] KV calls.
fp8sg_status kv_shape(int64_t B, int64_t S, int64_t H, int64_t D, int fmt, int64_t* numel) {
    if (!is_fp8(fmt)) return FP8SG_E_DTYPE;
    if (B < 0 || S < 0 || H < 0 || D < 0) return FP8SG_E_SHAPE;
    if (B >= kMaxDim || S >= kMaxDim || H >= kMaxDim || D >= kMaxDim) return FP8SG_E_SHAPE;
    if (D % 16 != 0) return FP8SG_E_SHAPE;
    if (H > 4096) return FP8SG_E_SHAPE;
    __int128 n = (__int128)B * S * H * D;
    if (n >= ((__int128)1 << 62)) return FP8SG_E_SHAPE;
    *numel = (int64_t)n;
    return FP8SG_OK;
}

}  // namespace

extern "C" {

const char* fp8sg_status_string(int status) {
    switch (status) {
        case FP8SG_OK: return "ok";
        case FP8SG_E_NULL: return "required pointer is NULL";
        case FP8SG_E_SHAPE: return "invalid shape";
        case FP8SG_E_ALIGN: return "misaligned pointer";
        case FP8SG_E_DTYPE: return "unsupported dtype, format or mode";
        case FP8SG_E_DEVICE: return "no gfx950 HIP device";
        case FP8SG_E_LAUNCH: return "kernel launch failed";
        case FP8SG_E_WORKSPACE: return "workspace missing or too small";
        case FP8SG_E_SCRATCH: return "call needs more than the library's static scratch (FP8SG_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int fp8sg_version(void) { return kAbiVersion; }

fp8sg_status fp8_quant_per_token(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* q, float* scales,
                                 void* stream) {
    return row_quant(x, x_dtype, M, K, q, scales, stream);
}

fp8sg_status fp8_quant_weight_per_channel(const void* w, int w_dtype, int64_t N, int64_t K, uint8_t* wq,
                                          float* w_scales, void* stream) {
    return row_quant(w, w_dtype, N, K, wq, w_scales, stream);
}

fp8sg_status fp8_quant_per_tensor_static(const void* x, int x_dtype, int64_t numel, const float* scale, int fmt,
                                         uint8_t* q, void* stream) {
    if (!is_hp(x_dtype) || !is_fp8(fmt)) return FP8SG_E_DTYPE;
    if (numel < 0 || numel >= ((int64_t)1 << 62)) return FP8SG_E_SHAPE;
    if (numel == 0) return FP8SG_OK;
    if (!x || !scale || !q) return FP8SG_E_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    return launched(fp8sg::launch_grouped_quant(x, x_dtype == FP8SG_BF16, numel, scale, 1, 1,
                                                fmt == FP8SG_E4M3 ? 0 : 1, q, (hipStream_t)stream));
}

// Activation codes quantized by fp8_scaled_gemm itself go to the workspace,
// then the scales, in the fragment order (rows padded to 16) wherever a
// quantizer writes that order at full speed: decode-sized activations (M <= 32;
// the skinny kernel reads all of A in every workgroup), every per-tensor static
// scale (whole kilobytes of the order per wave), and per-token rows in 16-row
// tiles when a tile's rows fit in registers (bf16 K <= 8192, fp32 K <= 4096:
// 23 us against 20 us row-major for [4096, 8192], while the large-tile exact
// GEMM on packed A measured 2-6% faster at 4096 x 28672 x 8192).  Other
// per-token activations stay row-major.
constexpr int64_t kPackedAMaxM = 32;

bool quantized_a_packed(bool per_token, bool x_is_bf16, int64_t M, int64_t K) {
    return M <= kPackedAMaxM || !per_token || fp8sg::row_quant_tiles_fit(x_is_bf16, K);
}

size_t quantized_a_bytes(bool per_token, bool x_is_bf16, int64_t M, int64_t K) {
    const int64_t rows = quantized_a_packed(per_token, x_is_bf16, M, K) ? (M + 15) / 16 * 16 : M;
    return align256((size_t)rows * (size_t)K);
}

size_t fp8_scaled_gemm_workspace_size(int a_dtype, int a_scale_mode, int64_t M, int64_t N, int64_t K) {
    (void)N;
    if (!is_hp(a_dtype) || M <= 0 || K < 0) return 0;
    // decode-sized per-token activations are quantized inside the GEMM kernel itself
    if (a_scale_mode == FP8SG_SCALE_PER_TOKEN && fp8sg::gemm_fused_quant_fits(a_dtype == FP8SG_BF16, M, K)) return 0;
    const bool per_token = a_scale_mode == FP8SG_SCALE_PER_TOKEN;
    size_t bytes = quantized_a_bytes(per_token, a_dtype == FP8SG_BF16, M, K);
    if (per_token) bytes += align256((size_t)M * 4);
    return bytes;
}

size_t fp8_packed_weight_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return 0;
    return (size_t)((N + 15) / 16 * 16) * (size_t)K;
}

fp8sg_status fp8_pack_weights(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wp, void* stream) {
    if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim || K % 128 != 0) return FP8SG_E_SHAPE;
    if (N == 0 || K == 0) return FP8SG_OK;
    if (!wq || !wp) return FP8SG_E_NULL;
    if (!aligned(wq, 16) || !aligned(wp, 16)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    return launched(fp8sg::launch_pack_weights(wq, N, K, wp, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------------------
// Static scratch of fp8_scaled_gemm_noalloc: the activation codes and scales
// that fp8_scaled_gemm writes to its caller's workspace.  Every device the
// library runs on holds one copy until the process ends.  In host code the
// array's name is only a stand-in; the device address of each device's copy
// is looked up once (hipGetSymbolAddress, with that device current) and only
// that address is passed to kernels.
constexpr size_t kScratchBytes = (size_t)FP8SG_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[64];

// Device address of the current device's scratch, or NULL on failure.  Called
// after device_ok(), so the device index is valid.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        // the same address for every thread that looks it up, so a race only repeats the lookup
        g_scratch_ptr[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

// fp8_scaled_gemm, fp8_scaled_gemm_fp8out and fp8_scaled_gemm_noalloc:
// out_kind fp8sg::kOutF32 / kOutBF16 / kOutE4M3 (then out_scale [1] is the
// per-tensor output scale).  use_scratch: the workspace is the static scratch
// (workspace and workspace_bytes are ignored).
fp8sg_status scaled_gemm_impl(const void* a, int a_dtype, float* a_scales, int a_scale_mode, const uint8_t* wq,
                              int layout, const float* w_scales, void* y, int out_kind, const float* out_scale,
                              int64_t M, int64_t N, int64_t K, int accum, void* workspace, size_t workspace_bytes,
                              void* stream, bool use_scratch = false) {
    if (!(a_dtype == FP8SG_E4M3 || is_hp(a_dtype))) return FP8SG_E_DTYPE;
    if (!(a_scale_mode == FP8SG_SCALE_PER_TOKEN || a_scale_mode == FP8SG_SCALE_PER_TENSOR)) return FP8SG_E_DTYPE;
    if (!(accum == FP8SG_ACCUM_EXACT || accum == FP8SG_ACCUM_MFMA_FP8)) return FP8SG_E_DTYPE;
    if ((layout & ~(FP8SG_W_PACKED | FP8SG_A_PACKED)) != 0) return FP8SG_E_DTYPE;
    if ((layout & FP8SG_A_PACKED) && a_dtype != FP8SG_E4M3) return FP8SG_E_DTYPE;  // only codes come packed
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxGemmK) return FP8SG_E_SHAPE;
    if (K % 128 != 0) return FP8SG_E_SHAPE;
    if (M == 0 || N == 0) return FP8SG_OK;
    if (!y || !w_scales) return FP8SG_E_NULL;
    if (out_kind == fp8sg::kOutE4M3 && !out_scale) return FP8SG_E_NULL;
    if (K > 0 && (!a || !wq)) return FP8SG_E_NULL;
    const bool per_token = a_scale_mode == FP8SG_SCALE_PER_TOKEN;
    const bool quantize_here = is_hp(a_dtype);
    const bool pack_here = quantize_here && quantized_a_packed(per_token, a_dtype == FP8SG_BF16, M, K);
    if (!quantize_here || !per_token) {
        if (!a_scales) return FP8SG_E_NULL;  // an input in these modes
    }
    if ((a && !aligned(a, 16)) || (wq && !aligned(wq, 16)) || !aligned(y, 16)) return FP8SG_E_ALIGN;
    if ((a_scales && !aligned(a_scales, 4)) || !aligned(w_scales, 4)) return FP8SG_E_ALIGN;
    if (out_scale && !aligned(out_scale, 4)) return FP8SG_E_ALIGN;
    const size_t need = fp8_scaled_gemm_workspace_size(a_dtype, a_scale_mode, M, N, K);
    if (use_scratch) {
        if (need > kScratchBytes) return FP8SG_E_SCRATCH;
    } else if (need > 0) {
        if (!workspace || workspace_bytes < need) return FP8SG_E_WORKSPACE;
        if (!aligned(workspace, 256)) return FP8SG_E_ALIGN;
    }
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    if (use_scratch) {
        workspace = need > 0 ? scratch_on_current_device() : nullptr;
        if (need > 0 && workspace == nullptr) return FP8SG_E_DEVICE;
        workspace_bytes = need > 0 ? kScratchBytes : 0;
    }
    hipStream_t s = (hipStream_t)stream;

    if (quantize_here && per_token && fp8sg::gemm_fused_quant_fits(a_dtype == FP8SG_BF16, M, K)) {
        return launched(fp8sg::launch_gemm_fused_quant((const uint16_t*)a, a_scales, wq,
                                                       (layout & FP8SG_W_PACKED) != 0, w_scales, y, out_kind,
                                                       out_scale, M, N, K, accum == FP8SG_ACCUM_MFMA_FP8, s));
    }
    const uint8_t* aq = (const uint8_t*)a;
    const float* sa = a_scales;
    if (quantize_here) {
        uint8_t* ws_q = (uint8_t*)workspace;
        hipError_t e;
        if (per_token) {
            float* sc = a_scales ? a_scales
                                 : (float*)((uint8_t*)workspace + quantized_a_bytes(true, a_dtype == FP8SG_BF16, M, K));
            if (pack_here && M > kPackedAMaxM)
                e = fp8sg::launch_row_quant_tiles(a, a_dtype == FP8SG_BF16, M, K, ws_q, sc, s);
            else
                e = fp8sg::launch_row_quant(a, a_dtype == FP8SG_BF16, M, K, ws_q, sc, pack_here, s);
            sa = sc;
        } else if (pack_here) {
            e = fp8sg::launch_static_quant_packed(a, a_dtype == FP8SG_BF16, M, K, a_scales, ws_q, s);
        } else {
            e = fp8sg::launch_grouped_quant(a, a_dtype == FP8SG_BF16, M * K, a_scales, 1, 1, 0, ws_q, s);
        }
        if (e != hipSuccess) return FP8SG_E_LAUNCH;
        aq = ws_q;
    }
    const bool a_packed = quantize_here ? pack_here : (layout & FP8SG_A_PACKED) != 0;
    return launched(fp8sg::launch_gemm(aq, a_packed, sa, per_token, wq, (layout & FP8SG_W_PACKED) != 0, w_scales, y,
                                       out_kind, out_scale, M, N, K, accum == FP8SG_ACCUM_MFMA_FP8, s));
}

}  // namespace

extern "C" {

fp8sg_status fp8_scaled_gemm_noalloc(const void* a, int a_dtype, float* a_scales, int a_scale_mode,
                                     const uint8_t* wq, int layout, const float* w_scales, void* y, int y_dtype,
                                     int64_t M, int64_t N, int64_t K, int accum, void* stream) {
    if (!(y_dtype == FP8SG_BF16 || y_dtype == FP8SG_F32)) return FP8SG_E_DTYPE;
    return scaled_gemm_impl(a, a_dtype, a_scales, a_scale_mode, wq, layout, w_scales, y,
                            y_dtype == FP8SG_BF16 ? fp8sg::kOutBF16 : fp8sg::kOutF32, nullptr, M, N, K, accum,
                            nullptr, 0, stream, true);
}

fp8sg_status fp8_scaled_gemm(const void* a, int a_dtype, float* a_scales, int a_scale_mode, const uint8_t* wq,
                             int layout, const float* w_scales, void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                             int accum, void* workspace, size_t workspace_bytes, void* stream) {
    if (!(y_dtype == FP8SG_BF16 || y_dtype == FP8SG_F32)) return FP8SG_E_DTYPE;
    return scaled_gemm_impl(a, a_dtype, a_scales, a_scale_mode, wq, layout, w_scales, y,
                            y_dtype == FP8SG_BF16 ? fp8sg::kOutBF16 : fp8sg::kOutF32, nullptr, M, N, K, accum,
                            workspace, workspace_bytes, stream);
}

fp8sg_status fp8_scaled_gemm_fp8out(const void* a, int a_dtype, float* a_scales, int a_scale_mode, const uint8_t* wq,
                                    int layout, const float* w_scales, const float* out_scale, uint8_t* y, int64_t M,
                                    int64_t N, int64_t K, int accum, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    return scaled_gemm_impl(a, a_dtype, a_scales, a_scale_mode, wq, layout, w_scales, y, fp8sg::kOutE4M3, out_scale, M,
                            N, K, accum, workspace, workspace_bytes, stream);
}

fp8sg_status fp8_quant_per_token_group(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* q, float* scales,
                                       int layout, void* stream) {
    if (!is_hp(x_dtype)) return FP8SG_E_DTYPE;
    if ((layout & ~(FP8SG_A_PACKED | FP8SG_SCALES_KMAJOR)) != 0) return FP8SG_E_DTYPE;
    if (M < 0 || K < 0 || M >= kMaxDim || K >= kMaxDim || K % 128 != 0) return FP8SG_E_SHAPE;
    if (M == 0 || K == 0) return FP8SG_OK;
    if (!x || !q || !scales) return FP8SG_E_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    return launched(fp8sg::launch_group_quant(x, x_dtype == FP8SG_BF16, M, K, q, scales,
                                              (layout & FP8SG_A_PACKED) != 0, (layout & FP8SG_SCALES_KMAJOR) != 0,
                                              (hipStream_t)stream));
}

fp8sg_status fp8_quant_weight_blockwise(const void* w, int w_dtype, int64_t N, int64_t K, uint8_t* wq,
                                        float* w_scales, void* stream) {
    if (!is_hp(w_dtype)) return FP8SG_E_DTYPE;
    if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim || K % 128 != 0) return FP8SG_E_SHAPE;
    if (N == 0 || K == 0) return FP8SG_OK;
    if ((N + 127) / 128 * (K / 128) >= kMaxDim) return FP8SG_E_SHAPE;  // one workgroup per block
    if (!w || !wq || !w_scales) return FP8SG_E_NULL;
    if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(w_scales, 4)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    return launched(fp8sg::launch_block_quant_weight(w, w_dtype == FP8SG_BF16, N, K, wq, w_scales,
                                                     (hipStream_t)stream));
}

fp8sg_status fp8_scaled_gemm_blockwise(const uint8_t* a_q, const float* a_scales, const uint8_t* wq, int layout,
                                       const float* w_scales, void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                       int accum, void* stream) {
    if (!(y_dtype == FP8SG_BF16 || y_dtype == FP8SG_F32)) return FP8SG_E_DTYPE;
    if (!(accum == FP8SG_ACCUM_EXACT || accum == FP8SG_ACCUM_MFMA_FP8)) return FP8SG_E_DTYPE;
    if ((layout & ~(FP8SG_W_PACKED | FP8SG_A_PACKED | FP8SG_SCALES_KMAJOR)) != 0) return FP8SG_E_DTYPE;
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxGemmK) return FP8SG_E_SHAPE;
    if (K % 128 != 0) return FP8SG_E_SHAPE;
    if (M == 0 || N == 0) return FP8SG_OK;
    if (!y) return FP8SG_E_NULL;
    if (K > 0 && (!a_q || !wq || !a_scales || !w_scales)) return FP8SG_E_NULL;
    if ((a_q && !aligned(a_q, 16)) || (wq && !aligned(wq, 16)) || !aligned(y, 16)) return FP8SG_E_ALIGN;
    if ((a_scales && !aligned(a_scales, 4)) || (w_scales && !aligned(w_scales, 4))) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    // K == 0 launches too: the kernels read no scale and write the empty sums (zeros)
    return launched(fp8sg::launch_gemm_blockwise(a_q, (layout & FP8SG_A_PACKED) != 0, a_scales,
                                                 (layout & FP8SG_SCALES_KMAJOR) != 0, wq,
                                                 (layout & FP8SG_W_PACKED) != 0, w_scales, y, y_dtype == FP8SG_BF16,
                                                 M, N, K, accum == FP8SG_ACCUM_MFMA_FP8, (hipStream_t)stream));
}

fp8sg_status fp8_rmsnorm_quant_per_token(const void* x, int x_dtype, const void* gamma, float eps, int64_t M,
                                         int64_t K, uint8_t* q, float* scales, float* y_out, int layout,
                                         void* stream) {
    if (!is_hp(x_dtype)) return FP8SG_E_DTYPE;
    if (layout != 0 && layout != FP8SG_A_PACKED) return FP8SG_E_DTYPE;
    if (M < 0 || K < 0 || M >= kMaxDim || K > 16384 || K % (layout ? 128 : 16) != 0) return FP8SG_E_SHAPE;
    if (!(eps >= 0.0f) || eps == __builtin_inff()) return FP8SG_E_SHAPE;
    if (M == 0) return FP8SG_OK;
    if (K == 0) return FP8SG_E_SHAPE;  // the mean of an empty row is undefined
    if (!x || !gamma || !q || !scales) return FP8SG_E_NULL;
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(q, 16) || !aligned(scales, 4)) return FP8SG_E_ALIGN;
    if (y_out && !aligned(y_out, 16)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    return launched(fp8sg::launch_rmsnorm_quant(x, x_dtype == FP8SG_BF16, gamma, eps, M, K, q, scales, y_out,
                                                layout == FP8SG_A_PACKED, (hipStream_t)stream));
}

size_t fp8_mx_packed_scale_bytes(int64_t rows, int64_t K) {
    if (rows <= 0 || K <= 0) return 0;
    return (size_t)((rows + 63) / 64) * 256 * (size_t)(K / 128);
}

fp8sg_status fp8_quant_mx(const void* x, int x_dtype, int64_t rows, int64_t K, int fmt, uint8_t* q,
                          uint8_t* scales, int layout, void* stream) {
    if (!is_hp(x_dtype) || !is_fp8(fmt)) return FP8SG_E_DTYPE;
    if ((layout & ~(FP8SG_A_PACKED | FP8SG_MX_SCALES_PACKED)) != 0) return FP8SG_E_DTYPE;
    if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim) return FP8SG_E_SHAPE;
    if (K % (layout != 0 ? 128 : 32) != 0) return FP8SG_E_SHAPE;
    if (rows * (K / 8) >= kMaxDim * 256) return FP8SG_E_SHAPE;  // one thread per 8 elements
    if (rows == 0 || K == 0) return FP8SG_OK;
    if (!x || !q || !scales) return FP8SG_E_NULL;
    if (!aligned(x, 16) || !aligned(q, 16)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    return launched(fp8sg::launch_mx_quant(x, x_dtype == FP8SG_BF16, rows, K, fmt == FP8SG_E4M3 ? 0 : 1, q,
                                           (layout & FP8SG_A_PACKED) != 0, scales,
                                           (layout & FP8SG_MX_SCALES_PACKED) != 0, (hipStream_t)stream));
}

fp8sg_status fp8_pack_mx_scales(const uint8_t* scales, int64_t rows, int64_t K, uint8_t* packed, void* stream) {
    if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim || K % 128 != 0) return FP8SG_E_SHAPE;
    if (rows == 0 || K == 0) return FP8SG_OK;
    if (fp8_mx_packed_scale_bytes(rows, K) / 256 >= (size_t)kMaxDim) return FP8SG_E_SHAPE;
    if (!scales || !packed) return FP8SG_E_NULL;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    return launched(fp8sg::launch_pack_mx_scales(scales, rows, K, packed, (hipStream_t)stream));
}

fp8sg_status fp8_scaled_gemm_mx(const uint8_t* a_q, const uint8_t* a_scales, int a_fmt, const uint8_t* wq,
                                const uint8_t* w_scales, int layout, void* y, int y_dtype, int64_t M, int64_t N,
                                int64_t K, void* stream) {
    if (!(y_dtype == FP8SG_BF16 || y_dtype == FP8SG_F32) || !is_fp8(a_fmt)) return FP8SG_E_DTYPE;
    if ((layout & ~(FP8SG_W_PACKED | FP8SG_A_PACKED)) != 0) return FP8SG_E_DTYPE;
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxGemmK) return FP8SG_E_SHAPE;
    if (K % 128 != 0) return FP8SG_E_SHAPE;
    if (M == 0 || N == 0) return FP8SG_OK;
    if (!y) return FP8SG_E_NULL;
    if (K > 0 && (!a_q || !wq || !a_scales || !w_scales)) return FP8SG_E_NULL;
    if ((a_q && !aligned(a_q, 16)) || (wq && !aligned(wq, 16)) || !aligned(y, 16)) return FP8SG_E_ALIGN;
    if ((a_scales && !aligned(a_scales, 4)) || (w_scales && !aligned(w_scales, 4))) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    // K == 0 launches too: the kernels read no operand and write the empty sums (zeros)
    return launched(fp8sg::launch_gemm_mx(a_q, (layout & FP8SG_A_PACKED) != 0, a_scales, a_fmt == FP8SG_E4M3 ? 0 : 1,
                                          wq, (layout & FP8SG_W_PACKED) != 0, w_scales, y,
                                          y_dtype == FP8SG_BF16 ? fp8sg::kOutBF16 : fp8sg::kOutF32, M, N, K,
                                          (hipStream_t)stream));
}

fp8sg_status fp8_scaled_gemm_mx_bf16(const uint16_t* x, int a_fmt, const uint8_t* wq, const uint8_t* w_scales,
                                     int layout, void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
    if (!(y_dtype == FP8SG_BF16 || y_dtype == FP8SG_F32) || !is_fp8(a_fmt)) return FP8SG_E_DTYPE;
    if ((layout & ~FP8SG_W_PACKED) != 0) return FP8SG_E_DTYPE;
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxGemmK) return FP8SG_E_SHAPE;
    if (K % 128 != 0 || M > 16) return FP8SG_E_SHAPE;
    if (M == 0 || N == 0) return FP8SG_OK;
    if (!y) return FP8SG_E_NULL;
    if (K > 0 && (!x || !wq || !w_scales)) return FP8SG_E_NULL;
    if ((x && !aligned(x, 16)) || (wq && !aligned(wq, 16)) || !aligned(y, 16)) return FP8SG_E_ALIGN;
    if (w_scales && !aligned(w_scales, 4)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    // K == 0 launches too: the kernel reads no operand and writes the empty sums (zeros)
    return launched(fp8sg::launch_gemm_mx_bf16x(x, a_fmt == FP8SG_E4M3 ? 0 : 1, wq, (layout & FP8SG_W_PACKED) != 0,
                                                w_scales, y, y_dtype == FP8SG_BF16 ? fp8sg::kOutBF16 : fp8sg::kOutF32,
                                                M, N, K, (hipStream_t)stream));
}

fp8sg_status fp8_kv_calibrate(const uint16_t* kv, int64_t B, int64_t S, int64_t H, int64_t D, int fmt,
                              float* head_scales, void* stream) {
    int64_t numel = 0;
    fp8sg_status st = kv_shape(B, S, H, D, fmt, &numel);
    if (st != FP8SG_OK) return st;
    if (H == 0) return FP8SG_OK;
    if (!head_scales || (numel > 0 && !kv)) return FP8SG_E_NULL;
    if ((kv && !aligned(kv, 16)) || !aligned(head_scales, 4)) return FP8SG_E_ALIGN;
    st = device_ok();
    if (st != FP8SG_OK) return st;
    return launched(fp8sg::launch_kv_calibrate(kv, B, S, H, D, fmt == FP8SG_E4M3 ? 0 : 1, head_scales,
                                               (hipStream_t)stream));
}

fp8sg_status fp8_kv_quant(const uint16_t* kv, int64_t B, int64_t S, int64_t H, int64_t D, const float* head_scales,
                          int fmt, uint8_t* out, void* stream) {
    int64_t numel = 0;
    fp8sg_status st = kv_shape(B, S, H, D, fmt, &numel);
    if (st != FP8SG_OK) return st;
    if (numel == 0) return FP8SG_OK;
    if (!kv || !head_scales || !out) return FP8SG_E_NULL;
    if (!aligned(kv, 16) || !aligned(out, 16) || !aligned(head_scales, 4)) return FP8SG_E_ALIGN;
    st = device_ok();
    if (st != FP8SG_OK) return st;
    return launched(fp8sg::launch_grouped_quant(kv, true, numel, head_scales, D / 16, (int)H,
                                                fmt == FP8SG_E4M3 ? 0 : 1, out, (hipStream_t)stream));
}

fp8sg_status fp8_kv_dequant(const uint8_t* kvq, int64_t B, int64_t S, int64_t H, int64_t D, const float* head_scales,
                            int fmt, uint16_t* out, void* stream) {
    int64_t numel = 0;
    fp8sg_status st = kv_shape(B, S, H, D, fmt, &numel);
    if (st != FP8SG_OK) return st;
    if (numel == 0) return FP8SG_OK;
    if (!kvq || !head_scales || !out) return FP8SG_E_NULL;
    if (!aligned(kvq, 16) || !aligned(out, 16) || !aligned(head_scales, 4)) return FP8SG_E_ALIGN;
    st = device_ok();
    if (st != FP8SG_OK) return st;
    return launched(fp8sg::launch_kv_dequant(kvq, numel, H, D, head_scales, fmt == FP8SG_E4M3 ? 0 : 1, out,
                                             (hipStream_t)stream));
}

fp8sg_status fp8_kv_append(const uint16_t* kv_new, const int32_t* pos, int64_t B, int64_t S_cap, int64_t H,
                           int64_t D, const float* head_scales, int fmt, uint8_t* cache, void* stream) {
    int64_t numel = 0;
    fp8sg_status st = kv_shape(B, S_cap, H, D, fmt, &numel);
    if (st != FP8SG_OK) return st;
    if (B == 0 || H == 0 || D == 0) return FP8SG_OK;
    if (!kv_new || !pos || !head_scales || (!cache && S_cap > 0)) return FP8SG_E_NULL;
    if (!aligned(kv_new, 16) || !aligned(pos, 4) || !aligned(head_scales, 4)) return FP8SG_E_ALIGN;
    if (cache && !aligned(cache, 16)) return FP8SG_E_ALIGN;
    if (S_cap == 0) return FP8SG_OK;  // no position is valid
    st = device_ok();
    if (st != FP8SG_OK) return st;
    return launched(fp8sg::launch_kv_append(kv_new, pos, B, S_cap, H, D, head_scales, fmt == FP8SG_E4M3 ? 0 : 1,
                                            cache, (hipStream_t)stream));
}

}  // extern "C"

namespace {
bool attn_shape_ok(int64_t B, int64_t S_cap, int64_t Hq, int64_t Hkv, int64_t D) {
    if (B < 0 || S_cap < 0 || Hq < 0 || Hkv <= 0 || D != 128) return false;
    if (B >= kMaxDim || S_cap > ((int64_t)1 << 20) || Hq >= 65536 || Hkv >= 65536) return false;  // chunk weights in LDS
    if (Hq % Hkv != 0) return false;
    const int64_t G = Hq / Hkv;
    if (Hq > 0 && !(G == 1 || G == 2 || G == 4 || G == 8)) return false;
    const __int128 cache = (__int128)B * S_cap * Hkv * D;
    const __int128 grid = (__int128)B * Hkv * ((S_cap + 1023) / 1024);
    return cache < ((__int128)1 << 62) && grid < kMaxDim && (__int128)B * Hq < kMaxDim;
}
}  // namespace

extern "C" {

size_t fp8_kv_decode_attention_workspace_size(int64_t B, int64_t S_cap, int64_t Hq, int64_t Hkv, int64_t D) {
    if (!attn_shape_ok(B, S_cap, Hq, Hkv, D) || B == 0 || Hq == 0) return 0;
    return fp8sg::attn_workspace_bytes(B, S_cap, Hq, Hkv);
}

fp8sg_status fp8_kv_decode_attention(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                     const float* k_scales, const float* v_scales, int fmt, const int32_t* lengths,
                                     int64_t B, int64_t S_cap, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                                     void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    if (!is_fp8(fmt)) return FP8SG_E_DTYPE;
    if (!(out_dtype == FP8SG_BF16 || out_dtype == FP8SG_F32)) return FP8SG_E_DTYPE;
    if (!attn_shape_ok(B, S_cap, Hq, Hkv, D)) return FP8SG_E_SHAPE;
    if (!(scale == scale) || scale == __builtin_inff()) return FP8SG_E_SHAPE;  // NaN or +inf softmax scale
    if (B == 0 || Hq == 0) return FP8SG_OK;
    if (!q || !k_scales || !v_scales || !lengths || !out) return FP8SG_E_NULL;
    if (S_cap > 0 && (!k_cache || !v_cache)) return FP8SG_E_NULL;
    if (!aligned(q, 16) || !aligned(out, 16) || (k_cache && !aligned(k_cache, 16)) ||
        (v_cache && !aligned(v_cache, 16)) || !aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(lengths, 4))
        return FP8SG_E_ALIGN;
    const size_t need = fp8_kv_decode_attention_workspace_size(B, S_cap, Hq, Hkv, D);
    if (!workspace || workspace_bytes < need) return FP8SG_E_WORKSPACE;
    if (!aligned(workspace, 16)) return FP8SG_E_ALIGN;
    fp8sg_status d = device_ok();
    if (d != FP8SG_OK) return d;
    const float sc = scale > 0.0f ? scale : 1.0f / __builtin_sqrtf((float)D);
    return launched(fp8sg::launch_kv_decode_attention(q, k_cache, v_cache, k_scales, v_scales,
                                                      fmt == FP8SG_E4M3 ? 0 : 1, lengths, B, S_cap, Hq, Hkv, sc, out,
                                                      out_dtype == FP8SG_BF16, (float*)workspace,
                                                      (hipStream_t)stream));
}

}  // extern "C"
