// FP8 quantizer kernels for gfx950.
//
//  * row_quant: dynamic per-row scaling (per-token activations, per-output-
//    channel weights).  One workgroup per row; the row stays in registers
//    between the absolute-maximum reduction and the encode, so X is read from
//    HBM once (FP8 Inference Explained, in depth -- "Inside a quantized linear
//    layer": find each token's amax, divide, cast to E4M3).
//  * group_quant / block_quant_weight: the block-wise variant -- one dynamic
//    scale per token and 128-element group along k for activations, one per
//    128 x 128 block for weights (FP8 Quantization notebook -- "Granularity";
//    FP8 Inference Explained, in depth -- "Scales and their granularity").
//  * grouped_quant: given scales, one per group of `inner` consecutive
//    elements, cycling over `nscales` groups (static per-tensor: one group;
//    KV cache [B,S,H,D]: inner = D, nscales = H).  Saturating (Quantization: FP8
//    inference and KV-cache quantization -- "Dynamic scales or static scales").
//
// Memory access: 16-byte loads and stores, consecutive lanes on consecutive
// 16-byte chunks; both kernels are bound by HBM bandwidth.
#include "fp8_device.h"
#include "launch.h"

namespace fp8sg {

// ---------------------------------------------------------------------------
// Row-wise dynamic quantization.
// Byte offset of element (m, k) of an [M, K] operand in the matrix-core
// fragment order shared by both GEMM operands (K % 128 == 0): the 16-row x
// 128-k block (m / 16, k / 128) is 2048 contiguous bytes; byte j of its 128 k
// belongs to lane (m % 16) + 16 (j / 32), whose first 16 bytes (j % 32 < 16)
// sit at lane * 16 and second 16 bytes at 1024 + lane * 16.
__device__ __forceinline__ int64_t packed_offset(int64_t m, int64_t k, int64_t nkb) {
    const int j = (int)(k & 127);
    return (((m >> 4) * nkb + (k >> 7)) << 11) + ((j >> 4) & 1) * 1024 + (((m & 15) + 16 * (j >> 5)) << 4) + (j & 15);
}

// kChunks chunks per thread held in registers (row length <= kChunks * 8 * blockDim).
// kPacked: the codes go to the fragment order (packed_offset) instead of [M, K].
// kStream: X is read with streaming loads (chosen for large inputs, where it
// measured 3-7% faster; for decode-sized rows it measured slightly slower).
template <typename InT, int kChunks, bool kPacked, bool kStream>
__global__ __launch_bounds__(256) void row_quant_resident(const InT* __restrict__ x, int64_t K,
                                                          uint8_t* __restrict__ q, float* __restrict__ scales) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const InT* xr = x + row * K;
    uint8_t* qr = q + row * K;
    const int nchunks = (int)(K >> 3);
    const int T = blockDim.x;
    float v[kChunks][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int c = threadIdx.x + i * T;
        if (c < nchunks) {
            if (kStream) load_chunk_stream<InT>(xr + (int64_t)c * 8, v[i]);
            else load_chunk<InT>(xr + (int64_t)c * 8, v[i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(v[i][j]));
        }
    }
    amax = block_max(amax, red);
    const float s = dynamic_scale(amax, kE4M3Max);
    if (threadIdx.x == 0) scales[row] = s;
    const QScale p = make_qscale(s, kE4M3Max);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int c = threadIdx.x + i * T;
        if (c < nchunks) {
            uint8_t* dst = kPacked ? q + packed_offset(row, (int64_t)c * 8, K >> 7) : qr + (int64_t)c * 8;
            *reinterpret_cast<uint2*>(dst) = encode_chunk_dynamic<InT>(v[i], p);
        }
    }
}

// Rows too long for registers: the maximum pass and the encode pass each read the row.
template <typename InT, bool kPacked>
__global__ __launch_bounds__(256) void row_quant_stream(const InT* __restrict__ x, int64_t K,
                                                        uint8_t* __restrict__ q, float* __restrict__ scales) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const InT* xr = x + row * K;
    uint8_t* qr = q + row * K;
    const int64_t nchunks = K >> 3;
    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < nchunks; c += blockDim.x) {
        float v[8];
        load_chunk<InT>(xr + c * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j]));
    }
    amax = block_max(amax, red);
    const float s = dynamic_scale(amax, kE4M3Max);
    if (threadIdx.x == 0) scales[row] = s;
    const QScale p = make_qscale(s, kE4M3Max);
    for (int64_t c = threadIdx.x; c < nchunks; c += blockDim.x) {
        float v[8];
        load_chunk<InT>(xr + c * 8, v);
        uint8_t* dst = kPacked ? q + packed_offset(row, c * 8, K >> 7) : qr + c * 8;
        *reinterpret_cast<uint2*>(dst) = encode_chunk_dynamic<InT>(v, p);
    }
}

template <typename InT, bool kPacked>
static hipError_t launch_row_quant_t(const InT* x, int64_t M, int64_t K, uint8_t* q, float* scales,
                                     hipStream_t stream) {
    const int64_t nchunks = K / 8;
    const int T = 256;
    const int64_t per = (nchunks + T - 1) / T;
    dim3 grid((unsigned)M), block(T);
    const bool big = M * K * (int64_t)sizeof(InT) >= ((int64_t)16 << 20);
#define FP8SG_RQ(C)                                                                             \
    do {                                                                                        \
        if (big) row_quant_resident<InT, C, kPacked, true><<<grid, block, 0, stream>>>(x, K, q, scales);  \
        else row_quant_resident<InT, C, kPacked, false><<<grid, block, 0, stream>>>(x, K, q, scales);     \
    } while (0)
    if (per <= 1) FP8SG_RQ(1);
    else if (per <= 2) FP8SG_RQ(2);
    else if (per <= 4) FP8SG_RQ(4);
    else if (per <= 8) FP8SG_RQ(8);
    else row_quant_stream<InT, kPacked><<<grid, block, 0, stream>>>(x, K, q, scales);
#undef FP8SG_RQ
    return hipGetLastError();
}

hipError_t launch_row_quant(const void* x, bool x_is_bf16, int64_t M, int64_t K, uint8_t* q, float* scales,
                            bool packed, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    if (x_is_bf16)
        return packed ? launch_row_quant_t<uint16_t, true>((const uint16_t*)x, M, K, q, scales, stream)
                      : launch_row_quant_t<uint16_t, false>((const uint16_t*)x, M, K, q, scales, stream);
    return packed ? launch_row_quant_t<float, true>((const float*)x, M, K, q, scales, stream)
                  : launch_row_quant_t<float, false>((const float*)x, M, K, q, scales, stream);
}

// ---------------------------------------------------------------------------
// RMSNorm with the per-token quantization fused into it: the quantizer's
// maximum is taken over the normalised row while it is still in registers, so
// the bf16 normalised activations are never written and read back (the pages'
// engines fuse the amax reduction into the preceding kernel).
//   ss = sum_k x_k^2 (fp32 fused multiply-adds over each thread's chunks in
//   order, then the wave tree, then the four waves in a fixed order),
//   r = RN32(1 / RN32(sqrt(RN32(RN32(ss / K) + eps)))),
//   y_k = RN32(RN32(x_k * r) * g_k), then the dynamic per-token rule on y.
// y_out (optional) receives y in fp32.  One workgroup per row, the row in
// registers (K <= 16384), as in row_quant_resident.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    const float t = (red[0] + red[1]) + (red[2] + red[3]);   // 4 waves, fixed order
    __syncthreads();
    return t;
}

template <typename InT, int kChunks, bool kPacked>
__global__ __launch_bounds__(256) void rmsnorm_quant(const InT* __restrict__ x, const InT* __restrict__ gamma,
                                                     float eps, int64_t K, uint8_t* __restrict__ q,
                                                     float* __restrict__ scales, float* __restrict__ y_out) {
    __shared__ float red[4];
    const int t = (int)threadIdx.x;
    const int64_t row = blockIdx.x;
    const InT* xr = x + row * K;
    const int nchunks = (int)(K >> 3);
    float v[kChunks][8];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int c = t + i * 256;
        if (c < nchunks) {
            load_chunk<InT>(xr + (int64_t)c * 8, v[i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(v[i][j], v[i][j], ss);
        }
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / __builtin_sqrtf(ss / (float)K + eps);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int c = t + i * 256;
        if (c < nchunks) {
            float g[8];
            load_chunk<InT>(gamma + (int64_t)c * 8, g);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[i][j] = (v[i][j] * r) * g[j];
                amax = fmaxf(amax, __builtin_fabsf(v[i][j]));
            }
            if (y_out) {
                float4* yo = reinterpret_cast<float4*>(y_out + row * K + (int64_t)c * 8);
                yo[0] = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
                yo[1] = make_float4(v[i][4], v[i][5], v[i][6], v[i][7]);
            }
        }
    }
    amax = block_max(amax, red);
    const float s = dynamic_scale(amax, kE4M3Max);
    if (t == 0) scales[row] = s;
    const QScale p = make_qscale(s, kE4M3Max);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int c = t + i * 256;
        if (c < nchunks) {
            uint8_t* dst = kPacked ? q + packed_offset(row, (int64_t)c * 8, K >> 7) : q + row * K + (int64_t)c * 8;
            *reinterpret_cast<uint2*>(dst) = encode_chunk_dynamic<float>(v[i], p);
        }
    }
}

template <typename InT, bool kPacked>
static void launch_rmsnorm_quant_t(const InT* x, const InT* g, float eps, int64_t M, int64_t K, uint8_t* q,
                                   float* scales, float* y_out, hipStream_t stream) {
    const int64_t per = (K / 8 + 255) / 256;
    dim3 grid((unsigned)M), block(256);
    if (per <= 1) rmsnorm_quant<InT, 1, kPacked><<<grid, block, 0, stream>>>(x, g, eps, K, q, scales, y_out);
    else if (per <= 2) rmsnorm_quant<InT, 2, kPacked><<<grid, block, 0, stream>>>(x, g, eps, K, q, scales, y_out);
    else if (per <= 4) rmsnorm_quant<InT, 4, kPacked><<<grid, block, 0, stream>>>(x, g, eps, K, q, scales, y_out);
    else rmsnorm_quant<InT, 8, kPacked><<<grid, block, 0, stream>>>(x, g, eps, K, q, scales, y_out);
}

hipError_t launch_rmsnorm_quant(const void* x, bool x_is_bf16, const void* gamma, float eps, int64_t M, int64_t K,
                                uint8_t* q, float* scales, float* y_out, bool packed, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    if (x_is_bf16) {
        if (packed) launch_rmsnorm_quant_t<uint16_t, true>((const uint16_t*)x, (const uint16_t*)gamma, eps, M, K, q,
                                                           scales, y_out, stream);
        else launch_rmsnorm_quant_t<uint16_t, false>((const uint16_t*)x, (const uint16_t*)gamma, eps, M, K, q, scales,
                                                     y_out, stream);
    } else {
        if (packed) launch_rmsnorm_quant_t<float, true>((const float*)x, (const float*)gamma, eps, M, K, q, scales,
                                                        y_out, stream);
        else launch_rmsnorm_quant_t<float, false>((const float*)x, (const float*)gamma, eps, M, K, q, scales, y_out,
                                                  stream);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block-wise dynamic quantization.
//
// Activations, one scale per (row, 128-element group): a group is 16 chunks of
// 8 elements, one chunk per thread, so the 16 threads of a group take its
// maximum with four shuffles and each encodes its own chunk.  The grid strides
// over chunks in multiples of 16 and the chunk count is a multiple of 16
// (K % 128 == 0), so a group's 16 threads are always active together.
// scales[m * (K / 128) + g] = RN32(amax / 448) (1.0 for an all-zero group).
template <typename InT, bool kPacked>
__global__ __launch_bounds__(256) void group_quant(const InT* __restrict__ x, int64_t K, int64_t nchunks,
                                                   uint8_t* __restrict__ q, float* __restrict__ scales, int64_t M,
                                                   int kmajor) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
        float v[8];
        load_chunk<InT>(x + c * 8, v);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j]));
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        const float s = dynamic_scale(amax, kE4M3Max);
        if ((c & 15) == 0) {
            // group g = c / 16 is (row g / nkb, k block g % nkb): row-major [M, K/128] or k-block-major [K/128, M]
            const int64_t g = c >> 4, nkb = K >> 7;
            scales[kmajor ? (g % nkb) * M + g / nkb : g] = s;
        }
        const QScale p = make_qscale(s, kE4M3Max);
        uint8_t* dst;
        if (kPacked) {
            const int64_t e = c * 8, m = e / K;
            dst = q + packed_offset(m, e - m * K, K >> 7);
        } else {
            dst = q + c * 8;
        }
        *reinterpret_cast<uint2*>(dst) = encode_chunk_dynamic<InT>(v, p);
    }
}

hipError_t launch_group_quant(const void* x, bool x_is_bf16, int64_t M, int64_t K, uint8_t* q, float* scales,
                              bool packed, bool scales_kmajor, hipStream_t stream) {
    const int64_t nchunks = M * (K / 8);
    if (nchunks == 0) return hipSuccess;
    int64_t blocks = (nchunks + 255) / 256;
    if (blocks > 256 * 16) blocks = 256 * 16;
    dim3 grid((unsigned)blocks), block(256);
    const int km = scales_kmajor ? 1 : 0;
    if (x_is_bf16) {
        if (packed) group_quant<uint16_t, true><<<grid, block, 0, stream>>>((const uint16_t*)x, K, nchunks, q, scales, M, km);
        else group_quant<uint16_t, false><<<grid, block, 0, stream>>>((const uint16_t*)x, K, nchunks, q, scales, M, km);
    } else {
        if (packed) group_quant<float, true><<<grid, block, 0, stream>>>((const float*)x, K, nchunks, q, scales, M, km);
        else group_quant<float, false><<<grid, block, 0, stream>>>((const float*)x, K, nchunks, q, scales, M, km);
    }
    return hipGetLastError();
}

// Weights, one scale per 128 x 128 block (the last row block is short when
// N % 128 != 0).  One workgroup per block: thread t holds chunk t % 16 of rows
// t / 16 + 16 i, i < 8, in registers between the block maximum and the encode.
// scales[(n / 128) * (K / 128) + k / 128].
template <typename InT>
__global__ __launch_bounds__(256) void block_quant_weight(const InT* __restrict__ w, int64_t N, int64_t K, int nkb,
                                                          uint8_t* __restrict__ q, float* __restrict__ scales) {
    __shared__ float red[4];
    const int64_t blk = blockIdx.x;
    const int64_t nb = blk / nkb;
    const int64_t col = (blk - nb * nkb) * 128 + (threadIdx.x & 15) * 8;
    float v[8][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = nb * 128 + (threadIdx.x >> 4) + 16 * i;
        if (row < N) {
            load_chunk<InT>(w + row * K + col, v[i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(v[i][j]));
        }
    }
    amax = block_max(amax, red);
    const float s = dynamic_scale(amax, kE4M3Max);
    if (threadIdx.x == 0) scales[blk] = s;
    const QScale p = make_qscale(s, kE4M3Max);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = nb * 128 + (threadIdx.x >> 4) + 16 * i;
        if (row < N) *reinterpret_cast<uint2*>(q + row * K + col) = encode_chunk_dynamic<InT>(v[i], p);
    }
}

hipError_t launch_block_quant_weight(const void* w, bool w_is_bf16, int64_t N, int64_t K, uint8_t* q, float* scales,
                                     hipStream_t stream) {
    const int64_t nkb = K / 128, nbw = (N + 127) / 128;
    if (nkb == 0 || nbw == 0) return hipSuccess;
    dim3 grid((unsigned)(nkb * nbw)), block(256);
    if (w_is_bf16)
        block_quant_weight<uint16_t><<<grid, block, 0, stream>>>((const uint16_t*)w, N, K, (int)nkb, q, scales);
    else
        block_quant_weight<float><<<grid, block, 0, stream>>>((const float*)w, N, K, (int)nkb, q, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Given-scale quantization, one scale per group of `inner` elements cycling
// over `nscales` scales.  A unit is 16 consecutive elements -> 16 codes (one
// 16-byte store).  The caller passes inner_units = inner / 16 (inner is a
// multiple of 16 whenever nscales > 1), so a unit never straddles two scales;
// with nscales == 1 every unit uses scale 0.  When the grid stride is a
// multiple of the scale period (inner_units * nscales units) a thread's scale
// never changes and is looked up once.  A partial last unit (numel % 16) takes a
// per-element path.
constexpr int kMaxLdsScales = 256;

template <typename InT, int kFmt>
__device__ __forceinline__ uint4 encode16_given(const InT* p, const QScale& sc) {
    constexpr bool kTwo = sizeof(InT) == 4;
    float v[8], w[8];
    load_chunk<InT>(p, v);
    load_chunk<InT>(p + 8, w);
    // the scale's range test once for the 16 values
    auto enc = [&](auto fast_tag) __attribute__((always_inline)) {
        constexpr bool kF = decltype(fast_tag)::value;
        uint4 o;
        o.x = pack4<kFmt>(quotient_given_known<kTwo, kF>(v[0], sc), quotient_given_known<kTwo, kF>(v[1], sc),
                          quotient_given_known<kTwo, kF>(v[2], sc), quotient_given_known<kTwo, kF>(v[3], sc));
        o.y = pack4<kFmt>(quotient_given_known<kTwo, kF>(v[4], sc), quotient_given_known<kTwo, kF>(v[5], sc),
                          quotient_given_known<kTwo, kF>(v[6], sc), quotient_given_known<kTwo, kF>(v[7], sc));
        o.z = pack4<kFmt>(quotient_given_known<kTwo, kF>(w[0], sc), quotient_given_known<kTwo, kF>(w[1], sc),
                          quotient_given_known<kTwo, kF>(w[2], sc), quotient_given_known<kTwo, kF>(w[3], sc));
        o.w = pack4<kFmt>(quotient_given_known<kTwo, kF>(w[4], sc), quotient_given_known<kTwo, kF>(w[5], sc),
                          quotient_given_known<kTwo, kF>(w[6], sc), quotient_given_known<kTwo, kF>(w[7], sc));
        return o;
    };
    return sc.fast ? enc(std::true_type{}) : enc(std::false_type{});
}

template <typename InT, int kFmt>
__global__ __launch_bounds__(256) void grouped_quant(const InT* __restrict__ x, int64_t numel,
                                                     const float* __restrict__ scales, int64_t inner_units,
                                                     int nscales, uint8_t* __restrict__ q) {
    constexpr bool kTwo = sizeof(InT) == 4;
    constexpr float fmax = kFmt == 0 ? kE4M3Max : kE5M2Max;
    __shared__ QScale tab[kMaxLdsScales];
    const bool in_lds = nscales <= kMaxLdsScales;
    if (in_lds) {
        for (int i = threadIdx.x; i < nscales; i += blockDim.x) tab[i] = make_qscale(scales[i], fmax);
        __syncthreads();
    }
    const int64_t nfull = numel >> 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t period = inner_units * nscales;
    int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (stride % period == 0) {
        const int g = (int)((u / inner_units) % nscales);
        const QScale p = in_lds ? tab[g] : make_qscale(scales[g], fmax);
        for (; u < nfull; u += stride)
            *reinterpret_cast<uint4*>(q + (u << 4)) = encode16_given<InT, kFmt>(x + (u << 4), p);
    } else {
        for (; u < nfull; u += stride) {
            const int g = (int)((u / inner_units) % nscales);
            const QScale p = in_lds ? tab[g] : make_qscale(scales[g], fmax);
            *reinterpret_cast<uint4*>(q + (u << 4)) = encode16_given<InT, kFmt>(x + (u << 4), p);
        }
    }
    // tail: the last numel % 16 elements, one thread
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        for (int64_t e = nfull << 4; e < numel; ++e) {
            const int g = (int)(((e >> 4) / inner_units) % nscales);
            const QScale p = in_lds ? tab[g] : make_qscale(scales[g], fmax);
            float xv;
            if (sizeof(InT) == 2) xv = bf16_lo((uint32_t)((const uint16_t*)x)[e]);
            else xv = ((const float*)x)[e];
            q[e] = (uint8_t)(pack4<kFmt>(quotient_given<kTwo>(xv, p), 0.0f, 0.0f, 0.0f) & 0xFFu);
        }
    }
}

hipError_t launch_grouped_quant(const void* x, bool x_is_bf16, int64_t numel, const float* scales,
                                int64_t inner_units, int nscales, int fmt, uint8_t* q, hipStream_t stream) {
    if (numel == 0) return hipSuccess;
    const int64_t nunits = (numel + 15) / 16;
    const int T = 256;
    // At most four units per thread, and at least 16 workgroups per CU of work
    // when there is that much: for the KV cache (2^24 units) 16 per CU looping
    // gave 5.1 TB/s and four units per thread 5.6 TB/s; for a [4096, 8192]
    // activation (2^21 units) 16 workgroups per CU is the faster of the two.
    const int64_t full = (nunits + T - 1) / T;
    int64_t blocks = full < 256 * 16 ? full : 256 * 16;
    if (blocks < (full + 3) / 4) blocks = (full + 3) / 4;
    if (blocks > ((int64_t)1 << 31) - 1) blocks = ((int64_t)1 << 31) - 1;
    if (blocks < 1) blocks = 1;
    dim3 grid((unsigned)blocks), block(T);
    if (x_is_bf16) {
        if (fmt == 0) grouped_quant<uint16_t, 0><<<grid, block, 0, stream>>>((const uint16_t*)x, numel, scales, inner_units, nscales, q);
        else grouped_quant<uint16_t, 1><<<grid, block, 0, stream>>>((const uint16_t*)x, numel, scales, inner_units, nscales, q);
    } else {
        if (fmt == 0) grouped_quant<float, 0><<<grid, block, 0, stream>>>((const float*)x, numel, scales, inner_units, nscales, q);
        else grouped_quant<float, 1><<<grid, block, 0, stream>>>((const float*)x, numel, scales, inner_units, nscales, q);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static per-tensor quantization of [M, K] activations (K % 128 == 0) straight
// into the fragment order: one 16-element unit per thread and grid step; the
// unit's 16 codes are one 16-byte half of one lane (packed_offset).
template <typename InT>
__global__ __launch_bounds__(256) void static_quant_packed(const InT* __restrict__ x, int64_t M, int64_t K,
                                                           const float* __restrict__ scale, uint8_t* __restrict__ q) {
    const QScale p = make_qscale(scale[0], kE4M3Max);
    const int64_t upr = K >> 4, nunits = M * upr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nunits; u += stride) {
        const int64_t m = u / upr, k = (u - m * upr) << 4;
        *reinterpret_cast<uint4*>(q + packed_offset(m, k, K >> 7)) = encode16_given<InT, 0>(x + m * K + k, p);
    }
}

hipError_t launch_static_quant_packed(const void* x, bool x_is_bf16, int64_t M, int64_t K, const float* scale,
                                      uint8_t* q, hipStream_t stream) {
    if (M == 0 || K == 0) return hipSuccess;
    const int64_t nunits = M * (K >> 4);
    int64_t blocks = (nunits + 255) / 256;
    if (blocks > 256 * 16) blocks = 256 * 16;
    dim3 grid((unsigned)blocks), block(256);
    if (x_is_bf16) static_quant_packed<uint16_t><<<grid, block, 0, stream>>>((const uint16_t*)x, M, K, scale, q);
    else static_quant_packed<float><<<grid, block, 0, stream>>>((const float*)x, M, K, scale, q);
    return hipGetLastError();
}

}  // namespace fp8sg
