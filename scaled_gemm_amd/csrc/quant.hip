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
// Memory access: 16-byte loads, consecutive lanes on consecutive 16-byte
// chunks; the codes leave with non-temporal stores (written once, never read
// back by the kernel).  All of these kernels are bound by HBM bandwidth.
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

// The 16 elements of a unit as two chunks of 8 (loads issued before any use).
template <typename InT, bool kStream>
__device__ __forceinline__ void load_unit(const InT* p, float (&v)[8], float (&w)[8]) {
    if (kStream) {
        load_chunk_stream<InT>(p, v);
        load_chunk_stream<InT>(p + 8, w);
    } else {
        load_chunk<InT>(p, v);
        load_chunk<InT>(p + 8, w);
    }
}

// One workgroup of 256 threads per row; thread t holds units t, t + 256, ...
// (kUnits of them, 16 consecutive elements each) as raw words between the
// maximum and the encode, so X is read once.  Each unit's 16 codes leave in one
// 16-byte non-temporal store (16 contiguous bytes in the fragment order too).
// On [8192, 4096] and [4096, 8192] bf16 this measured 7% faster than 8-element
// chunks with 8-byte stores, and 4-14% faster than one wave per row (which
// leaves too few rows in flight to overlap one row's stores with the next
// row's loads).
template <typename InT, int kUnits, bool kPacked>
__global__ __launch_bounds__(256) void row_quant_units(const InT* __restrict__ x, int64_t K,
                                                       uint8_t* __restrict__ q, float* __restrict__ scales) {
    constexpr int kWords = (int)sizeof(InT);      // 16-byte words per unit: 2 (bf16) or 4 (fp32)
    constexpr int kPerWord = 16 / kWords;          // elements per word
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const InT* xr = x + row * K;
    const int nunits = (int)(K >> 4);
    uint4 r[kUnits][kWords];
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        const int u = threadIdx.x + 256 * i;
        if (u < nunits) {
#pragma unroll
            for (int w = 0; w < kWords; ++w)
                r[i][w] = *reinterpret_cast<const uint4*>(xr + (int64_t)u * 16 + w * kPerWord);
        }
    }
    auto unpack = [&](int i, float (&v)[16]) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 0; w < kWords; ++w) {
            const uint4 a = r[i][w];
            if constexpr (kWords == 2) {
                v[8 * w + 0] = bf16_lo(a.x); v[8 * w + 1] = bf16_hi(a.x); v[8 * w + 2] = bf16_lo(a.y);
                v[8 * w + 3] = bf16_hi(a.y); v[8 * w + 4] = bf16_lo(a.z); v[8 * w + 5] = bf16_hi(a.z);
                v[8 * w + 6] = bf16_lo(a.w); v[8 * w + 7] = bf16_hi(a.w);
            } else {
                v[4 * w + 0] = __uint_as_float(a.x); v[4 * w + 1] = __uint_as_float(a.y);
                v[4 * w + 2] = __uint_as_float(a.z); v[4 * w + 3] = __uint_as_float(a.w);
            }
        }
    };
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        if ((int)threadIdx.x + 256 * i < nunits) {
            float v[16];
            unpack(i, v);
#pragma unroll
            for (int j = 0; j < 16; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j]));
        }
    }
    amax = block_max(amax, red);
    // keep the raw words, not their unpacked floats, live into the encode pass
#pragma unroll
    for (int i = 0; i < kUnits; ++i)
#pragma unroll
        for (int w = 0; w < kWords; ++w) opaque_words(r[i][w]);
    const float s = dynamic_scale(amax, kE4M3Max);
    if (threadIdx.x == 0) scales[row] = s;
    const QScale p = make_qscale(s, kE4M3Max);
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        const int u = threadIdx.x + 256 * i;
        if (u < nunits) {
            float v[16];
            unpack(i, v);
            float lo[8], hi[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) { lo[j] = v[j]; hi[j] = v[8 + j]; }
            const uint2 c0 = encode_chunk_dynamic<InT>(lo, p), c1 = encode_chunk_dynamic<InT>(hi, p);
            const int64_t k = (int64_t)u * 16;
            uint8_t* dst = kPacked ? q + packed_offset(row, k, K >> 7) : q + row * K + k;
            store16_stream(dst, make_uint4(c0.x, c0.y, c1.x, c1.y));
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

// Per-row quantization straight into the fragment order for rows in whole
// 16-row tiles: one workgroup of 16 waves per tile; wave w takes the k blocks
// w, w + 16, ... (kKb of them) and lane l the 32 elements of row l % 16 at
// 32 (l / 16) in each, which are exactly the bytes of that lane's two 16-byte
// halves of the block (packed_offset).  The row maxima reduce over the four
// lanes of a row (shuffles) and over the waves (LDS); the elements stay in
// registers, and every store instruction writes one contiguous kilobyte.  Rows
// past M are read as row M - 1 and not stored.
template <typename InT, int kKb>
__global__ __launch_bounds__(1024) void row_quant_tile16(const InT* __restrict__ x, int64_t M, int64_t K,
                                                         uint8_t* __restrict__ q, float* __restrict__ scales) {
    constexpr int kWords = (int)sizeof(InT) * 2;   // 16-byte words per 32 elements: 4 (bf16) or 8 (fp32)
    constexpr int kPerWord = 32 / kWords;           // elements per word
    __shared__ float red[16][16];                   // [wave][row]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nkb = K >> 7;
    const int r16 = lane & 15;
    int64_t row = ((int64_t)blockIdx.x << 4) + r16;
    const bool live = row < M;
    row = live ? row : M - 1;
    const InT* xr = x + row * K + 32 * (lane >> 4);
    uint4 d[kKb][kWords];
#pragma unroll
    for (int i = 0; i < kKb; ++i) {
        int64_t kb = wave + 16 * i;
        kb = kb < nkb ? kb : nkb - 1;   // a clamped (repeated) block is loaded but neither counted nor stored
#pragma unroll
        for (int w = 0; w < kWords; ++w) d[i][w] = *reinterpret_cast<const uint4*>(xr + kb * 128 + w * kPerWord);
    }
    auto unpack8 = [&](const uint4& a, float (&v)[8]) __attribute__((always_inline)) {
        if constexpr (sizeof(InT) == 2) {
            v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
            v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
        }
    };
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kKb; ++i) {
        if (wave + 16 * i < nkb) {
#pragma unroll
            for (int w = 0; w < kWords; ++w) {
                if constexpr (sizeof(InT) == 2) {
                    float v[8];
                    unpack8(d[i][w], v);
#pragma unroll
                    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j]));
                } else {
                    amax = fmaxf(amax, fmaxf(fmaxf(__builtin_fabsf(__uint_as_float(d[i][w].x)),
                                                   __builtin_fabsf(__uint_as_float(d[i][w].y))),
                                             fmaxf(__builtin_fabsf(__uint_as_float(d[i][w].z)),
                                                   __builtin_fabsf(__uint_as_float(d[i][w].w)))));
                }
            }
        }
    }
    // the four lanes of a row: l, l + 16, l + 32, l + 48
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (lane < 16) red[wave][lane] = amax;
    __syncthreads();
    amax = red[0][r16];
#pragma unroll
    for (int w = 1; w < 16; ++w) amax = fmaxf(amax, red[w][r16]);
    // keep the raw words, not their unpacked floats, live into the encode pass
#pragma unroll
    for (int i = 0; i < kKb; ++i)
#pragma unroll
        for (int w = 0; w < kWords; ++w) opaque_words(d[i][w]);
    const float s = dynamic_scale(amax, kE4M3Max);
    if (wave == 0 && lane < 16 && live) scales[row] = s;
    const QScale p = make_qscale(s, kE4M3Max);
    if (!live) return;   // no barrier below
#pragma unroll
    for (int i = 0; i < kKb; ++i) {
        const int64_t kb = wave + 16 * i;
        if (kb >= nkb) continue;
        uint2 c[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {   // 8 elements each
            float v[8];
            if constexpr (sizeof(InT) == 2) {
                unpack8(d[i][h], v);
            } else {
                const uint4 a = d[i][2 * h], b = d[i][2 * h + 1];
                v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z);
                v[3] = __uint_as_float(a.w); v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
                v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
            }
            c[h] = encode_chunk_dynamic<InT>(v, p);
        }
        uint8_t* blk = q + (((int64_t)blockIdx.x * nkb + kb) << 11) + (lane << 4);
        store16_stream(blk, make_uint4(c[0].x, c[0].y, c[1].x, c[1].y));
        store16_stream(blk + 1024, make_uint4(c[2].x, c[2].y, c[3].x, c[3].y));
    }
}

// The tile kernel holds 32 elements per k block per lane in at most 128
// registers (16 waves per workgroup): up to 4 k blocks per wave for bf16
// (K <= 8192), 2 for fp32 (K <= 4096).
bool row_quant_tiles_fit(bool x_is_bf16, int64_t K) {
    return K > 0 && K % 128 == 0 && K <= (x_is_bf16 ? 8192 : 4096);
}

hipError_t launch_row_quant_tiles(const void* x, bool x_is_bf16, int64_t M, int64_t K, uint8_t* q, float* scales,
                                  hipStream_t stream) {
    if (M == 0) return hipSuccess;
    if (!row_quant_tiles_fit(x_is_bf16, K)) return hipErrorInvalidValue;
    const int64_t per = (K / 128 + 15) / 16;   // k blocks per wave
    const dim3 grid((unsigned)((M + 15) / 16)), block(1024);
    if (x_is_bf16) {
        const uint16_t* xb = (const uint16_t*)x;
        if (per <= 1) row_quant_tile16<uint16_t, 1><<<grid, block, 0, stream>>>(xb, M, K, q, scales);
        else if (per <= 2) row_quant_tile16<uint16_t, 2><<<grid, block, 0, stream>>>(xb, M, K, q, scales);
        else row_quant_tile16<uint16_t, 4><<<grid, block, 0, stream>>>(xb, M, K, q, scales);
    } else {
        const float* xf = (const float*)x;
        if (per <= 1) row_quant_tile16<float, 1><<<grid, block, 0, stream>>>(xf, M, K, q, scales);
        else row_quant_tile16<float, 2><<<grid, block, 0, stream>>>(xf, M, K, q, scales);
    }
    return hipGetLastError();
}

template <typename InT, bool kPacked>
static hipError_t launch_row_quant_t(const InT* x, int64_t M, int64_t K, uint8_t* q, float* scales,
                                     hipStream_t stream) {
    const int64_t per = (K / 16 + 255) / 256;  // units per thread
    dim3 grid((unsigned)M), block(256);
    if (per <= 1) row_quant_units<InT, 1, kPacked><<<grid, block, 0, stream>>>(x, K, q, scales);
    else if (per <= 2) row_quant_units<InT, 2, kPacked><<<grid, block, 0, stream>>>(x, K, q, scales);
    else if (per <= 4) row_quant_units<InT, 4, kPacked><<<grid, block, 0, stream>>>(x, K, q, scales);
    else row_quant_stream<InT, kPacked><<<grid, block, 0, stream>>>(x, K, q, scales);
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
// registers (K <= 16384), as in row_quant_units.
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

// One workgroup per row; each thread holds kUnits 16-element units of x as
// raw words through the sum of squares, then the normalised values through the
// row maximum and the encode (16-byte loads, 16-byte non-temporal code stores,
// as in row_quant_units).  The sum of squares takes 16 kUnits sequential fused
// multiply-adds per thread, then the wave tree and the fixed-order sum of the
// four waves.
template <typename InT, int kUnits, bool kPacked>
__global__ __launch_bounds__(256) void rmsnorm_quant(const InT* __restrict__ x, const InT* __restrict__ gamma,
                                                     float eps, int64_t K, uint8_t* __restrict__ q,
                                                     float* __restrict__ scales, float* __restrict__ y_out) {
    constexpr int kWords = (int)sizeof(InT);      // 16-byte words per unit: 2 (bf16) or 4 (fp32)
    constexpr int kPerWord = 16 / kWords;          // elements per word
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const InT* xr = x + row * K;
    const int nunits = (int)(K >> 4);
    auto unpack = [](const uint4 (&w)[kWords], float (&v)[16]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kWords; ++i) {
            const uint4 a = w[i];
            if constexpr (kWords == 2) {
                v[8 * i + 0] = bf16_lo(a.x); v[8 * i + 1] = bf16_hi(a.x); v[8 * i + 2] = bf16_lo(a.y);
                v[8 * i + 3] = bf16_hi(a.y); v[8 * i + 4] = bf16_lo(a.z); v[8 * i + 5] = bf16_hi(a.z);
                v[8 * i + 6] = bf16_lo(a.w); v[8 * i + 7] = bf16_hi(a.w);
            } else {
                v[4 * i + 0] = __uint_as_float(a.x); v[4 * i + 1] = __uint_as_float(a.y);
                v[4 * i + 2] = __uint_as_float(a.z); v[4 * i + 3] = __uint_as_float(a.w);
            }
        }
    };
    uint4 r[kUnits][kWords];
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        const int u = threadIdx.x + 256 * i;
        if (u < nunits) {
#pragma unroll
            for (int w = 0; w < kWords; ++w)
                r[i][w] = *reinterpret_cast<const uint4*>(xr + (int64_t)u * 16 + w * kPerWord);
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        if ((int)threadIdx.x + 256 * i < nunits) {
            float v[16];
            unpack(r[i], v);
#pragma unroll
            for (int j = 0; j < 16; ++j) ss = __builtin_fmaf(v[j], v[j], ss);
        }
    }
    ss = block_sum(ss, red);
    const float rs = 1.0f / __builtin_sqrtf(ss / (float)K + eps);
    float y[kUnits][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        const int u = threadIdx.x + 256 * i;
        if (u < nunits) {
            uint4 gw[kWords];
#pragma unroll
            for (int w = 0; w < kWords; ++w)
                gw[w] = *reinterpret_cast<const uint4*>(gamma + (int64_t)u * 16 + w * kPerWord);
            float v[16], g[16];
            unpack(r[i], v);
            unpack(gw, g);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                y[i][j] = (v[j] * rs) * g[j];
                amax = fmaxf(amax, __builtin_fabsf(y[i][j]));
            }
            if (y_out) {
                float4* yo = reinterpret_cast<float4*>(y_out + row * K + (int64_t)u * 16);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    yo[j] = make_float4(y[i][4 * j], y[i][4 * j + 1], y[i][4 * j + 2], y[i][4 * j + 3]);
            }
        }
    }
    amax = block_max(amax, red);
    const float s = dynamic_scale(amax, kE4M3Max);
    if (threadIdx.x == 0) scales[row] = s;
    const QScale p = make_qscale(s, kE4M3Max);
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        const int u = threadIdx.x + 256 * i;
        if (u < nunits) {
            float lo[8], hi[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) { lo[j] = y[i][j]; hi[j] = y[i][8 + j]; }
            const uint2 c0 = encode_chunk_dynamic<float>(lo, p), c1 = encode_chunk_dynamic<float>(hi, p);
            const int64_t k = (int64_t)u * 16;
            uint8_t* dst = kPacked ? q + packed_offset(row, k, K >> 7) : q + row * K + k;
            store16_stream(dst, make_uint4(c0.x, c0.y, c1.x, c1.y));
        }
    }
}

template <typename InT, bool kPacked>
static void launch_rmsnorm_quant_t(const InT* x, const InT* g, float eps, int64_t M, int64_t K, uint8_t* q,
                                   float* scales, float* y_out, hipStream_t stream) {
    const int64_t per = (K / 16 + 255) / 256;   // units per thread (K <= 16384: at most 4)
    dim3 grid((unsigned)M), block(256);
    if (per <= 1) rmsnorm_quant<InT, 1, kPacked><<<grid, block, 0, stream>>>(x, g, eps, K, q, scales, y_out);
    else if (per <= 2) rmsnorm_quant<InT, 2, kPacked><<<grid, block, 0, stream>>>(x, g, eps, K, q, scales, y_out);
    else rmsnorm_quant<InT, 4, kPacked><<<grid, block, 0, stream>>>(x, g, eps, K, q, scales, y_out);
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
// Activations, one scale per (row, 128-element group): a group is 8 units of
// 16 elements, one unit per thread (two 16-byte loads for bf16), so the 8
// threads of a group take its maximum with three shuffles and each encodes its
// own unit into one 16-byte non-temporal store.  Units per row are a multiple
// of 8 (K % 128 == 0), and the grid strides over units in multiples of 256, so
// a group's 8 threads are always active together (the shuffles stay inside the
// group).  The grid covers every unit once up to 2^28 units.  Row-major codes
// (the fragment order: group_quant_packed below).
// scales[m * (K / 128) + g] = RN32(amax / 448) (1.0 for an all-zero group).
template <typename InT>
__global__ __launch_bounds__(256) void group_quant(const InT* __restrict__ x, int64_t K, int64_t nunits,
                                                   uint8_t* __restrict__ q, float* __restrict__ scales, int64_t M,
                                                   int kmajor) {
    constexpr int kWords = (int)sizeof(InT);      // 16-byte words per unit: 2 (bf16) or 4 (fp32)
    constexpr int kPerWord = 16 / kWords;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nunits; u += stride) {
        uint4 w[kWords];
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = *reinterpret_cast<const uint4*>(x + u * 16 + i * kPerWord);
        float v[16];
#pragma unroll
        for (int i = 0; i < kWords; ++i) {
            const uint4 a = w[i];
            if constexpr (kWords == 2) {
                v[8 * i + 0] = bf16_lo(a.x); v[8 * i + 1] = bf16_hi(a.x); v[8 * i + 2] = bf16_lo(a.y);
                v[8 * i + 3] = bf16_hi(a.y); v[8 * i + 4] = bf16_lo(a.z); v[8 * i + 5] = bf16_hi(a.z);
                v[8 * i + 6] = bf16_lo(a.w); v[8 * i + 7] = bf16_hi(a.w);
            } else {
                v[4 * i + 0] = __uint_as_float(a.x); v[4 * i + 1] = __uint_as_float(a.y);
                v[4 * i + 2] = __uint_as_float(a.z); v[4 * i + 3] = __uint_as_float(a.w);
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j]));
#pragma unroll
        for (int off = 4; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        const float s = dynamic_scale(amax, kE4M3Max);
        if ((u & 7) == 0) {
            // group g = u / 8 is (row g / nkb, k block g % nkb): row-major [M, K/128] or k-block-major [K/128, M]
            const int64_t g = u >> 3, nkb = K >> 7;
            scales[kmajor ? (g % nkb) * M + g / nkb : g] = s;
        }
        const QScale p = make_qscale(s, kE4M3Max);
        float lo[8], hi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) { lo[j] = v[j]; hi[j] = v[8 + j]; }
        const uint2 c0 = encode_chunk_dynamic<InT>(lo, p), c1 = encode_chunk_dynamic<InT>(hi, p);
        store16_stream(q + u * 16, make_uint4(c0.x, c0.y, c1.x, c1.y));
    }
}

// The same rule written straight into the fragment order: thread t takes lane
// slot l = t % 64 of fragment block b = t / 64 (16-row tile b / nkb, k block
// b % nkb), i.e. the 32 elements of row 16 (b / nkb) + l % 16 at
// 128 (b % nkb) + 32 (l / 16), whose codes are the lane's two 16-byte halves.
// A group (row, k block) is the four lanes l % 16 of one wave (two shuffles),
// and every store instruction writes a contiguous kilobyte.  Rows past M are
// read as row M - 1 and not written.
template <typename InT>
__global__ __launch_bounds__(256) void group_quant_packed(const InT* __restrict__ x, int64_t M, int64_t K,
                                                          uint8_t* __restrict__ q, float* __restrict__ scales,
                                                          int kmajor) {
    const int64_t nkb = K >> 7;
    const int64_t nthreads = ((M + 15) >> 4) * nkb * 64;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;   // a multiple of 64: waves stay whole
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nthreads; t += stride) {
        const int64_t b = t >> 6;
        const int l = (int)(t & 63);
        const int64_t kb = b % nkb;
        int64_t m = ((b / nkb) << 4) + (l & 15);
        const bool live = m < M;
        m = live ? m : M - 1;
        const InT* src = x + m * K + kb * 128 + 32 * (l >> 4);
        float v0[8], v1[8], v2[8], v3[8];
        load_unit<InT, false>(src, v0, v1);
        load_unit<InT, false>(src + 16, v2, v3);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            amax = fmaxf(amax, fmaxf(fmaxf(__builtin_fabsf(v0[j]), __builtin_fabsf(v1[j])),
                                     fmaxf(__builtin_fabsf(v2[j]), __builtin_fabsf(v3[j]))));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const float s = dynamic_scale(amax, kE4M3Max);
        if (!live) continue;
        if (l < 16) scales[kmajor ? kb * M + m : m * nkb + kb] = s;
        const QScale p = make_qscale(s, kE4M3Max);
        const uint2 c0 = encode_chunk_dynamic<InT>(v0, p), c1 = encode_chunk_dynamic<InT>(v1, p);
        const uint2 c2 = encode_chunk_dynamic<InT>(v2, p), c3 = encode_chunk_dynamic<InT>(v3, p);
        uint8_t* dst = q + (b << 11) + (l << 4);
        store16_stream(dst, make_uint4(c0.x, c0.y, c1.x, c1.y));
        store16_stream(dst + 1024, make_uint4(c2.x, c2.y, c3.x, c3.y));
    }
}

hipError_t launch_group_quant(const void* x, bool x_is_bf16, int64_t M, int64_t K, uint8_t* q, float* scales,
                              bool packed, bool scales_kmajor, hipStream_t stream) {
    if (M == 0 || K == 0) return hipSuccess;
    const int km = scales_kmajor ? 1 : 0;
    if (packed) {
        const int64_t nthreads = ((M + 15) / 16) * (K / 128) * 64;
        // small calls (decode rows) in 64-thread workgroups: more of them to spread over the chip
        const int tpb = nthreads < ((int64_t)1 << 16) ? 64 : 256;
        int64_t blocks = (nthreads + tpb - 1) / tpb;
        if (blocks > ((int64_t)1 << 20)) blocks = (int64_t)1 << 20;
        dim3 grid((unsigned)blocks), block((unsigned)tpb);
        if (x_is_bf16) group_quant_packed<uint16_t><<<grid, block, 0, stream>>>((const uint16_t*)x, M, K, q, scales, km);
        else group_quant_packed<float><<<grid, block, 0, stream>>>((const float*)x, M, K, q, scales, km);
        return hipGetLastError();
    }
    const int64_t nunits = M * (K / 16);
    const int tpb = nunits < ((int64_t)1 << 16) ? 64 : 256;
    int64_t blocks = (nunits + tpb - 1) / tpb;
    if (blocks > ((int64_t)1 << 20)) blocks = (int64_t)1 << 20;
    dim3 grid((unsigned)blocks), block((unsigned)tpb);
    if (x_is_bf16) group_quant<uint16_t><<<grid, block, 0, stream>>>((const uint16_t*)x, K, nunits, q, scales, M, km);
    else group_quant<float><<<grid, block, 0, stream>>>((const float*)x, K, nunits, q, scales, M, km);
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
// with nscales == 1 every unit uses scale 0.  A partial last unit (numel % 16)
// takes a per-element path.

// Sixteen values -> sixteen codes under a given scale, the scale's range test
// taken once for the unit.
template <typename InT, int kFmt>
__device__ __forceinline__ uint4 encode16_given(const float (&v)[8], const float (&w)[8], const QScale& sc) {
    constexpr bool kTwo = sizeof(InT) == 4;
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

// One 16-element unit per thread: the loads go out first, then the unit's
// scale is read and the codes leave with a non-temporal store.
template <typename InT, int kFmt, int kSel, bool kStream>
__global__ __launch_bounds__(256) void grouped_quant(const InT* __restrict__ x, int64_t numel,
                                                     const float* __restrict__ scales, int64_t inner_units,
                                                     int nscales, int shift, uint8_t* __restrict__ q) {
    constexpr bool kTwo = sizeof(InT) == 4;
    constexpr float fmax = kFmt == 0 ? kE4M3Max : kE5M2Max;
    const int64_t nfull = numel >> 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nfull; u += stride) {
        float v[8], w[8];
        load_unit<InT, kStream>(x + (u << 4), v, w);
        const QScale p = make_qscale(scales[unit_group<kSel>(u, inner_units, nscales, shift)], fmax);
        store16_stream(q + (u << 4), encode16_given<InT, kFmt>(v, w, p));
    }
    // tail: the last numel % 16 elements, one thread
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        for (int64_t e = nfull << 4; e < numel; ++e) {
            const QScale p = make_qscale(scales[unit_group<2>(e >> 4, inner_units, nscales, shift)], fmax);
            float xv;
            if (sizeof(InT) == 2) xv = bf16_lo((uint32_t)((const uint16_t*)x)[e]);
            else xv = ((const float*)x)[e];
            q[e] = (uint8_t)(pack4<kFmt>(quotient_given<kTwo>(xv, p), 0.0f, 0.0f, 0.0f) & 0xFFu);
        }
    }
}

template <typename InT, int kFmt>
static void launch_grouped_quant_t(const InT* x, int64_t numel, const float* scales, int64_t inner_units,
                                   int nscales, uint8_t* q, unsigned blocks, bool stream_loads, hipStream_t stream) {
    int shift;
    const int sel = unit_group_select(inner_units, nscales, &shift);
#define FP8SG_GQ(S)                                                                                               \
    do {                                                                                                          \
        if (stream_loads)                                                                                         \
            grouped_quant<InT, kFmt, S, true><<<blocks, 256, 0, stream>>>(x, numel, scales, inner_units, nscales,  \
                                                                          shift, q);                              \
        else                                                                                                      \
            grouped_quant<InT, kFmt, S, false><<<blocks, 256, 0, stream>>>(x, numel, scales, inner_units, nscales, \
                                                                           shift, q);                             \
    } while (0)
    if (sel == 0) FP8SG_GQ(0);
    else if (sel == 1) FP8SG_GQ(1);
    else FP8SG_GQ(2);
#undef FP8SG_GQ
}

hipError_t launch_grouped_quant(const void* x, bool x_is_bf16, int64_t numel, const float* scales,
                                int64_t inner_units, int nscales, int fmt, uint8_t* q, hipStream_t stream) {
    if (numel == 0) return hipSuccess;
    const int64_t nunits = (numel + 15) / 16;
    // One unit per thread: on a 2-byte-read / 1-byte-write stream this grid
    // measured 5-10% faster than grid-stride loops over 2048-8192 workgroups,
    // both at 100 MB and at 1.6 GB.  Inputs larger than the 256 MB last-level
    // cache are also read with streaming loads (4% faster at 1.6 GB, 2% slower
    // at 100 MB).
    int64_t blocks = (nunits + 255) / 256;
    if (blocks > ((int64_t)1 << 31) - 1) blocks = ((int64_t)1 << 31) - 1;
    if (blocks < 1) blocks = 1;
    const bool stream_loads = numel * (x_is_bf16 ? 2 : 4) > ((int64_t)256 << 20);
    if (x_is_bf16) {
        if (fmt == 0) launch_grouped_quant_t<uint16_t, 0>((const uint16_t*)x, numel, scales, inner_units, nscales, q, (unsigned)blocks, stream_loads, stream);
        else launch_grouped_quant_t<uint16_t, 1>((const uint16_t*)x, numel, scales, inner_units, nscales, q, (unsigned)blocks, stream_loads, stream);
    } else {
        if (fmt == 0) launch_grouped_quant_t<float, 0>((const float*)x, numel, scales, inner_units, nscales, q, (unsigned)blocks, stream_loads, stream);
        else launch_grouped_quant_t<float, 1>((const float*)x, numel, scales, inner_units, nscales, q, (unsigned)blocks, stream_loads, stream);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static per-tensor quantization of [M, K] activations (K % 128 == 0) straight
// into the fragment order.  Thread t serves lane l = t % 64 of the 16-row x
// 128-k block b = t / 64: it reads the 32 elements of row 16 (b / nkb) + l % 16
// at k = 128 (b % nkb) + 32 (l / 16) and writes their codes to the lane's two
// 16-byte halves (packed_offset), so each wave writes the block's 2048 bytes
// as two contiguous 1024-byte runs.  Rows past M are not written.
template <typename InT>
__global__ __launch_bounds__(256) void static_quant_packed(const InT* __restrict__ x, int64_t M, int64_t K,
                                                           const float* __restrict__ scale, uint8_t* __restrict__ q) {
    const int64_t nkb = K >> 7;
    const int64_t nthreads = ((M + 15) >> 4) * nkb * 64;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nthreads; t += stride) {
        const int64_t b = t >> 6;
        const int l = (int)(t & 63);
        const int64_t m = ((b / nkb) << 4) + (l & 15);
        if (m >= M) continue;
        const InT* src = x + m * K + (b % nkb) * 128 + 32 * (l >> 4);
        float v0[8], v1[8], v2[8], v3[8];
        load_unit<InT, false>(src, v0, v1);
        load_unit<InT, false>(src + 16, v2, v3);
        const QScale p = make_qscale(scale[0], kE4M3Max);
        uint8_t* dst = q + (b << 11) + (l << 4);
        store16_stream(dst, encode16_given<InT, 0>(v0, v1, p));
        store16_stream(dst + 1024, encode16_given<InT, 0>(v2, v3, p));
    }
}

hipError_t launch_static_quant_packed(const void* x, bool x_is_bf16, int64_t M, int64_t K, const float* scale,
                                      uint8_t* q, hipStream_t stream) {
    if (M == 0 || K == 0) return hipSuccess;
    const int64_t nthreads = ((M + 15) / 16) * (K / 128) * 64;
    int64_t blocks = (nthreads + 255) / 256;
    if (blocks > ((int64_t)1 << 20)) blocks = (int64_t)1 << 20;   // the loop strides over the rest
    dim3 grid((unsigned)blocks), block(256);
    if (x_is_bf16) static_quant_packed<uint16_t><<<grid, block, 0, stream>>>((const uint16_t*)x, M, K, scale, q);
    else static_quant_packed<float><<<grid, block, 0, stream>>>((const float*)x, M, K, scale, q);
    return hipGetLastError();
}

}  // namespace fp8sg
