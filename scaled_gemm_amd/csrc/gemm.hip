// FP8 W8A8 scaled GEMM for gfx950:  Y[m, n] = s_a[m] * s_w[n] * sum_k a_q[m, k] w_q[n, k].
//
// The scales are constant along k, so they leave the sum and are applied once
// per output in the epilogue (FP8 Inference Explained, in depth -- "Inside a
// quantized linear layer"); the products accumulate in fp32 and the result is
// written as bf16 (FP8 Quantization notebook -- "How FP8 Matmul Works at the
// Hardware Level").
//
// Operands are K-contiguous: A_q [M, K] and W_q [N, K] (W_q^T is the column-major
// "B" of the pages' scaled-matmul call).  The matrix-core "A" operand is W (its
// rows index n) and the "B" operand is A_q (its columns index m), so the 16x16
// output fragment of a lane holds four consecutive n of one row m of Y and the
// bf16 stores are 8-byte vectors.
//
// One lane's share of a 128-deep k block is 32 consecutive FP8 bytes of one row,
// at byte offset 32 * (lane / 16).  Both operands use this same k assignment,
// so the products pair up correctly whatever order the hardware sums them in.
//  * FP8 mode: one v_mfma_f32_16x16x128_f8f6f4 per 16x16 tile and k block.
//  * Exact mode: the 32 bytes are widened exactly to bf16 (every E4M3 value is a
//    bf16 value) and fed to four v_mfma_f32_16x16x32_bf16, bytes 8s..8s+7 to
//    step s.  The bf16 matrix cores form these products exactly and add them at
//    fp32 precision, whereas the FP8 matrix cores align each group of 8
//    products to the group's largest one and drop bits below 2^(e_max - 13).
#include "fp8_device.h"
#include "launch.h"

#ifndef SKINNY_NS
#define SKINNY_NS 2
#endif
#ifndef SKINNY_KS
#define SKINNY_KS 4
#endif
#ifndef SKINNY_DEPTH
#define SKINNY_DEPTH 2
#endif

namespace fp8sg {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Frag {  // 32 FP8 bytes
    uint4 lo, hi;
};

__device__ __forceinline__ Frag zero_frag() {
    Frag f;
    f.lo = make_uint4(0, 0, 0, 0);
    f.hi = f.lo;
    return f;
}

__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
    uint32_t u[4] = {e4m3x2_to_bf16x2(w0, false), e4m3x2_to_bf16x2(w0, true), e4m3x2_to_bf16x2(w1, false),
                     e4m3x2_to_bf16x2(w1, true)};
    bf16x8 v;
    __builtin_memcpy(&v, u, 16);
    return v;
}

__device__ __forceinline__ f32x4 mma_fp8(const Frag& a, const Frag& b, f32x4 acc) {
    i32x8 av, bv;
    __builtin_memcpy(&av, &a, 32);
    __builtin_memcpy(&bv, &b, 32);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_exact(const Frag& a, const Frag& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(a.lo.x, a.lo.y), widen8(b.lo.x, b.lo.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(a.lo.z, a.lo.w), widen8(b.lo.z, b.lo.w), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(a.hi.x, a.hi.y), widen8(b.hi.x, b.hi.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(a.hi.z, a.hi.w), widen8(b.hi.z, b.hi.w), acc, 0, 0, 0);
    return acc;
}

template <bool kFp8>
__device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 acc) {
    return kFp8 ? mma_fp8(a, b, acc) : mma_exact(a, b, acc);
}

__device__ __forceinline__ Frag load_frag_global(const uint8_t* p) {
    Frag f;
    f.lo = reinterpret_cast<const uint4*>(p)[0];
    f.hi = reinterpret_cast<const uint4*>(p)[1];
    return f;
}

// Packed weights: the 2048-byte block of 16-row tile t and k block kb holds the
// 64 lanes' first 16-byte halves, then their second halves, in lane order.
constexpr int64_t kPackBlock = 2048;

__device__ __forceinline__ Frag load_frag_packed(const uint8_t* block, int lane) {
    Frag f;
    f.lo = reinterpret_cast<const uint4*>(block)[lane];
    f.hi = reinterpret_cast<const uint4*>(block + 1024)[lane];
    return f;
}

// Epilogue for one 16x16 fragment: lane holds acc[r] = C[n0 + r][m], r = 0..3.
template <bool kYbf16>
__device__ __forceinline__ void store4(void* y, int64_t N, int64_t m, int64_t n0, f32x4 acc, float sa,
                                       const float* __restrict__ sw, bool vec_ok) {
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (n0 + r < N) ? (acc[r] * sa) * sw[n0 + r] : 0.0f;
    if (kYbf16) {
        uint16_t* yr = (uint16_t*)y + m * N;
        if (vec_ok && n0 + 3 < N) {
            uint2 o;
            o.x = pack_bf16x2(v[0], v[1]);
            o.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(yr + n0) = o;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n0 + r < N) yr[n0 + r] = (uint16_t)(pack_bf16x2(v[r], 0.0f) & 0xFFFFu);
        }
    } else {
        float* yr = (float*)y + m * N;
        if (vec_ok && n0 + 3 < N) {
            *reinterpret_cast<float4*>(yr + n0) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n0 + r < N) yr[n0 + r] = v[r];
        }
    }
}

// ---------------------------------------------------------------------------
// Skinny GEMM (M <= 16 * kMT), the decode shape: every byte of W is used once,
// so W streams from HBM straight into registers.  A workgroup owns kNS 16-row
// subtiles of W; its kKS waves split the k blocks round-robin (wave w takes
// blocks w, w + kKS, ...).  Each wave issues the loads of kDepth of its blocks
// back to back, then multiplies them, so kDepth * (kNS + kMT) * 32 bytes per lane
// are in flight; the loop body has no branches around loads (rows past M or N
// are clamped to the last valid row and masked in the epilogue), which lets
// the compiler wait for each block's loads separately.  The kKS partial sums
// are added in a fixed order through LDS, so the result does not depend on
// timing.
template <bool kFp8, bool kYbf16, int kMT, int kNS, int kKS, int kDepth, bool kWPacked>
__global__ __launch_bounds__(64 * kKS) void gemm_skinny(const uint8_t* __restrict__ A, const float* __restrict__ sa,
                                                        int sa_per_token, const uint8_t* __restrict__ W,
                                                        const float* __restrict__ sw, void* __restrict__ Y, int M,
                                                        int N, int K) {
    __shared__ f32x4 red[kKS > 1 ? kKS - 1 : 1][kNS * kMT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n_base = (int64_t)blockIdx.x * (16 * kNS);
    const int nkb = K >> 7;
    const int r16 = lane & 15, kofs = (lane >> 4) * 32;

    // row-major: this lane's row of each subtile; packed: the subtile's first block
    const uint8_t* wrow[kNS];
    const int64_t last_tile = ((int64_t)N + 15) / 16 - 1;
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
        if (kWPacked) {
            int64_t t = (n_base >> 4) + s;
            t = t < last_tile ? t : last_tile;
            wrow[s] = W + t * nkb * kPackBlock;
        } else {
            int64_t n = n_base + 16 * s + r16;
            n = n < N ? n : N - 1;
            wrow[s] = W + n * (int64_t)K + kofs;
        }
    }
    const uint8_t* arow[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
        int m = 16 * t + r16;
        m = m < M ? m : M - 1;
        arow[t] = A + (int64_t)m * K + kofs;
    }

    f32x4 acc[kNS][kMT];
#pragma unroll
    for (int s = 0; s < kNS; ++s)
#pragma unroll
        for (int t = 0; t < kMT; ++t) acc[s][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // this wave's blocks: wave + j * kKS, j < nper
    const int nper = nkb > wave ? (nkb - wave + kKS - 1) / kKS : 0;
    for (int j0 = 0; j0 < nper; j0 += kDepth) {
        Frag wf[kDepth][kNS], af[kDepth][kMT];
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            int j = j0 + d;
            j = j < nper ? j : nper - 1;  // a clamped (repeated) block past the end is loaded but not used
            const int kb = wave + j * kKS;
            const int64_t off = (int64_t)kb << 7;
#pragma unroll
            for (int s = 0; s < kNS; ++s)
                wf[d][s] = kWPacked ? load_frag_packed(wrow[s] + kb * kPackBlock, lane) : load_frag_global(wrow[s] + off);
#pragma unroll
            for (int t = 0; t < kMT; ++t) af[d][t] = load_frag_global(arow[t] + off);
        }
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (j0 + d < nper) {
#pragma unroll
                for (int s = 0; s < kNS; ++s)
#pragma unroll
                    for (int t = 0; t < kMT; ++t) acc[s][t] = mma<kFp8>(wf[d][s], af[d][t], acc[s][t]);
            }
        }
    }

    if (kKS > 1) {
        if (wave > 0) {
#pragma unroll
            for (int s = 0; s < kNS; ++s)
#pragma unroll
                for (int t = 0; t < kMT; ++t) red[wave - 1][s * kMT + t][lane] = acc[s][t];
        }
        __syncthreads();
    }
    if (wave == 0) {
        const bool vec_ok = (N & 3) == 0;
#pragma unroll
        for (int s = 0; s < kNS; ++s)
#pragma unroll
            for (int t = 0; t < kMT; ++t) {
                f32x4 v = acc[s][t];
#pragma unroll
                for (int w = 0; w < kKS - 1; ++w) v += red[w][s * kMT + t][lane];
                const int m = 16 * t + r16;
                const int64_t n0 = n_base + 16 * s + 4 * (lane >> 4);
                if (m < M && n0 < N) store4<kYbf16>(Y, N, m, n0, v, sa[sa_per_token ? m : 0], sw, vec_ok);
            }
    }
}

// ---------------------------------------------------------------------------
// Tiled GEMM: 128 (m) x 128 (n) output tile per workgroup, 4 waves in a 2 x 2
// arrangement of 64 x 64, k in blocks of 128.  Both 128 x 128-byte operand
// tiles are staged through LDS, double buffered: the global loads of block
// kb + 1 are in flight while block kb is multiplied.  LDS rows are 128 bytes;
// the 16-byte chunk c of row r is stored at chunk c ^ (r & 7), so the 16 lanes
// of a fragment read hit distinct banks.
constexpr int kTile = 128;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <bool kFp8, bool kYbf16, bool kWPacked>
__global__ __launch_bounds__(256, 2) void gemm_tiled(const uint8_t* __restrict__ A, const float* __restrict__ sa,
                                                     int sa_per_token, const uint8_t* __restrict__ W,
                                                     const float* __restrict__ sw, void* __restrict__ Y, int M,
                                                     int N, int K) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTile * 128];  // [stage][A=0/W=1]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int tiles_n = (N + kTile - 1) / kTile;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int64_t m_base = (int64_t)tm * kTile, n_base = (int64_t)tn * kTile;
    const int nkb = K >> 7;

    // loader: 1024 16-byte chunks per operand tile, 4 per thread.  A (and
    // row-major W) go to the swizzled row layout; packed W keeps its fragment
    // order (eight 2048-byte blocks), so its fragment reads are lane-contiguous.
    const int64_t last_tile = ((int64_t)N + 15) / 16 - 1;
    uint4 ra[4], rw[4];
    auto gload = [&](int kb) {
        const int64_t koff = (int64_t)kb << 7;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + 256 * i, row = id >> 3, c = id & 7;
            const int64_t m = m_base + row;
            ra[i] = m < M ? *reinterpret_cast<const uint4*>(A + m * K + koff + c * 16) : make_uint4(0, 0, 0, 0);
            if (kWPacked) {
                int64_t t = (n_base >> 4) + (id >> 7);
                t = t < last_tile ? t : last_tile;
                rw[i] = *reinterpret_cast<const uint4*>(W + (t * nkb + kb) * kPackBlock + (id & 127) * 16);
            } else {
                const int64_t n = n_base + row;
                rw[i] = n < N ? *reinterpret_cast<const uint4*>(W + n * K + koff + c * 16) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto swrite = [&](int stage) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + 256 * i, row = id >> 3, c = id & 7;
            *reinterpret_cast<uint4*>(&lds[stage][0][swz(row, c)]) = ra[i];
            *reinterpret_cast<uint4*>(&lds[stage][1][kWPacked ? id * 16 : swz(row, c)]) = rw[i];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int r16 = lane & 15, c0 = (lane >> 4) * 2;  // this lane's two 16-byte chunks of a row
    if (nkb > 0) {
        gload(0);
        swrite(0);
    }
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int st = kb & 1;
        if (kb + 1 < nkb) gload(kb + 1);
        Frag wf[4], af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (kWPacked) {
                wf[i] = load_frag_packed(&lds[st][1][(wn * 4 + i) * kPackBlock], lane);
            } else {
                const int rw_ = wn * 64 + 16 * i + r16;
                wf[i].lo = *reinterpret_cast<const uint4*>(&lds[st][1][swz(rw_, c0)]);
                wf[i].hi = *reinterpret_cast<const uint4*>(&lds[st][1][swz(rw_, c0 + 1)]);
            }
            const int ra_ = wm * 64 + 16 * i + r16;
            af[i].lo = *reinterpret_cast<const uint4*>(&lds[st][0][swz(ra_, c0)]);
            af[i].hi = *reinterpret_cast<const uint4*>(&lds[st][0][swz(ra_, c0 + 1)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mma<kFp8>(wf[i], af[j], acc[i][j]);
        if (kb + 1 < nkb) swrite(st ^ 1);
        __syncthreads();
    }

    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m_base + wm * 64 + 16 * j + r16;
        if (m >= M) continue;
        const float sam = sa[sa_per_token ? m : 0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n0 = n_base + wn * 64 + 16 * i + 4 * (lane >> 4);
            if (n0 < N) store4<kYbf16>(Y, N, m, n0, acc[i][j], sam, sw, vec_ok);
        }
    }
}

template <bool kFp8, bool kYbf16, bool kWPacked, int kMT, int kNS, int kKS, int kDepth>
static void launch_skinny(const uint8_t* aq, const float* sa, int sa_pt, const uint8_t* wq, const float* sw, void* y,
                          int M, int N, int K, hipStream_t stream) {
    dim3 grid((unsigned)((N + 16 * kNS - 1) / (16 * kNS))), block(64 * kKS);
    gemm_skinny<kFp8, kYbf16, kMT, kNS, kKS, kDepth, kWPacked>
        <<<grid, block, 0, stream>>>(aq, sa, sa_pt, wq, sw, y, M, N, K);
}

template <bool kFp8, bool kYbf16, bool kWPacked>
static hipError_t launch_gemm_t(const uint8_t* aq, const float* sa, int sa_pt, const uint8_t* wq, const float* sw,
                                void* y, int M, int N, int K, hipStream_t stream) {
    if (M <= 16) {
        launch_skinny<kFp8, kYbf16, kWPacked, 1, SKINNY_NS, SKINNY_KS, SKINNY_DEPTH>(aq, sa, sa_pt, wq, sw, y, M, N, K,
                                                                                     stream);
    } else if (M <= 32) {
        launch_skinny<kFp8, kYbf16, kWPacked, 2, SKINNY_NS, SKINNY_KS, SKINNY_DEPTH>(aq, sa, sa_pt, wq, sw, y, M, N, K,
                                                                                     stream);
    } else {
        const int64_t tiles = (int64_t)((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile);
        dim3 grid((unsigned)tiles), block(256);
        gemm_tiled<kFp8, kYbf16, kWPacked><<<grid, block, 0, stream>>>(aq, sa, sa_pt, wq, sw, y, M, N, K);
    }
    return hipGetLastError();
}

template <bool kFp8, bool kWPacked>
static hipError_t launch_gemm_y(const uint8_t* aq, const float* sa, int pt, const uint8_t* wq, const float* sw, void* y,
                                bool y_bf16, int M, int N, int K, hipStream_t stream) {
    return y_bf16 ? launch_gemm_t<kFp8, true, kWPacked>(aq, sa, pt, wq, sw, y, M, N, K, stream)
                  : launch_gemm_t<kFp8, false, kWPacked>(aq, sa, pt, wq, sw, y, M, N, K, stream);
}

hipError_t launch_gemm(const uint8_t* aq, const float* a_scales, bool a_per_token, const uint8_t* wq, bool w_packed,
                       const float* w_scales, void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, bool fp8_mfma,
                       hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const int pt = a_per_token ? 1 : 0;
    const int m = (int)M, n = (int)N, k = (int)K;
    if (fp8_mfma)
        return w_packed ? launch_gemm_y<true, true>(aq, a_scales, pt, wq, w_scales, y, y_bf16, m, n, k, stream)
                        : launch_gemm_y<true, false>(aq, a_scales, pt, wq, w_scales, y, y_bf16, m, n, k, stream);
    return w_packed ? launch_gemm_y<false, true>(aq, a_scales, pt, wq, w_scales, y, y_bf16, m, n, k, stream)
                    : launch_gemm_y<false, false>(aq, a_scales, pt, wq, w_scales, y, y_bf16, m, n, k, stream);
}

// ---------------------------------------------------------------------------
// Weight packing: one thread per 16-byte chunk of the packed buffer.  Chunk c
// belongs to block c / 128 = (tile t, k block kb) and to half h = (c % 128) / 64
// of lane l = c % 64, which reads row 16 t + l % 16 at byte kb * 128 + 32 (l / 16)
// + 16 h; rows past N are written as zero codes.
__global__ __launch_bounds__(256) void pack_weights(const uint8_t* __restrict__ wq, int64_t N, int64_t K,
                                                    uint8_t* __restrict__ wp, int64_t nchunks) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= nchunks) return;
    const int64_t nkb = K >> 7;
    const int64_t block = c >> 7;
    const int within = (int)(c & 127), h = within >> 6, l = within & 63;
    const int64_t t = block / nkb, kb = block % nkb;
    const int64_t row = 16 * t + (l & 15);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < N) v = *reinterpret_cast<const uint4*>(wq + row * K + kb * 128 + 32 * (l >> 4) + 16 * h);
    reinterpret_cast<uint4*>(wp)[c] = v;
}

hipError_t launch_pack_weights(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wp, hipStream_t stream) {
    const int64_t rows = (N + 15) / 16 * 16;
    const int64_t nchunks = rows * K / 16;
    if (nchunks == 0) return hipSuccess;
    const int64_t blocks = (nchunks + 255) / 256;
    pack_weights<<<(unsigned)blocks, 256, 0, stream>>>(wq, N, K, wp, nchunks);
    return hipGetLastError();
}

}  // namespace fp8sg
