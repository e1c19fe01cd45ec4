// MXFP8 for gfx950: every 32 consecutive k of a row share one power-of-two
// scale, stored as an E8M0 byte e with the value 2^(e - 127).
//
// Microscaling formats give small blocks of consecutive elements their own
// 8-bit scale ("Quantization for LLM inference: FP8, INT4 (GPTQ, AWQ) and GGUF",
// blog.lo0.es -- "Microscaling: NVFP4 and MXFP4"), laid out along the
// reduction dimension ("Quantization: FP8 inference and KV-cache quantization"
// -- "Training in FP8 or lower").  Scale rule: the pages' dynamic rule
// s = amax / FMAX restricted to powers of two and rounded up, so no element of
// a block saturates; a block of zeros gets 2^0.
//
// The GEMM runs on v_mfma_scale_f32_16x16x128_f8f6f4.  The instruction's own
// k order inside a 128-deep block gives lane l (row l % 16, g = l / 16) the k
// [16 g, 16 g + 16) in its first 16 bytes and [64 + 16 g, 64 + 16 g + 16) in
// its second, and it scales k [32 b, 32 b + 32) of row r by the E8M0 byte of
// lane 16 b + r (both measured on the device with one nonzero code and one
// changed scale at a time).  The unscaled FP8 kernels may give a lane any 32
// bytes as long as both operands agree; here a lane's bytes must be the
// instruction's k, so MX operands use that "MX fragment order": row-major
// operands are read as two 16-byte pieces 64 bytes apart, and packed MX codes
// (written by fp8_quant_mx) hold those pieces at 16 l and 1024 + 16 l of the
// 2048-byte block of (16-row tile, 128-k block).  The instruction applies the
// two scales to the products of each block and accumulates in fp32, with the
// FP8 matrix cores' in-instruction alignment of each 8-product group.
//
// Scale layout the GEMM reads ("packed"): for k block kb (128 deep) and group
// of four 16-row tiles g, 256 bytes at (kb * T4 + g) * 256, T4 = ceil(rows / 64);
// inside, lane l's scale of tile 4 g + j is byte 4 l + j, for row
// 16 (4 g + j) + l % 16 and 32-k group l / 16.  A 256-row GEMM tile's scales of
// one k block are then one contiguous kilobyte, and one dword per lane holds
// the scales of four tiles.
#include <type_traits>

#include "gemm_common.h"

namespace fp8sg {

constexpr int kMxBlock = 32;

// The block's scale exponent: the smallest k with amax <= FMAX 2^k, clamped
// to [-127, 127]; 0 for amax == 0.  FMAX = 1.75 * 2^emax (emax 8 for E4M3, 15
// for E5M2), so for a normal amax = (1 + f) 2^E the answer is E - emax, plus
// one when 1 + f > 1.75.  A subnormal amax lies below 448 * 2^-127 and clamps.
template <int kFmt>
__device__ __forceinline__ int mx_scale_exp(float amax) {
    constexpr int kEmax = kFmt == 0 ? 8 : 15;
    const uint32_t u = __float_as_uint(amax);
    if (u == 0) return 0;
    const int e = (int)(u >> 23);
    if (e == 0) return -127;
    const int k = e - 127 - kEmax + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// Byte offset of the scale of (row r, 32-k block b) in the packed layout.
__device__ __forceinline__ int64_t mx_packed_scale_offset(int64_t r, int b, int64_t T4) {
    const int64_t t = r >> 4;
    const int kb = b >> 2, grp = b & 3;
    const int lane = grp * 16 + (int)(r & 15);
    return (((int64_t)kb * T4 + (t >> 2)) * 64 + lane) * 4 + (t & 3);
}

// ---------------------------------------------------------------------------
// Quantization.  A team of four consecutive threads takes one 32-element
// block, 8 elements (one 16-byte bf16 load, two for fp32) per thread: the
// block maximum comes from two lane exchanges, the quotient x / 2^k is the
// product x * 2^-k (both correctly rounded, so equal), and every |quotient|
// is at most FMAX, which the hardware converter rounds to nearest even
// exactly.  Codes go out row-major; the team's first thread writes the scale
// byte (row-major or packed).
template <typename InT, int kFmt, bool kPackedScales>
__global__ __launch_bounds__(256) void mx_quant(const InT* __restrict__ x, int64_t R, int K, uint8_t* __restrict__ q,
                                                uint8_t* __restrict__ sc) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int cpr = K >> 3;                // chunks of 8 per row; a multiple of 4
    if (g >= R * cpr) return;              // whole teams only: R * cpr is a multiple of 4
    const int64_t r = g / cpr;
    const int kk = (int)(g - r * cpr) * 8;
    float v[8];
    load_chunk<InT>(x + r * K + kk, v);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    const int k = mx_scale_exp<kFmt>(a);
    const float rr = __uint_as_float((uint32_t)(127 - k) << 23);   // 2^-k; k <= 120 for finite inputs
    uint2 o;
    o.x = pack4<kFmt>(v[0] * rr, v[1] * rr, v[2] * rr, v[3] * rr);
    o.y = pack4<kFmt>(v[4] * rr, v[5] * rr, v[6] * rr, v[7] * rr);
    *reinterpret_cast<uint2*>(q + r * K + kk) = o;
    if ((kk & 31) == 0) {
        const uint8_t e = (uint8_t)(k + 127);
        if (kPackedScales) sc[mx_packed_scale_offset(r, kk >> 5, (R + 63) >> 6)] = e;
        else sc[r * (K >> 5) + (kk >> 5)] = e;
    }
}

// Quantization into the MX fragment order: one wave per (16-row tile, 128-k
// block), lane l = 16 g + r reads row r's k [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16) (the two halves of its fragment) and writes them
// as 16-byte codes at 16 l and 1024 + 16 l, so every store instruction writes
// one contiguous kilobyte.  The 32-k block of each half is shared with lane
// l ^ 16 (one exchange); each lane writes one scale byte: block g / 2 of its
// first half for even g, block 2 + g / 2 of its second half for odd g.  Rows
// past R read nothing and write no codes.
template <typename InT, int kFmt, bool kPackedScales>
__global__ __launch_bounds__(256) void mx_quant_packed(const InT* __restrict__ x, int64_t R, int K,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
    const int lane = threadIdx.x & 63;
    const int nkb = K >> 7;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (tile, kb), kb fastest
    const int64_t T = (R + 15) >> 4;
    if (unit >= T * nkb) return;                                         // whole waves only
    const int64_t t = unit / nkb;
    const int kb = (int)(unit - t * nkb);
    const int g = lane >> 4, r16 = lane & 15;
    const int64_t r = t * 16 + r16;
    const bool live = r < R;
    float v[2][16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (live) {
            const InT* p = x + r * K + kb * 128 + 64 * h + 16 * g;
            float c0[8], c1[8];
            load_chunk<InT>(p, c0);
            load_chunk<InT>(p + 8, c1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[h][i] = c0[i];
                v[h][8 + i] = c1[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[h][i] = 0.0f;
        }
    }
    int kx[2];
    uint8_t* blk = q + (t * nkb + kb) * kPackBlock;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, __builtin_fabsf(v[h][i]));
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        kx[h] = mx_scale_exp<kFmt>(a);
        const float rr = __uint_as_float((uint32_t)(127 - kx[h]) << 23);
        uint4 o;
        o.x = pack4<kFmt>(v[h][0] * rr, v[h][1] * rr, v[h][2] * rr, v[h][3] * rr);
        o.y = pack4<kFmt>(v[h][4] * rr, v[h][5] * rr, v[h][6] * rr, v[h][7] * rr);
        o.z = pack4<kFmt>(v[h][8] * rr, v[h][9] * rr, v[h][10] * rr, v[h][11] * rr);
        o.w = pack4<kFmt>(v[h][12] * rr, v[h][13] * rr, v[h][14] * rr, v[h][15] * rr);
        if (live) *reinterpret_cast<uint4*>(blk + h * 1024 + lane * 16) = o;
    }
    if (live) {
        const int b = (g & 1) ? 2 + (g >> 1) : (g >> 1);       // this lane's scale: its block in the k block
        const uint8_t e = (uint8_t)(((g & 1) ? kx[1] : kx[0]) + 127);
        if (kPackedScales) sc[mx_packed_scale_offset(r, kb * 4 + b, (R + 63) >> 6)] = e;
        else sc[r * (K >> 5) + kb * 4 + b] = e;
    }
}

template <typename InT, int kFmt>
static void launch_mx_quant_t(const InT* x, int64_t R, int K, uint8_t* q, bool pc, uint8_t* sc, bool ps,
                              hipStream_t stream) {
    if (pc) {
        const int64_t units = ((R + 15) >> 4) * (K >> 7);
        dim3 grid((unsigned)((units + 3) / 4)), block(256);
        if (ps) mx_quant_packed<InT, kFmt, true><<<grid, block, 0, stream>>>(x, R, K, q, sc);
        else mx_quant_packed<InT, kFmt, false><<<grid, block, 0, stream>>>(x, R, K, q, sc);
        return;
    }
    const int64_t threads = R * (K >> 3);
    dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (ps) mx_quant<InT, kFmt, true><<<grid, block, 0, stream>>>(x, R, K, q, sc);
    else mx_quant<InT, kFmt, false><<<grid, block, 0, stream>>>(x, R, K, q, sc);
}

hipError_t launch_mx_quant(const void* x, bool x_is_bf16, int64_t R, int64_t K, int fmt, uint8_t* q,
                           bool packed_codes, uint8_t* scales, bool packed_scales, hipStream_t stream) {
    if (R == 0 || K == 0) return hipSuccess;
    const int k = (int)K;
    if (x_is_bf16) {
        if (fmt == 0) launch_mx_quant_t<uint16_t, 0>((const uint16_t*)x, R, k, q, packed_codes, scales, packed_scales, stream);
        else launch_mx_quant_t<uint16_t, 1>((const uint16_t*)x, R, k, q, packed_codes, scales, packed_scales, stream);
    } else {
        if (fmt == 0) launch_mx_quant_t<float, 0>((const float*)x, R, k, q, packed_codes, scales, packed_scales, stream);
        else launch_mx_quant_t<float, 1>((const float*)x, R, k, q, packed_codes, scales, packed_scales, stream);
    }
    return hipGetLastError();
}

// Row-major scale bytes [R, K / 32] -> the packed layout; one thread per
// packed byte, rows past R get 127 (2^0).
__global__ __launch_bounds__(256) void pack_mx_scales(const uint8_t* __restrict__ s, int64_t R, int K,
                                                      uint8_t* __restrict__ p) {
    const int64_t T4 = (R + 63) >> 6;
    const int64_t total = (int64_t)(K >> 7) * T4 * 256;
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= total) return;
    const int64_t kb = o / (T4 * 256);
    const int64_t rem = o - kb * T4 * 256;
    const int64_t g = rem >> 8;
    const int lane = (int)((rem >> 2) & 63), j = (int)(rem & 3);
    const int64_t r = (4 * g + j) * 16 + (lane & 15);
    const int64_t b = kb * 4 + (lane >> 4);
    p[o] = r < R ? s[r * (K >> 5) + b] : (uint8_t)127;
}

hipError_t launch_pack_mx_scales(const uint8_t* s, int64_t R, int64_t K, uint8_t* p, hipStream_t stream) {
    if (R == 0 || K == 0) return hipSuccess;
    const int64_t total = (K >> 7) * ((R + 63) >> 6) * 256;
    pack_mx_scales<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(s, R, (int)K, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The scaled matrix-core product: W is the instruction's first operand (E4M3),
// the activations its second (E4M3 or E5M2); each takes the E8M0 scale in
// byte 0 of its lane's scale register.
template <int kAFmt>
__device__ __forceinline__ f32x4 mma_mx(const Frag& w, const Frag& a, f32x4 acc, uint32_t sw, uint32_t sa) {
    i32x8 wv, av;
    __builtin_memcpy(&wv, &w, 32);
    __builtin_memcpy(&av, &a, 32);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, av, acc, 0, kAFmt, 0, (int)sw, 0, (int)sa);
}

__device__ __forceinline__ uint32_t scale_byte(uint32_t word, int j) {
    return (word >> (8 * j)) & 0xFFu;
}

// Lane fragment of a row-major operand in MX fragment order: p points at the
// lane's row, k = 128 kb + 16 (lane / 16); the second half lies 64 bytes on.
__device__ __forceinline__ Frag load_frag_mx_global(const uint8_t* p) {
    Frag f;
    f.lo = *reinterpret_cast<const uint4*>(p);
    f.hi = *reinterpret_cast<const uint4*>(p + 64);
    return f;
}

// tile_copy_offsets for MX operands: identical for packed operands; row-major
// copy (j, h) reads row 16 j + lane % 16 at k bytes 16 (lane / 16) + 64 h.
template <bool kPacked>
__device__ __forceinline__ void mx_tile_copy_offsets(uint32_t (&o)[8], int64_t base_row, int rows, int K, int wave,
                                                     int lane) {
    if (kPacked) {
        tile_copy_offsets<true>(o, base_row, rows, K, wave, lane);
        return;
    }
    const int r16 = lane & 15, kq = (lane >> 4) * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = wave * 8 + i, j = c >> 1, h = c & 1;
        int64_t r = base_row + 16 * j + r16;
        r = r < rows ? r : rows - 1;
        o[i] = (uint32_t)((r - base_row) * K + kq + 64 * h);
    }
}

// One lane's MX fragment of a bf16 activation block, quantized in registers by
// the rule of mx_quant_packed (the same codes and scale bytes).  p holds the
// lane's two halves as bf16: p[0..1] are row r's k [16 g, 16 g + 16) of the
// 128-k block and p[2..3] its k [64 + 16 g, 64 + 16 g + 16) (l = 16 g + r);
// the 32-k block of each half is shared with lane l ^ 16.  The instruction
// takes the scale of 32-k block g of row r from lane 16 g + r: blocks 0 and 1
// are the first halves of lanes r and 32 + r, blocks 2 and 3 their second
// halves, so one exchange per half brings each lane its byte.
template <int kFmt>
__device__ __forceinline__ void mx_quant_frag(const uint4 (&p)[4], int lane, Frag& f, uint32_t& sbyte) {
    int kx[2];
    uint4 o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w[8] = {p[2 * h].x, p[2 * h].y, p[2 * h].z, p[2 * h].w,
                               p[2 * h + 1].x, p[2 * h + 1].y, p[2 * h + 1].z, p[2 * h + 1].w};
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        kx[h] = mx_scale_exp<kFmt>(a);
        const float rr = __uint_as_float((uint32_t)(127 - kx[h]) << 23);
        o[h].x = pack4<kFmt>(v[0] * rr, v[1] * rr, v[2] * rr, v[3] * rr);
        o[h].y = pack4<kFmt>(v[4] * rr, v[5] * rr, v[6] * rr, v[7] * rr);
        o[h].z = pack4<kFmt>(v[8] * rr, v[9] * rr, v[10] * rr, v[11] * rr);
        o[h].w = pack4<kFmt>(v[12] * rr, v[13] * rr, v[14] * rr, v[15] * rr);
    }
    f.lo = o[0];
    f.hi = o[1];
    const int g = lane >> 4, src = 32 * (g & 1) + (lane & 15);
    const int k0 = __shfl(kx[0], src, 64), k1 = __shfl(kx[1], src, 64);
    sbyte = (uint32_t)((g < 2 ? k0 : k1) + 127);
}

// Decode shape (M <= 16 kMT): the skinny kernel's organisation -- 32 weight
// rows (two 16-row subtiles) per workgroup, four waves splitting the k blocks
// round-robin, weights streamed into registers with the next block's loads in
// flight while the current block is multiplied, partial sums added in a fixed
// order through LDS.  Per k block a wave also reads one scale dword for its
// two weight subtiles and one for the activation tiles (both in the packed
// layout: 256 contiguous bytes per wave).
//
// kAFromX: A is bf16 X [M, K] row-major (as unused); each wave quantizes its
// own fragments of each k block in registers (mx_quant_frag), so no quantized
// copy of X is written and no separate launch is needed.  The products and
// their order are those of the pre-quantized kernel, so the two paths give
// identical results.  Every workgroup reads all of X, twice the bytes of its
// codes: at M = 8 the call runs at the speed of the GEMM on pre-quantized
// codes (12.0 vs 11.7 us for N = 14336, K = 4096), at M = 32 (two m-tiles)
// those re-reads made it 22.8 us against 3 + 13.4 us for the two launches, so
// the launcher offers one m-tile (M <= 16) only.
template <int kAFmt, int kOut, int kMT, bool kWPacked, bool kAPacked, bool kAFromX = false>
__global__ __launch_bounds__(256) void gemm_skinny_mx(const uint8_t* __restrict__ A, const uint32_t* __restrict__ as,
                                                      const uint8_t* __restrict__ W, const uint32_t* __restrict__ ws,
                                                      void* __restrict__ Y, int M, int N, int K) {
    constexpr int kNS = 2, kKS = 4;
    __shared__ f32x4 red[kKS - 1][kNS * kMT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n_base = (int64_t)blockIdx.x * (16 * kNS);
    const int nkb = K >> 7;
    const int r16 = lane & 15, kofs = (lane >> 4) * 16;

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
        if (kAFromX) {
            int m = 16 * t + r16;
            m = m < M ? m : M - 1;
            arow[t] = A + ((int64_t)m * K + kofs) * 2;   // bf16 elements
        } else if (kAPacked) {
            arow[t] = A + (int64_t)t * nkb * kPackBlock;
        } else {
            int m = 16 * t + r16;
            m = m < M ? m : M - 1;
            arow[t] = A + (int64_t)m * K + kofs;
        }
    }
    // packed scales: the workgroup's two weight tiles share one dword (bytes
    // (n_base / 16) % 4 and the next); the activation tiles are bytes 0 and 1
    const int64_t T4w = ((int64_t)N + 63) >> 6, T4a = ((int64_t)M + 63) >> 6;
    const uint32_t* wsp = ws + (n_base >> 6) * 64 + lane;
    const int wj = (int)((n_base >> 4) & 3);
    const uint32_t* asp = as + lane;

    f32x4 acc[kNS][kMT];
#pragma unroll
    for (int s = 0; s < kNS; ++s)
#pragma unroll
        for (int t = 0; t < kMT; ++t) acc[s][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // the activation operand of one k block: codes (Frag) or, with kAFromX, the
    // lane's 64 bytes of bf16 X (two 16-element halves)
    struct XHalves {
        uint4 p[4];
    };
    using AIn = std::conditional_t<kAFromX, XHalves, Frag>;
    auto load_block = [&](int j, Frag (&wx)[kNS], AIn (&ax)[kMT], uint32_t& swx, uint32_t& sax) {
        const int kb = wave + j * kKS;
        const int64_t off = (int64_t)kb << 7;
#pragma unroll
        for (int s = 0; s < kNS; ++s)
            wx[s] = kWPacked ? load_frag_packed_stream(wrow[s] + kb * kPackBlock, lane)
                              : load_frag_mx_global(wrow[s] + off);
#pragma unroll
        for (int t = 0; t < kMT; ++t) {
            if constexpr (kAFromX) {
                const uint4* px = reinterpret_cast<const uint4*>(arow[t] + off * 2);
                ax[t].p[0] = px[0];
                ax[t].p[1] = px[1];
                ax[t].p[2] = px[8];   // + 64 elements
                ax[t].p[3] = px[9];
            } else {
                ax[t] = kAPacked ? load_frag_packed(arow[t] + kb * kPackBlock, lane)
                                 : load_frag_mx_global(arow[t] + off);
            }
        }
        swx = wsp[(int64_t)kb * T4w * 64];
        sax = kAFromX ? 0u : asp[(int64_t)kb * T4a * 64];
    };
    auto mul_block = [&](const Frag (&wx)[kNS], const AIn (&ax)[kMT], uint32_t swx, uint32_t sax) {
        Frag af[kMT];
        uint32_t sb[kMT];
#pragma unroll
        for (int t = 0; t < kMT; ++t) {
            if constexpr (kAFromX) {
                mx_quant_frag<kAFmt>(ax[t].p, lane, af[t], sb[t]);
            } else {
                af[t] = ax[t];
                sb[t] = scale_byte(sax, t);
            }
        }
#pragma unroll
        for (int s = 0; s < kNS; ++s)
#pragma unroll
            for (int t = 0; t < kMT; ++t)
                acc[s][t] = mma_mx<kAFmt>(wx[s], af[t], acc[s][t], scale_byte(swx, wj + s), sb[t]);
    };
    const int nper = nkb > wave ? (nkb - wave + kKS - 1) / kKS : 0;
    if (nper > 0) {
        Frag wf[kNS];
        AIn af[kMT];
        uint32_t swf, saf;
        load_block(0, wf, af, swf, saf);
        for (int j = 0; j + 1 < nper; ++j) {
            Frag wn[kNS];
            AIn an[kMT];
            uint32_t swn, san;
            load_block(j + 1, wn, an, swn, san);
            __builtin_amdgcn_sched_barrier(0);
            mul_block(wf, af, swf, saf);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < kNS; ++s) wf[s] = wn[s];
#pragma unroll
            for (int t = 0; t < kMT; ++t) af[t] = an[t];
            swf = swn;
            saf = san;
        }
        mul_block(wf, af, swf, saf);
    }

    if (wave > 0) {
#pragma unroll
        for (int s = 0; s < kNS; ++s)
#pragma unroll
            for (int t = 0; t < kMT; ++t) red[wave - 1][s * kMT + t][lane] = acc[s][t];
    }
    __syncthreads();
    if (wave == 0) {
        const bool vec_ok = (N & 3) == 0;
        const QScale q = out_qscale<kOut>(nullptr);
#pragma unroll
        for (int s = 0; s < kNS; ++s)
#pragma unroll
            for (int t = 0; t < kMT; ++t) {
                f32x4 v = acc[s][t];
#pragma unroll
                for (int w = 0; w < kKS - 1; ++w) v += red[w][s * kMT + t][lane];
                const int m = 16 * t + r16;
                const int64_t n0 = n_base + 16 * s + 4 * (lane >> 4);
                if (m < M && n0 < N) store4_raw<kOut>(Y, N, m, n0, v, vec_ok, q);
            }
    }
}

// Large tiles (M > 32): the FP8 large-tile kernel's pipeline (256 x 256
// tiles, 4 waves of 128 x 128, operands copied straight into two LDS stages
// two k blocks ahead, tile order by XCD) with each stage also holding the
// k block's scales: one kilobyte for the tile's 256 A rows and one for its
// 256 W rows, which the packed layout keeps contiguous.  Each wave copies one
// 256-byte group of each, so a stage is 18 copies per wave.
template <int kAFmt, int kOut, bool kWPacked, bool kAPacked>
__global__ __launch_bounds__(256, 1) void gemm_big_mx(const uint8_t* __restrict__ A, const uint8_t* __restrict__ as,
                                                      const uint8_t* __restrict__ W, const uint8_t* __restrict__ ws,
                                                      void* __restrict__ Y, int M, int N, int K, int tiles_per_xcd) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr int kCodes = 32 * kPackBlock;        // A 32 KB + W 32 KB
    constexpr int kStage = kCodes + 2048;          // + A scales 1 KB + W scales 1 KB
    constexpr int kCopies = 18;                    // copies per wave per stage
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    int tile;
    int64_t m_base, n_base;
    tile_coords(M, N, tiles_per_xcd, tile, m_base, n_base);
    if (tile < 0) return;
    const int nkb = K >> 7;

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    uint32_t oa[8], ow[8];
    mx_tile_copy_offsets<kAPacked>(oa, m_base, M, K, wave, lane);
    mx_tile_copy_offsets<kWPacked>(ow, n_base, N, K, wave, lane);
    const uint8_t* a_tile = kAPacked ? A + (m_base >> 4) * (int64_t)nkb * kPackBlock : A + m_base * K;
    const uint8_t* w_tile = kWPacked ? W + (n_base >> 4) * (int64_t)nkb * kPackBlock : W + n_base * K;
    const int64_t a_kb = kAPacked ? kPackBlock : 128;
    const int64_t w_kb = kWPacked ? kPackBlock : 128;
    // this wave's scale group of each operand (clamped to the last group)
    const int64_t T4a = ((int64_t)M + 63) >> 6, T4w = ((int64_t)N + 63) >> 6;
    int64_t ga = (m_base >> 6) + wave, gw = (n_base >> 6) + wave;
    ga = ga < T4a ? ga : T4a - 1;
    gw = gw < T4w ? gw : T4w - 1;
    const uint8_t* as_src = as + ga * 256 + 4 * lane;
    const uint8_t* ws_src = ws + gw * 256 + 4 * lane;
    const int64_t as_kb = T4a * 256, ws_kb = T4w * 256;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

    auto copy_scales = [&](uint32_t stage_lds, int kb) {
        copy4_to_lds(as_src + kb * as_kb, stage_lds + kCodes + 256 * wave);
        copy4_to_lds(ws_src + kb * ws_kb, stage_lds + kCodes + 1024 + 256 * wave);
    };

    if (nkb > 0) {
        const int b1 = nkb > 1 ? 1 : 0;
        issue_tile_copy(smem, a_tile, 0, wave, oa);
        issue_tile_copy(smem + 16 * kPackBlock, w_tile, 0, wave, ow);
        copy_scales(lds0, 0);
        issue_tile_copy(smem + kStage, a_tile, (int64_t)b1 * a_kb, wave, oa);
        issue_tile_copy(smem + kStage + 16 * kPackBlock, w_tile, (int64_t)b1 * w_kb, wave, ow);
        copy_scales(lds0 + kStage, b1);
    }
    for (int kb = 0; kb < nkb; ++kb) {
        uint8_t* cur = smem + (kb & 1) * kStage;
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(kCopies));  // this wave's copies of block kb have landed
        barrier_no_fence();                                // ... and every other wave's
        const uint8_t* la = cur + wm * 8 * kPackBlock;
        const uint8_t* lw = cur + (16 + wn * 8) * kPackBlock;
        Frag wf[8], af[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) af[j] = load_frag_packed(la + j * kPackBlock, lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) wf[i] = load_frag_packed(lw + i * kPackBlock, lane);
        // scale dwords: A tiles 8 wm + j are groups 2 wm + j / 4, W tiles 8 wn + i groups 2 wn + i / 4
        const uint32_t* ls = reinterpret_cast<const uint32_t*>(cur + kCodes);
        const uint32_t sa0 = ls[(2 * wm) * 64 + lane], sa1 = ls[(2 * wm + 1) * 64 + lane];
        const uint32_t sw0 = ls[256 + (2 * wn) * 64 + lane], sw1 = ls[256 + (2 * wn + 1) * 64 + lane];
        uint32_t sab[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sab[j] = scale_byte(j < 4 ? sa0 : sa1, j & 3);
        {
            const uint32_t s0 = scale_byte(sw0, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[0][j] = mma_mx<kAFmt>(wf[0], af[j], acc[0][j], s0, sab[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): all of this wave's LDS reads are done
        barrier_no_fence();                  // ... and every other wave's: the stage may be refilled
        const int n = kb + 2 < nkb ? kb + 2 : nkb - 1;
        const int64_t a_off = (int64_t)n * a_kb, w_off = (int64_t)n * w_kb;
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            const int c0 = kCopySplit[i - 1], c1 = kCopySplit[i];
#pragma unroll
            for (int c = c0; c < c1; ++c) issue_stage_copy(c, cur, a_tile, w_tile, a_off, w_off, wave, oa, ow);
            if (i == 7) copy_scales(lds0 + (uint32_t)((kb & 1) * kStage), n);
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t si = scale_byte(i < 4 ? sw0 : sw1, i & 3);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = mma_mx<kAFmt>(wf[i], af[j], acc[i][j], si, sab[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // no copy into LDS may outlive the workgroup

    if (kOut == kOutBF16) {
        __syncthreads();  // every wave is done with the stages: the LDS now holds the output tiles
        uint8_t* wl = smem + wave * kEpiWaveBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const f32x4 a = acc[i][j];
                epi_put4(wl, 16 * j + (lane & 15), 16 * i + 4 * (lane >> 4), a[0], a[1], a[2], a[3]);
            }
        __syncthreads();
        epi_store(wl, (uint16_t*)Y, M, N, m_base + wm * 128, n_base + wn * 128, lane);
        return;
    }
    const bool vec_ok = (N & 3) == 0;
    const QScale q = out_qscale<kOut>(nullptr);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t m = m_base + wm * 128 + 16 * j + (lane & 15);
        if (m >= M) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t n0 = n_base + wn * 128 + 16 * i + 4 * (lane >> 4);
            if (n0 < N) store4_raw<kOut>(Y, N, m, n0, acc[i][j], vec_ok, q);
        }
    }
}

static_assert(4 * kEpiWaveBytes <= 2 * (32 * kPackBlock + 2048), "the staged output fits the two stages");

template <int kAFmt, int kOut, bool kWPacked, bool kAPacked>
static void launch_mx_t(const uint8_t* aq, const uint8_t* as, const uint8_t* wq, const uint8_t* ws, void* y, int M,
                        int N, int K, hipStream_t stream) {
    if (M <= 32) {
        dim3 grid((unsigned)((N + 31) / 32)), block(256);
        if (M <= 16)
            gemm_skinny_mx<kAFmt, kOut, 1, kWPacked, kAPacked><<<grid, block, 0, stream>>>(
                aq, (const uint32_t*)as, wq, (const uint32_t*)ws, y, M, N, K);
        else
            gemm_skinny_mx<kAFmt, kOut, 2, kWPacked, kAPacked><<<grid, block, 0, stream>>>(
                aq, (const uint32_t*)as, wq, (const uint32_t*)ws, y, M, N, K);
        return;
    }
    const int tiles = ((M + kBig - 1) / kBig) * ((N + kBig - 1) / kBig);
    const int per = (tiles + 7) / 8;
    gemm_big_mx<kAFmt, kOut, kWPacked, kAPacked>
        <<<dim3((unsigned)(per * 8)), dim3(256), 2 * (32 * kPackBlock + 2048), stream>>>(aq, as, wq, ws, y, M, N, K,
                                                                                        per);
}

template <int kAFmt, int kOut>
static void launch_mx_l(const uint8_t* aq, bool a_packed, const uint8_t* as, const uint8_t* wq, bool w_packed,
                        const uint8_t* ws, void* y, int M, int N, int K, hipStream_t stream) {
    if (a_packed) {
        if (w_packed) launch_mx_t<kAFmt, kOut, true, true>(aq, as, wq, ws, y, M, N, K, stream);
        else launch_mx_t<kAFmt, kOut, false, true>(aq, as, wq, ws, y, M, N, K, stream);
    } else {
        if (w_packed) launch_mx_t<kAFmt, kOut, true, false>(aq, as, wq, ws, y, M, N, K, stream);
        else launch_mx_t<kAFmt, kOut, false, false>(aq, as, wq, ws, y, M, N, K, stream);
    }
}

template <int kAFmt, int kOut, bool kWPacked>
static void launch_mx_x_t(const uint16_t* x, const uint8_t* wq, const uint8_t* ws, void* y, int M, int N, int K,
                          hipStream_t stream) {
    dim3 grid((unsigned)((N + 31) / 32)), block(256);
    const uint8_t* xa = reinterpret_cast<const uint8_t*>(x);
    gemm_skinny_mx<kAFmt, kOut, 1, kWPacked, false, true><<<grid, block, 0, stream>>>(
        xa, nullptr, wq, (const uint32_t*)ws, y, M, N, K);
}

hipError_t launch_gemm_mx_bf16x(const uint16_t* x, int a_fmt, const uint8_t* wq, bool w_packed,
                                const uint8_t* w_scales, void* y, int out_kind, int64_t M, int64_t N, int64_t K,
                                hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (M > 16) return hipErrorInvalidValue;  // one 16-row m-tile only (checked by the ABI)
    const int m = (int)M, n = (int)N, k = (int)K;
#define FP8SG_MXX(F, O)                                                            \
    (w_packed ? launch_mx_x_t<F, O, true>(x, wq, w_scales, y, m, n, k, stream)     \
              : launch_mx_x_t<F, O, false>(x, wq, w_scales, y, m, n, k, stream))
    if (a_fmt == 0) {
        if (out_kind == kOutBF16) FP8SG_MXX(0, kOutBF16);
        else FP8SG_MXX(0, kOutF32);
    } else {
        if (out_kind == kOutBF16) FP8SG_MXX(1, kOutBF16);
        else FP8SG_MXX(1, kOutF32);
    }
#undef FP8SG_MXX
    return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* aq, bool a_packed, const uint8_t* a_scales, int a_fmt, const uint8_t* wq,
                          bool w_packed, const uint8_t* w_scales, void* y, int out_kind, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const int m = (int)M, n = (int)N, k = (int)K;
    if (a_fmt == 0) {
        if (out_kind == kOutBF16) launch_mx_l<0, kOutBF16>(aq, a_packed, a_scales, wq, w_packed, w_scales, y, m, n, k, stream);
        else launch_mx_l<0, kOutF32>(aq, a_packed, a_scales, wq, w_packed, w_scales, y, m, n, k, stream);
    } else {
        if (out_kind == kOutBF16) launch_mx_l<1, kOutBF16>(aq, a_packed, a_scales, wq, w_packed, w_scales, y, m, n, k, stream);
        else launch_mx_l<1, kOutF32>(aq, a_packed, a_scales, wq, w_packed, w_scales, y, m, n, k, stream);
    }
    return hipGetLastError();
}

}  // namespace fp8sg
