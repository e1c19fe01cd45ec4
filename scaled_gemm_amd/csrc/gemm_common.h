// Building blocks shared by the GEMM kernels (gemm_skinny.hip, gemm_big.hip,
// mx.hip): matrix-core fragments, epilogue stores, the LDS copy machinery and
// tile order of the large-tile kernels, and their staged epilogue.
#pragma once

#include "fp8_device.h"
#include "launch.h"

namespace fp8sg {

// Launchers of the two kernel families, called by the dispatch in gemm.hip:
// the skinny kernels (gemm_skinny.hip, M <= 32) and the large-tile kernels
// (gemm_big.hip, M > 32).  Shapes are validated by the caller.
hipError_t launch_skinny_gemm(const uint8_t* aq, bool a_packed, const float* sa, int sa_per_token, const uint8_t* wq,
                              bool w_packed, const float* sw, void* y, int out_kind, const float* out_scale, int M,
                              int N, int K, bool fp8_mfma, hipStream_t stream);
hipError_t launch_skinny_blockwise(const uint8_t* aq, bool a_packed, const float* sa, bool sa_kmajor,
                                   const uint8_t* wq, bool w_packed, const float* sw, void* y, bool y_bf16, int M,
                                   int N, int K, bool fp8_mfma, hipStream_t stream);
hipError_t launch_big_gemm(const uint8_t* aq, bool a_packed, const float* sa, int sa_per_token, const uint8_t* wq,
                           bool w_packed, const float* sw, void* y, int out_kind, const float* out_scale, int M, int N,
                           int K, bool fp8_mfma, hipStream_t stream);
hipError_t launch_big_blockwise(const uint8_t* aq, bool a_packed, const float* sa, bool sa_kmajor, const uint8_t* wq,
                                bool w_packed, const float* sw, void* y, bool y_bf16, int M, int N, int K,
                                bool fp8_mfma, hipStream_t stream);

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Frag {  // 32 FP8 bytes
    uint4 lo, hi;
};

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

// Streaming loads of packed weight blocks in the decode kernels: every weight
// byte is used once per call, so the loads carry the non-temporal hint and do
// not displace the activations that every workgroup re-reads from L2.  (On
// row-major weights the hint measured slower, so those loads do without it.)
__device__ __forceinline__ Frag load_frag_packed_stream(const uint8_t* block, int lane) {
    Frag f;
    f.lo = load16_stream(block + 16 * lane);
    f.hi = load16_stream(block + 1024 + 16 * lane);
    return f;
}

// Output kinds (kOutF32 / kOutBF16 / kOutE4M3, launch.h): for E4M3 the code of
// the fp32 result y is FMT(RN32(y / s_out)) with the given per-tensor output
// scale s_out, saturating -- the input of a next layer that takes static
// per-tensor activation scales.
template <int kOut>
__device__ __forceinline__ QScale out_qscale(const float* __restrict__ qs) {
    return make_qscale(kOut == kOutE4M3 ? qs[0] : 1.0f, kE4M3Max);
}

// Four fp32 results -> four E4M3 codes (byte r = code of v[r]).
__device__ __forceinline__ uint32_t out_codes4(float v0, float v1, float v2, float v3, const QScale& q) {
    return pack4<0>(quotient_given<true>(v0, q), quotient_given<true>(v1, q), quotient_given<true>(v2, q),
                    quotient_given<true>(v3, q));
}

// The same with the scale's range test taken once by the caller (kFast ==
// q.fast): the large-tile epilogues encode 256 values per lane.
template <bool kFast>
__device__ __forceinline__ uint32_t out_codes4_known(float v0, float v1, float v2, float v3, const QScale& q) {
    return pack4<0>(quotient_given_known<true, kFast>(v0, q), quotient_given_known<true, kFast>(v1, q),
                    quotient_given_known<true, kFast>(v2, q), quotient_given_known<true, kFast>(v3, q));
}

// Epilogue for one 16x16 fragment: lane holds acc[r] = C[n0 + r][m], r = 0..3.
// store4 applies the per-token / per-channel scales; store4_raw stores the
// values as they are (block-wise scales were applied inside the k loop).
template <int kOut>
__device__ __forceinline__ void store4_vals(void* y, int64_t N, int64_t m, int64_t n0, const float (&v)[4],
                                           bool vec_ok, const QScale& q);

template <int kOut>
__device__ __forceinline__ void store4_raw(void* y, int64_t N, int64_t m, int64_t n0, f32x4 acc, bool vec_ok,
                                           const QScale& q) {
    const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    store4_vals<kOut>(y, N, m, n0, v, vec_ok, q);
}

template <int kOut>
__device__ __forceinline__ void store4(void* y, int64_t N, int64_t m, int64_t n0, f32x4 acc, float sa,
                                       const float* __restrict__ sw, bool vec_ok, const QScale& q) {
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (n0 + r < N) ? (acc[r] * sa) * sw[n0 + r] : 0.0f;
    store4_vals<kOut>(y, N, m, n0, v, vec_ok, q);
}

template <int kOut>
__device__ __forceinline__ void store4_vals(void* y, int64_t N, int64_t m, int64_t n0, const float (&v)[4],
                                           bool vec_ok, const QScale& q) {
    if (kOut == kOutBF16) {
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
    } else if (kOut == kOutE4M3) {
        uint8_t* yr = (uint8_t*)y + m * N;
        const uint32_t c = out_codes4(v[0], v[1], v[2], v[3], q);
        if (vec_ok && n0 + 3 < N) {
            *reinterpret_cast<uint32_t*>(yr + n0) = c;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n0 + r < N) yr[n0 + r] = (uint8_t)((c >> (8 * r)) & 0xFFu);
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
// Large-tile kernels: 256 (m) x 256 (n) output tile per workgroup, k in blocks
// of 128, operands copied straight from global memory into LDS in fragment
// order.
constexpr int kBig = 256;
constexpr int kGroupM = 4;

// s_waitcnt immediate for vmcnt(n), other counters not waited on.
constexpr int wait_vmcnt(int n) {
    return 0x0F70 | (n & 15) | ((n >> 4) << 14);
}

// Per-lane offsets of the 8 one-kilobyte copies wave w issues for one 16-subtile
// operand tile per stage: copy c = 8 w + i fills half h = c % 2 of subtile
// j = c / 2.  Row-major operands: subtile row r = lane % 16 of the 16 rows at
// tile row 16 j, k bytes 32 (lane / 16) + 16 h; rows past the valid count are
// clamped to the last valid row (their results are never stored).  Packed W:
// 16-row tile j of the workgroup's tiles (clamped to the last tile), whose k
// blocks are nkb * 2048 bytes apart.  The offsets are relative to the tile's
// first row at k = 0 and fit 32 bits for K < 2^24.
template <bool kPacked>
__device__ __forceinline__ void tile_copy_offsets(uint32_t (&o)[8], int64_t base_row, int rows, int K, int wave,
                                                  int lane) {
    const int r16 = lane & 15, kq = (lane >> 4) * 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = wave * 8 + i, j = c >> 1, h = c & 1;
        if (kPacked) {
            int64_t t = (base_row >> 4) + j;
            const int64_t last_tile = ((int64_t)rows + 15) / 16 - 1;
            t = t < last_tile ? t : last_tile;
            o[i] = (uint32_t)((t - (base_row >> 4)) * (int64_t)(K >> 7) * kPackBlock + 1024 * h + 16 * lane);
        } else {
            int64_t r = base_row + 16 * j + r16;
            r = r < rows ? r : rows - 1;
            o[i] = (uint32_t)((r - base_row) * K + kq + 16 * h);
        }
    }
}

// Copy k block kb of one 16-subtile operand tile into LDS (subtile j at
// lds + 2048 j).  kb_off: kb * 128 for row-major operands, kb * 2048 for packed
// W.  Each copy is one global_load_lds_dwordx4: lane l's 16 bytes land at
// M0 + 16 l.
//
// The instruction is written out rather than left to the compiler: the compiler
// cannot tell which LDS bytes a copy writes, so it waits for every copy in
// flight before any LDS read, which would cap the pipeline at one block.  The
// kernels order copies and reads themselves: s_waitcnt vmcnt(n) for their own
// copies, then a workgroup barrier, before reading a stage; a barrier after
// the last read of a stage before copying into it; vmcnt(0) before exit.  The
// compiler issues no global loads of its own while copies are in flight.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* src, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds_addr), "v"(src)
        : "memory", "m0");
}

// The four-byte form (global_load_lds_dword): lane l's 4 bytes land at M0 + 4 l.
__device__ __forceinline__ void copy4_to_lds(const void* src, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off"
        :
        : "s"(lds_addr), "v"(src)
        : "memory", "m0");
}

__device__ __forceinline__ void issue_tile_copy(uint8_t* __restrict__ lds, const uint8_t* __restrict__ tile,
                                                int64_t kb_off, int wave, const uint32_t (&o)[8]) {
    const uint8_t* base = tile + kb_off;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = wave * 8 + i, j = c >> 1, h = c & 1;
        copy16_to_lds(base + o[i], lds_base + (uint32_t)(j * kPackBlock + h * 1024));
    }
}

// Copy i (0..15) of one stage: A copies 0..7, then W copies 8..15 (subtile
// layout as in issue_tile_copy).  The kernels spread a stage's 16 copies over
// the multiplies of a k block: a burst of copies fills the vector-memory queue,
// and with in-order issue every multiply behind it waits.
// Copies issued before rows (steps) 1..7: [kCopySplit[i - 1], kCopySplit[i]).
__device__ constexpr int kCopySplit[8] = {0, 3, 6, 8, 10, 12, 14, 16};

__device__ __forceinline__ void issue_stage_copy(int i, uint8_t* __restrict__ stage, const uint8_t* __restrict__ a_tile,
                                                 const uint8_t* __restrict__ w_tile, int64_t a_off, int64_t w_off,
                                                 int wave, const uint32_t (&oa)[8], const uint32_t (&ow)[8]) {
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)stage;
    const int k = i & 7, c = wave * 8 + k, j = c >> 1, h = c & 1;
    if (i < 8)
        copy16_to_lds(a_tile + a_off + oa[k], lds_base + (uint32_t)(j * kPackBlock + h * 1024));
    else
        copy16_to_lds(w_tile + w_off + ow[k], lds_base + (uint32_t)((16 + j) * kPackBlock + h * 1024));
}

// Tile of workgroup blockIdx.x: 256 (m) x kTileN (n) tiles, tiles_per_xcd of them
// on each of the 8 XCDs (consecutive workgroups go to consecutive XCDs).
template <int kTileN = kBig>
__device__ __forceinline__ void tile_coords(int M, int N, int tiles_per_xcd, int& tile, int64_t& m_base,
                                            int64_t& n_base) {
    const int tiles_n = (N + kTileN - 1) / kTileN;
    const int tiles = ((M + kBig - 1) / kBig) * tiles_n;
    tile = (int)(blockIdx.x & 7) * tiles_per_xcd + (int)(blockIdx.x >> 3);
    if (tile >= tiles) {
        tile = -1;
        return;
    }
    // Groups of kGroupM m tiles: within a group the tiles run m-fastest, so the
    // 32 workgroups an XCD runs at once cover 4 m tiles x 8 n tiles.
    const int tiles_m = (M + kBig - 1) / kBig;
    const int grp = kGroupM * tiles_n;
    const int first_m = (tile / grp) * kGroupM;
    const int gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
    const int t = tile % grp;
    m_base = (int64_t)(first_m + t % gm) * kBig;
    n_base = (int64_t)(t / gm) * kTileN;
}

// Workgroup barrier without a memory fence.  __syncthreads() also orders
// memory, and for that the compiler waits for every outstanding global load,
// including the LDS copies meant to stay in flight across the barrier.  The
// kernels below wait for exactly the copies they need (s_waitcnt) before
// calling this; the "memory" clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
    asm volatile("s_barrier" ::: "memory");
}

// Epilogue of the large-tile kernels for bf16 output.  A matrix-core result
// fragment gives each lane four consecutive n of one row m, so storing
// fragments directly writes 32-byte pieces of 16 different rows per
// instruction, and the write path, not the multiplies, then dominates short-K
// tiles.  Instead each wave scales and rounds its 128 x 128 share, stages it in
// LDS row-major (256 bytes per row), and stores whole 256-byte row segments:
// one instruction covers four rows.  The 16-byte column slots of a row are
// permuted by XOR with the row's low four bits, so the 16 rows one fragment
// writes fall on different banks, and a row read back is still 16 slots.
constexpr int kEpiRowBytes = 256;
constexpr int kEpiWaveBytes = 128 * kEpiRowBytes;  // 32 KB per wave, 128 KB per workgroup
static_assert(4 * kEpiWaveBytes <= 2 * 32 * kPackBlock, "the staged output reuses the two operand stages");

__device__ __forceinline__ uint32_t epi_offset(int row, int col_bytes) {
    return (uint32_t)(row * kEpiRowBytes + (col_bytes ^ ((row & 15) << 4)));
}

// Row `row`, columns col .. col + 3 (col % 4 == 0) of the wave's staged tile.
__device__ __forceinline__ void epi_put4(uint8_t* wl, int row, int col, float v0, float v1, float v2, float v3) {
    uint2 o;
    o.x = pack_bf16x2(v0, v1);
    o.y = pack_bf16x2(v2, v3);
    *reinterpret_cast<uint2*>(wl + epi_offset(row, col * 2)) = o;
}

// Store the wave's staged kRows x 128 tile to Y rows m0.., columns n0.. .
template <int kRows = 128>
__device__ __forceinline__ void epi_store(const uint8_t* wl, uint16_t* __restrict__ Y, int64_t M, int64_t N,
                                          int64_t m0, int64_t n0, int lane) {
    const int c = lane & 15;
    const int64_t n = n0 + 8 * c;
    const bool vec = (N & 7) == 0 && n + 8 <= N;
#pragma unroll 4
    for (int it = 0; it < kRows / 4; ++it) {
        const int row = 4 * it + (lane >> 4);
        const int64_t m = m0 + row;
        if (m >= M) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(wl + epi_offset(row, 16 * c));
        uint16_t* yr = Y + m * N;
        if (vec) {
            *reinterpret_cast<uint4*>(yr + n) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) yr[n + e] = (uint16_t)((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
    }
}

// The same staging for E4M3 output: 128-byte rows, the 16-byte slots of a row
// XORed with the row's low three bits; one store instruction covers eight rows.
constexpr int kEpiQRowBytes = 128;

__device__ __forceinline__ uint32_t epi_q_offset(int row, int col) {
    return (uint32_t)(row * kEpiQRowBytes + (col ^ ((row & 7) << 4)));
}

__device__ __forceinline__ void epi_put4_q(uint8_t* wl, int row, int col, uint32_t codes) {
    *reinterpret_cast<uint32_t*>(wl + epi_q_offset(row, col)) = codes;
}

template <int kRows>
__device__ __forceinline__ void epi_store_q(const uint8_t* wl, uint8_t* __restrict__ Y, int64_t M, int64_t N,
                                            int64_t m0, int64_t n0, int lane) {
    const int c = lane & 7;
    const int64_t n = n0 + 16 * c;
    const bool vec = (N & 15) == 0 && n + 16 <= N;
#pragma unroll 4
    for (int it = 0; it < kRows / 8; ++it) {
        const int row = 8 * it + (lane >> 3);
        const int64_t m = m0 + row;
        if (m >= M) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(wl + epi_q_offset(row, 16 * c));
        uint8_t* yr = Y + m * N;
        if (vec) {
            *reinterpret_cast<uint4*>(yr + n) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (n + e < N) yr[n + e] = (uint8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
        }
    }
}

// The four per-channel scales of columns n0 .. n0 + 3 (0 past N).
__device__ __forceinline__ void load_sw4(const float* __restrict__ sw, int64_t N, int64_t n0, float (&v)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = n0 + r < N ? sw[n0 + r] : 0.0f;
}

}  // namespace fp8sg
