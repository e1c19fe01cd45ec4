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
//  * Exact mode: the bytes are widened exactly to bf16 (every E4M3 value is a
//    bf16 value) and fed to the bf16 matrix cores: four v_mfma_f32_16x16x32_bf16
//    per 16x16 tile (bytes 8s..8s+7 to step s) in the small-M kernels, and
//    v_mfma_f32_32x32x16_bf16 in the large-tile kernel (lane layout described
//    there).  The bf16 matrix cores form these products exactly and add them at
//    fp32 precision, whereas the FP8 matrix cores align each group of 8
//    products to the group's largest one and drop bits below 2^(e_max - 13).
#include "gemm_common.h"

#ifndef SKINNY_NS
#define SKINNY_NS 2
#endif
#ifndef SKINNY_KS
#define SKINNY_KS 4
#endif
#ifndef SKINNY_DEPTH
#define SKINNY_DEPTH 1
#endif

namespace fp8sg {

// ---------------------------------------------------------------------------
// Skinny GEMM (M <= 16 * kMT), the decode shape: every byte of W is used once,
// so W streams from HBM straight into registers.  Every workgroup reads all of
// A (from L2); in the fragment order (kAPacked) each fragment half is one
// contiguous kilobyte instead of 64-byte pieces of 16 rows, which halves the
// cache lines touched per load.  A workgroup owns kNS 16-row
// subtiles of W; its kKS waves split the k blocks round-robin (wave w takes
// blocks w, w + kKS, ...).  With kDepth = 1 the loop is software-pipelined: the
// loads of a wave's next block are issued before its current block is
// multiplied.  Otherwise (and for block-wise scales) each wave issues the loads
// of kDepth of its blocks back to back, then multiplies them.  The loop bodies
// have no branches around loads (rows past M or N are clamped to the last valid
// row and masked in the epilogue), which lets the compiler wait for each
// block's loads separately.  The kKS partial sums
// are added in a fixed order through LDS, so the result does not depend on
// timing.
//
// kBlock: block-wise scales, sa [M, K / 128] and sw [ceil(N / 128), K / 128].
// Each k block's 16 x 16 partial products start from zero, are multiplied by
// s_a[m, kb] * s_w[n / 128, kb] and added to the fp32 accumulator, so the
// epilogue only rounds.  A 16-row subtile never straddles a 128-row block.
template <bool kFp8, int kOut, int kMT, int kNS, int kKS, int kDepth, bool kWPacked, bool kAPacked,
          bool kBlock = false>
__global__ __launch_bounds__(64 * kKS) void gemm_skinny(const uint8_t* __restrict__ A, const float* __restrict__ sa,
                                                        int sa_per_token, const uint8_t* __restrict__ W,
                                                        const float* __restrict__ sw, void* __restrict__ Y, int M,
                                                        int N, int K, const float* __restrict__ qs) {
    // Software pipelining pays in exact mode (M = 32: 15.0 -> 14.3 us at N = 14336,
    // K = 4096) and is neutral for one m-tile; FP8 mode with two m-tiles is 3% slower
    // with it, so that case keeps the plain loop.
    constexpr bool kPipe = !kBlock && kDepth == 1 && !(kFp8 && kMT > 1);
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
    // row-major: this lane's row of each m-tile; packed: the m-tile's first block
    const uint8_t* arow[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
        if (kAPacked) {
            arow[t] = A + (int64_t)t * nkb * kPackBlock;
        } else {
            int m = 16 * t + r16;
            m = m < M ? m : M - 1;
            arow[t] = A + (int64_t)m * K + kofs;
        }
    }

    f32x4 acc[kNS][kMT];
#pragma unroll
    for (int s = 0; s < kNS; ++s)
#pragma unroll
        for (int t = 0; t < kMT; ++t) acc[s][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // block-wise scales: this lane's rows of s_a and the subtiles' rows of s_w
    const float* sa_row[kMT];
    const float* sw_row[kNS];
    if (kBlock) {
#pragma unroll
        for (int t = 0; t < kMT; ++t) {
            const int m = 16 * t + r16 < M ? 16 * t + r16 : M - 1;
            sa_row[t] = sa + (int64_t)m * nkb;
        }
#pragma unroll
        for (int s = 0; s < kNS; ++s) {
            const int64_t n = n_base + 16 * s < N ? n_base + 16 * s : N - 1;
            sw_row[s] = sw + (n >> 7) * nkb;
        }
    }

    // this wave's blocks: wave + j * kKS, j < nper
    const int nper = nkb > wave ? (nkb - wave + kKS - 1) / kKS : 0;
    if constexpr (kPipe) {
        // One block in registers while the next block's loads are in flight.  The
        // scheduling barriers keep the compiler from sinking those loads below the
        // multiplies (it otherwise issues them at the end of the loop body, which
        // serialises load latency and matrix work again).
        auto load_block = [&](int j, Frag (&wx)[kNS], Frag (&ax)[kMT]) {
            const int kb = wave + j * kKS;
            const int64_t off = (int64_t)kb << 7;
#pragma unroll
            for (int s = 0; s < kNS; ++s)
                wx[s] = kWPacked ? load_frag_packed_stream(wrow[s] + kb * kPackBlock, lane)
                                  : load_frag_global(wrow[s] + off);
#pragma unroll
            for (int t = 0; t < kMT; ++t)
                ax[t] = kAPacked ? load_frag_packed(arow[t] + kb * kPackBlock, lane) : load_frag_global(arow[t] + off);
        };
        auto mul_block = [&](const Frag (&wx)[kNS], const Frag (&ax)[kMT]) {
#pragma unroll
            for (int s = 0; s < kNS; ++s)
#pragma unroll
                for (int t = 0; t < kMT; ++t) acc[s][t] = mma<kFp8>(wx[s], ax[t], acc[s][t]);
        };
        if (nper > 0) {
            Frag wf[kNS], af[kMT];
            load_block(0, wf, af);
            for (int j = 0; j + 1 < nper; ++j) {
                Frag wn[kNS], an[kMT];
                load_block(j + 1, wn, an);
                __builtin_amdgcn_sched_barrier(0);
                mul_block(wf, af);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < kNS; ++s) wf[s] = wn[s];
#pragma unroll
                for (int t = 0; t < kMT; ++t) af[t] = an[t];
            }
            mul_block(wf, af);
        }
    } else {
        for (int j0 = 0; j0 < nper; j0 += kDepth) {
            Frag wf[kDepth][kNS], af[kDepth][kMT];
            float fa[kDepth][kMT], fw[kDepth][kNS];
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                int j = j0 + d;
                j = j < nper ? j : nper - 1;  // a clamped (repeated) block past the end is loaded but not used
                const int kb = wave + j * kKS;
                const int64_t off = (int64_t)kb << 7;
#pragma unroll
                for (int s = 0; s < kNS; ++s)
                    wf[d][s] = kWPacked ? load_frag_packed_stream(wrow[s] + kb * kPackBlock, lane)
                                        : load_frag_global(wrow[s] + off);
#pragma unroll
                for (int t = 0; t < kMT; ++t)
                    af[d][t] = kAPacked ? load_frag_packed(arow[t] + kb * kPackBlock, lane)
                                        : load_frag_global(arow[t] + off);
                if (kBlock) {
#pragma unroll
                    for (int t = 0; t < kMT; ++t) fa[d][t] = sa_row[t][kb];
#pragma unroll
                    for (int s = 0; s < kNS; ++s) fw[d][s] = sw_row[s][kb];
                }
            }
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                if (j0 + d < nper) {
#pragma unroll
                    for (int s = 0; s < kNS; ++s)
#pragma unroll
                        for (int t = 0; t < kMT; ++t) {
                            if (kBlock) {
                                const f32x4 p = mma<kFp8>(wf[d][s], af[d][t], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
                                const float f = fa[d][t] * fw[d][s];
#pragma unroll
                                for (int r = 0; r < 4; ++r) acc[s][t][r] = __builtin_fmaf(p[r], f, acc[s][t][r]);
                            } else {
                                acc[s][t] = mma<kFp8>(wf[d][s], af[d][t], acc[s][t]);
                            }
                        }
                }
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
        const QScale q = out_qscale<kOut>(qs);
#pragma unroll
        for (int s = 0; s < kNS; ++s)
#pragma unroll
            for (int t = 0; t < kMT; ++t) {
                f32x4 v = acc[s][t];
#pragma unroll
                for (int w = 0; w < kKS - 1; ++w) v += red[w][s * kMT + t][lane];
                const int m = 16 * t + r16;
                const int64_t n0 = n_base + 16 * s + 4 * (lane >> 4);
                if (m < M && n0 < N) {
                    if (kBlock) store4_raw<kOut>(Y, N, m, n0, v, vec_ok, q);
                    else store4<kOut>(Y, N, m, n0, v, sa[sa_per_token ? m : 0], sw, vec_ok, q);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Large tiled GEMMs: 256 (m) x 256 (n) output tile per workgroup, 4 waves in a
// 2 x 2 arrangement of 128 x 128, k in blocks of 128.
//
// Operands reach LDS by direct copies from global memory
// (global_load_lds_dwordx4, no register staging) in matrix-core fragment order:
// the 16-row x 128-k block of each subtile occupies 2 KB, the 64 lanes' first
// 16-byte halves and then their second halves, so every fragment read is a
// lane-contiguous 1 KB ds_read per half, free of bank conflicts.  Two LDS
// stages: the copy of block kb + 1 is in flight while block kb is multiplied.
//
// Workgroups are dealt to the 8 XCDs round-robin; the tile order gives XCD x a
// contiguous range of tiles, so the workgroups sharing an XCD's L2 share A rows
// and W columns.  Tiles are ordered in groups of kGroupM m tiles (m fastest
// within a group): the 32 tiles an XCD holds at once then span 4 m x 8 n tiles,
// 384 KB of distinct operand bytes per k block instead of 576 KB for 2 x 16.
// The copy machinery, tile order and epilogue staging are in gemm_common.h.

// FP8 mode.  Each wave's 128 x 128 share takes 8 x 8 v_mfma_f32_16x16x128_f8f6f4
// per k block, with all 256 accumulator registers.  Both operand tiles go
// through LDS (each W subtile serves the two waves of its column, each A
// subtile the two waves of its row), so each byte crosses L2 once per
// workgroup.
//
// The copies run two k blocks ahead in two 64 KB stages: once every wave holds
// block kb's fragments in registers (second barrier), block kb + 2 is copied
// into the stage they came from while block kb is multiplied.  At the top of
// step kb the wave waits for its copies of block kb only (vmcnt(16): the 16
// copies of block kb + 1 stay in flight).  Past the last block the copies
// repeat block nkb - 1, so the loop body has no branch.
template <int kOut, bool kWPacked, bool kAPacked>
__global__ __launch_bounds__(256, 1) void gemm_big_fp8(const uint8_t* __restrict__ A, const float* __restrict__ sa,
                                                       int sa_per_token, const uint8_t* __restrict__ W,
                                                       const float* __restrict__ sw, void* __restrict__ Y, int M,
                                                       int N, int K, int tiles_per_xcd, const float* __restrict__ qs) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // 2 stages x (A 32 KB + W 32 KB)
    constexpr int kStage = 32 * kPackBlock;
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
    tile_copy_offsets<kAPacked>(oa, m_base, M, K, wave, lane);
    tile_copy_offsets<kWPacked>(ow, n_base, N, K, wave, lane);
    const uint8_t* a_tile = kAPacked ? A + (m_base >> 4) * (int64_t)nkb * kPackBlock : A + m_base * K;
    const uint8_t* w_tile = kWPacked ? W + (n_base >> 4) * (int64_t)nkb * kPackBlock : W + n_base * K;
    const int64_t a_kb = kAPacked ? kPackBlock : 128;
    const int64_t w_kb = kWPacked ? kPackBlock : 128;

    if (nkb > 0) {
        const int b1 = nkb > 1 ? 1 : 0;
        issue_tile_copy(smem, a_tile, 0, wave, oa);
        issue_tile_copy(smem + 16 * kPackBlock, w_tile, 0, wave, ow);
        issue_tile_copy(smem + kStage, a_tile, (int64_t)b1 * a_kb, wave, oa);
        issue_tile_copy(smem + kStage + 16 * kPackBlock, w_tile, (int64_t)b1 * w_kb, wave, ow);
    }
    for (int kb = 0; kb < nkb; ++kb) {
        uint8_t* cur = smem + (kb & 1) * kStage;
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));  // this wave's copies of block kb have landed
        barrier_no_fence();                           // ... and every other wave's
        const uint8_t* la = cur + wm * 8 * kPackBlock;
        const uint8_t* lw = cur + (16 + wn * 8) * kPackBlock;
        Frag wf[8], af[8];
        // A fragments first: the first row of multiplies needs all of them and W fragment 0
#pragma unroll
        for (int j = 0; j < 8; ++j) af[j] = load_frag_packed(la + j * kPackBlock, lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) wf[i] = load_frag_packed(lw + i * kPackBlock, lane);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[0][j] = mma_fp8(wf[0], af[j], acc[0][j]);
        __builtin_amdgcn_sched_barrier(0);   // the first row of multiplies overlaps the remaining reads
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): all of this wave's fragment reads are done
        barrier_no_fence();                  // ... and every other wave's: the stage may be refilled
        const int n = kb + 2 < nkb ? kb + 2 : nkb - 1;
        const int64_t a_off = (int64_t)n * a_kb, w_off = (int64_t)n * w_kb;
        // Rows 1..7 of the multiplies, with the 16 copies of block kb + 2 spread
        // between them (3, 3, 2, 2, 2, 2, 2 before rows 1..7).
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            const int c0 = kCopySplit[i - 1], c1 = kCopySplit[i];
#pragma unroll
            for (int c = c0; c < c1; ++c) issue_stage_copy(c, cur, a_tile, w_tile, a_off, w_off, wave, oa, ow);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = mma_fp8(wf[i], af[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // no copy into LDS may outlive the workgroup

    if (kOut == kOutBF16 || kOut == kOutE4M3) {
        __syncthreads();  // every wave is done with the stages: the LDS now holds the output tiles
        uint8_t* wl = smem + wave * kEpiWaveBytes;
        const QScale q = out_qscale<kOut>(qs);
        float sam[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int64_t m = m_base + wm * 128 + 16 * j + (lane & 15);
            m = m < M ? m : M - 1;
            sam[j] = sa[sa_per_token ? m : 0];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float s4[4];
            load_sw4(sw, N, n_base + wn * 128 + 16 * i + 4 * (lane >> 4), s4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const f32x4 a = acc[i][j];
                const int row = 16 * j + (lane & 15), col = 16 * i + 4 * (lane >> 4);
                const float v0 = (a[0] * sam[j]) * s4[0], v1 = (a[1] * sam[j]) * s4[1];
                const float v2 = (a[2] * sam[j]) * s4[2], v3 = (a[3] * sam[j]) * s4[3];
                if (kOut == kOutBF16) epi_put4(wl, row, col, v0, v1, v2, v3);
                else epi_put4_q(wl, row, col, out_codes4(v0, v1, v2, v3, q));
            }
        }
        __syncthreads();
        if (kOut == kOutBF16) epi_store(wl, (uint16_t*)Y, M, N, m_base + wm * 128, n_base + wn * 128, lane);
        else epi_store_q<128>(wl, (uint8_t*)Y, M, N, m_base + wm * 128, n_base + wn * 128, lane);
        return;
    }
    const bool vec_ok = (N & 3) == 0;
    const QScale q = out_qscale<kOut>(qs);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t m = m_base + wm * 128 + 16 * j + (lane & 15);
        if (m >= M) continue;
        const float sam = sa[sa_per_token ? m : 0];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t n0 = n_base + wn * 128 + 16 * i + 4 * (lane >> 4);
            if (n0 < N) store4<kOut>(Y, N, m, n0, acc[i][j], sam, sw, vec_ok, q);
        }
    }
}

// Exact mode.  The FP8 codes are widened to bf16 (exact) and multiplied by
// v_mfma_f32_32x32x16_bf16: each wave's 128 x 128 share is 4 x 4 tiles of
// 32 x 32, 8 steps of 16 k per k block.  Staging and copy schedule as in FP8
// mode: two stages, copies two blocks ahead, each stage refilled as soon as
// every wave holds its bytes in registers.
//
// Operand lane layout of the 32 x 32 x 16 instruction: lane l supplies row
// l % 32 and k 8 (l / 32) .. 8 (l / 32) + 7 of the step.  Step s of a k block
// gives lane l the 8 bytes at offset 8 (s % 4) of the row's 32-byte slice
// q = 2 (l / 32) + s / 4, i.e. exactly the bytes that lane (l % 16) + 16 q of the
// row's 16-row subtile holds in the 16 x 16 fragment order of LDS; A and W use
// the same assignment, so every product pairs matching k.  Output lane layout:
// acc[r] of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] of the tile.
template <int kOut, bool kWPacked, bool kAPacked>
__global__ __launch_bounds__(256, 1) void gemm_big_exact(const uint8_t* __restrict__ A, const float* __restrict__ sa,
                                                         int sa_per_token, const uint8_t* __restrict__ W,
                                                         const float* __restrict__ sw, void* __restrict__ Y, int M,
                                                         int N, int K, int tiles_per_xcd,
                                                         const float* __restrict__ qs) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // 2 stages x (A 32 KB + W 32 KB)
    constexpr int kStage = 32 * kPackBlock;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    int tile;
    int64_t m_base, n_base;
    tile_coords(M, N, tiles_per_xcd, tile, m_base, n_base);
    if (tile < 0) return;
    const int nkb = K >> 7;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    uint32_t oa[8], ow[8];
    tile_copy_offsets<kAPacked>(oa, m_base, M, K, wave, lane);
    tile_copy_offsets<kWPacked>(ow, n_base, N, K, wave, lane);
    const uint8_t* a_tile = kAPacked ? A + (m_base >> 4) * (int64_t)nkb * kPackBlock : A + m_base * K;
    const uint8_t* w_tile = kWPacked ? W + (n_base >> 4) * (int64_t)nkb * kPackBlock : W + n_base * K;
    const int64_t a_kb = kAPacked ? kPackBlock : 128;
    const int64_t w_kb = kWPacked ? kPackBlock : 128;

    // Byte offset of this lane's first 16-byte half of slice q = 2 (lane / 32)
    // within a 32-row tile: subtile (lane % 32) / 16, row lane % 16.
    const int lane_off = ((lane & 31) >> 4) * (int)kPackBlock + (lane & 15) * 16 + (lane >> 5) * 512;

    if (nkb > 0) {
        const int b1 = nkb > 1 ? 1 : 0;
        issue_tile_copy(smem, a_tile, 0, wave, oa);
        issue_tile_copy(smem + 16 * kPackBlock, w_tile, 0, wave, ow);
        issue_tile_copy(smem + kStage, a_tile, (int64_t)b1 * a_kb, wave, oa);
        issue_tile_copy(smem + kStage + 16 * kPackBlock, w_tile, (int64_t)b1 * w_kb, wave, ow);
    }
    for (int kb = 0; kb < nkb; ++kb) {
        uint8_t* cur = smem + (kb & 1) * kStage;
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));  // this wave's copies of block kb have landed
        barrier_no_fence();                           // ... and every other wave's
        const uint8_t* la = cur + wm * 8 * kPackBlock + lane_off;
        const uint8_t* lw = cur + (16 + wn * 8) * kPackBlock + lane_off;
        // raw[g][t][half]: slice q = 2 (lane / 32) + g of tile t (W tiles 0..3, A tiles 4..7)
        uint4 raw[2][8][2];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint8_t* p = (t < 4 ? lw + 2 * t * kPackBlock : la + 2 * (t - 4) * kPackBlock) + g * 256;
                raw[g][t][0] = *reinterpret_cast<const uint4*>(p);
                raw[g][t][1] = *reinterpret_cast<const uint4*>(p + 1024);
            }
        auto step = [&](int g, int s4) __attribute__((always_inline)) {
            bf16x8 v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint4 r = raw[g][t][s4 >> 1];
                v[t] = (s4 & 1) ? widen8(r.z, r.w) : widen8(r.x, r.y);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[i], v[4 + j], acc[i][j], 0, 0, 0);
        };
        step(0, 0);
        __builtin_amdgcn_sched_barrier(0);   // the first step overlaps the remaining reads
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): all of this wave's reads are done
        barrier_no_fence();                  // ... and every other wave's: the stage may be refilled
        const int n = kb + 2 < nkb ? kb + 2 : nkb - 1;
        const int64_t a_off = (int64_t)n * a_kb, w_off = (int64_t)n * w_kb;
        // Steps 1..7, with the 16 copies of block kb + 2 spread between them
        // (3, 3, 2, 2, 2, 2, 2 before steps 1..7).
#pragma unroll
        for (int st = 1; st < 8; ++st) {
            const int c0 = kCopySplit[st - 1], c1 = kCopySplit[st];
#pragma unroll
            for (int c = c0; c < c1; ++c) issue_stage_copy(c, cur, a_tile, w_tile, a_off, w_off, wave, oa, ow);
            __builtin_amdgcn_sched_barrier(0);
            step(st >> 2, st & 3);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // no copy into LDS may outlive the workgroup

    if (kOut == kOutBF16 || kOut == kOutE4M3) {
        __syncthreads();  // every wave is done with the stages: the LDS now holds the output tiles
        uint8_t* wl = smem + wave * kEpiWaveBytes;
        const QScale q = out_qscale<kOut>(qs);
        float sam[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t m = m_base + wm * 128 + 32 * j + (lane & 31);
            m = m < M ? m : M - 1;
            sam[j] = sa[sa_per_token ? m : 0];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * i + 8 * g + 4 * (lane >> 5);
                float s4[4];
                load_sw4(sw, N, n_base + wn * 128 + col, s4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x16 a = acc[i][j];
                    const int row = 32 * j + (lane & 31);
                    const float v0 = (a[4 * g] * sam[j]) * s4[0], v1 = (a[4 * g + 1] * sam[j]) * s4[1];
                    const float v2 = (a[4 * g + 2] * sam[j]) * s4[2], v3 = (a[4 * g + 3] * sam[j]) * s4[3];
                    if (kOut == kOutBF16) epi_put4(wl, row, col, v0, v1, v2, v3);
                    else epi_put4_q(wl, row, col, out_codes4(v0, v1, v2, v3, q));
                }
            }
        __syncthreads();
        if (kOut == kOutBF16) epi_store(wl, (uint16_t*)Y, M, N, m_base + wm * 128, n_base + wn * 128, lane);
        else epi_store_q<128>(wl, (uint8_t*)Y, M, N, m_base + wm * 128, n_base + wn * 128, lane);
        return;
    }
    const bool vec_ok = (N & 3) == 0;
    const QScale q = out_qscale<kOut>(qs);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m_base + wm * 128 + 32 * j + (lane & 31);
        if (m >= M) continue;
        const float sam = sa[sa_per_token ? m : 0];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t n0 = n_base + wn * 128 + 32 * i + 8 * g + 4 * (lane >> 5);
                const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                if (n0 < N) store4<kOut>(Y, N, m, n0, v, sam, sw, vec_ok, q);
            }
    }
}

// ---------------------------------------------------------------------------
// Block-wise scaled GEMM for M > 32 on the FP8 matrix cores:
//   y[m, n] = sum_kb s_a[m, kb] * s_w[n / 128, kb] * P_kb[m, n],
// with P_kb the 128-deep partial product of k block kb (FP8 Inference
// Explained, in depth -- "Inside a quantized linear layer": scales that vary
// along k cannot leave the sum; Quantization: FP8 inference and KV-cache
// quantization -- "Training in FP8 or lower": each 128-element partial sum
// moves to fp32 with its scales).  A k block is exactly one
// v_mfma_f32_16x16x128_f8f6f4 per 16 x 16 fragment, started from zero; the
// result is multiplied by the fragment's scale product and added to an fp32
// accumulator with vector FMAs, so the accumulators live in the vector
// registers the FMAs can address.
//
// 256 x 256 tile per workgroup of 8 waves (two per SIMD).  Wave (wm, wn) =
// (wave % 4, wave / 4) owns tile rows 64 wm .. 64 wm + 63 and columns
// 128 wn .. 128 wn + 127: 4 A fragments x 8 W fragments, 128 accumulator
// registers.  It holds its 4 A fragments and streams the 8 W fragments from
// LDS two at a time, which keeps the wave within 256 registers.
//
// Staging as in the per-token kernels (direct global-to-LDS copies in fragment
// order, two stages, copies two k blocks ahead, fence-free barriers), with
// the copies split by operand: waves 0-3 copy the A tile, waves 4-7 the W
// tile, 8 one-kilobyte copies each.  Each wave also copies one 4-byte value
// per lane of the block's scales: waves 0-3 the s_a of tile rows 64 w + lane,
// waves 4-7 the s_w of the tile's two 128-column blocks (lane % 2), so every
// wave has 9 copies per stage.  A stage is refilled once every wave has read
// all of it (the W fragments are read until the last row of multiplies).
constexpr int kBwOps = 32 * kPackBlock;       // A 32 KB + W 32 KB
constexpr int kBwStage = kBwOps + 2048;       // + s_a (256 floats) + s_w (4 x 64 floats)
constexpr int kBwCopies = 9;                  // copies per wave per stage

template <int kOut, bool kWPacked, bool kAPacked>
__global__ __launch_bounds__(512, 1) void gemm_big_blockwise(const uint8_t* __restrict__ A,
                                                             const float* __restrict__ sa,
                                                             const uint8_t* __restrict__ W,
                                                             const float* __restrict__ sw, void* __restrict__ Y,
                                                             int M, int N, int K, int tiles_per_xcd,
                                                             const float* __restrict__ qs) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // 2 stages of kBwStage
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    int tile;
    int64_t m_base, n_base;
    tile_coords(M, N, tiles_per_xcd, tile, m_base, n_base);
    if (tile < 0) return;
    const int nkb = K >> 7;
    const int64_t nbw = ((int64_t)N + 127) >> 7;

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // this wave's copies: 8 kilobytes of one operand tile and 256 bytes of scales
    const bool cp_a = wave < 4;
    uint32_t o[8];
    if (cp_a) tile_copy_offsets<kAPacked>(o, m_base, M, K, wave & 3, lane);
    else tile_copy_offsets<kWPacked>(o, n_base, N, K, wave & 3, lane);
    const uint8_t* src = cp_a ? (kAPacked ? A + (m_base >> 4) * (int64_t)nkb * kPackBlock : A + m_base * K)
                              : (kWPacked ? W + (n_base >> 4) * (int64_t)nkb * kPackBlock : W + n_base * K);
    const int64_t src_kb = cp_a ? (kAPacked ? kPackBlock : 128) : (kWPacked ? kPackBlock : 128);
    const uint32_t dst_op = cp_a ? 0u : (uint32_t)(16 * kPackBlock);
    const float* ssrc;
    if (cp_a) {
        int64_t m = m_base + 64 * wave + lane;
        m = m < M ? m : M - 1;
        ssrc = sa + m * nkb;
    } else {
        int64_t nb = (n_base >> 7) + (lane & 1);
        nb = nb < nbw ? nb : nbw - 1;
        ssrc = sw + nb * nkb;
    }
    const uint32_t dst_sc = (uint32_t)(kBwOps + 256 * wave);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

    // copy c (0..8) of block kb into the stage at LDS address `stage`
    auto issue_copy = [&](int c, uint32_t stage, int kb) __attribute__((always_inline)) {
        if (c < 8) {
            const int q = (wave & 3) * 8 + c, j = q >> 1, h = q & 1;
            copy16_to_lds(src + (int64_t)kb * src_kb + o[c], stage + dst_op + (uint32_t)(j * kPackBlock + h * 1024));
        } else {
            copy4_to_lds(ssrc + kb, stage + dst_sc);
        }
    };

    if (nkb > 0) {
        const int b1 = nkb > 1 ? 1 : 0;
#pragma unroll
        for (int c = 0; c < kBwCopies; ++c) issue_copy(c, lds0, 0);
#pragma unroll
        for (int c = 0; c < kBwCopies; ++c) issue_copy(c, lds0 + kBwStage, b1);
    }
    for (int kb = 0; kb < nkb; ++kb) {
        const uint32_t cur_lds = lds0 + (uint32_t)((kb & 1) * kBwStage);
        const uint8_t* cur = smem + (kb & 1) * kBwStage;
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(kBwCopies));  // this wave's copies of block kb have landed
        barrier_no_fence();                                 // ... and every other wave's
        const float* ls = reinterpret_cast<const float*>(cur + kBwOps);
        const float swv = ls[256 + wn];
        float f[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = ls[64 * wm + 16 * j + (lane & 15)] * swv;
        Frag af[4], wf[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = load_frag_packed(cur + (4 * wm + j) * kPackBlock, lane);
        const uint8_t* lw = cur + (16 + 8 * wn) * kPackBlock;
        wf[0] = load_frag_packed(lw, lane);
        const int nxt = kb + 2 < nkb ? kb + 2 : nkb - 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < 7) {
                wf[(i + 1) & 1] = load_frag_packed(lw + (i + 1) * kPackBlock, lane);
            } else {
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of the stage are done
                barrier_no_fence();                  // ... and every other wave's: refill it with block kb + 2
#pragma unroll
                for (int c = 0; c < kBwCopies; ++c) issue_copy(c, cur_lds, nxt);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 p = mma_fp8(wf[i & 1], af[j], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], f[j], acc[i][j][r]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // no copy into LDS may outlive the workgroup

    static_assert(kOut != kOutE4M3, "block-wise GEMMs write bf16 or fp32");
    const QScale q = out_qscale<kOut>(qs);
    if (kOut == kOutBF16) {
        __syncthreads();  // every wave is done with the stages: the LDS now holds the output tiles
        uint8_t* wl = smem + wave * (kEpiWaveBytes / 2);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 a = acc[i][j];
                epi_put4(wl, 16 * j + (lane & 15), 16 * i + 4 * (lane >> 4), a[0], a[1], a[2], a[3]);
            }
        __syncthreads();
        epi_store<64>(wl, (uint16_t*)Y, M, N, m_base + wm * 64, n_base + wn * 128, lane);
        return;
    }
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m_base + wm * 64 + 16 * j + (lane & 15);
        if (m >= M) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t n0 = n_base + wn * 128 + 16 * i + 4 * (lane >> 4);
            if (n0 < N) store4_raw<kOut>(Y, N, m, n0, acc[i][j], vec_ok, q);
        }
    }
}
static_assert(8 * (kEpiWaveBytes / 2) <= 2 * kBwStage, "the staged output reuses the two operand stages");

template <bool kFp8, int kOut, bool kWPacked, bool kAPacked, int kMT, int kNS, int kKS, int kDepth>
static void launch_skinny(const uint8_t* aq, const float* sa, int sa_pt, const uint8_t* wq, const float* sw, void* y,
                          int M, int N, int K, const float* qs, hipStream_t stream) {
    dim3 grid((unsigned)((N + 16 * kNS - 1) / (16 * kNS))), block(64 * kKS);
    gemm_skinny<kFp8, kOut, kMT, kNS, kKS, kDepth, kWPacked, kAPacked>
        <<<grid, block, 0, stream>>>(aq, sa, sa_pt, wq, sw, y, M, N, K, qs);
}

template <bool kFp8, int kOut, bool kWPacked, bool kAPacked>
static hipError_t launch_gemm_t(const uint8_t* aq, const float* sa, int sa_pt, const uint8_t* wq, const float* sw,
                                void* y, int M, int N, int K, const float* qs, hipStream_t stream) {
    if (M <= 16) {
        launch_skinny<kFp8, kOut, kWPacked, kAPacked, 1, SKINNY_NS, SKINNY_KS, SKINNY_DEPTH>(aq, sa, sa_pt, wq, sw, y,
                                                                                             M, N, K, qs, stream);
    } else if (M <= 32) {
        launch_skinny<kFp8, kOut, kWPacked, kAPacked, 2, SKINNY_NS, SKINNY_KS, SKINNY_DEPTH>(aq, sa, sa_pt, wq, sw, y,
                                                                                             M, N, K, qs, stream);
    } else {
        const int tiles = ((M + kBig - 1) / kBig) * ((N + kBig - 1) / kBig);
        const int per = (tiles + 7) / 8;
        dim3 grid((unsigned)(per * 8)), block(256);
        if (kFp8)
            gemm_big_fp8<kOut, kWPacked, kAPacked>
                <<<grid, block, 2 * 32 * kPackBlock, stream>>>(aq, sa, sa_pt, wq, sw, y, M, N, K, per, qs);
        else
            gemm_big_exact<kOut, kWPacked, kAPacked>
                <<<grid, block, 2 * 32 * kPackBlock, stream>>>(aq, sa, sa_pt, wq, sw, y, M, N, K, per, qs);
    }
    return hipGetLastError();
}

template <bool kFp8, bool kWPacked, bool kAPacked>
static hipError_t launch_gemm_y(const uint8_t* aq, const float* sa, int pt, const uint8_t* wq, const float* sw, void* y,
                                int out_kind, int M, int N, int K, const float* qs, hipStream_t stream) {
    if (out_kind == kOutBF16)
        return launch_gemm_t<kFp8, kOutBF16, kWPacked, kAPacked>(aq, sa, pt, wq, sw, y, M, N, K, qs, stream);
    if (out_kind == kOutE4M3)
        return launch_gemm_t<kFp8, kOutE4M3, kWPacked, kAPacked>(aq, sa, pt, wq, sw, y, M, N, K, qs, stream);
    return launch_gemm_t<kFp8, kOutF32, kWPacked, kAPacked>(aq, sa, pt, wq, sw, y, M, N, K, qs, stream);
}

template <bool kFp8>
static hipError_t launch_gemm_m(const uint8_t* aq, bool a_packed, const float* sa, int pt, const uint8_t* wq,
                                bool w_packed, const float* sw, void* y, int out_kind, int M, int N, int K,
                                const float* qs, hipStream_t stream) {
    if (a_packed)
        return w_packed ? launch_gemm_y<kFp8, true, true>(aq, sa, pt, wq, sw, y, out_kind, M, N, K, qs, stream)
                        : launch_gemm_y<kFp8, false, true>(aq, sa, pt, wq, sw, y, out_kind, M, N, K, qs, stream);
    return w_packed ? launch_gemm_y<kFp8, true, false>(aq, sa, pt, wq, sw, y, out_kind, M, N, K, qs, stream)
                    : launch_gemm_y<kFp8, false, false>(aq, sa, pt, wq, sw, y, out_kind, M, N, K, qs, stream);
}

hipError_t launch_gemm(const uint8_t* aq, bool a_packed, const float* a_scales, bool a_per_token, const uint8_t* wq,
                       bool w_packed, const float* w_scales, void* y, int out_kind, const float* out_scale, int64_t M,
                       int64_t N, int64_t K, bool fp8_mfma, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const int pt = a_per_token ? 1 : 0;
    const int m = (int)M, n = (int)N, k = (int)K;
    if (fp8_mfma)
        return launch_gemm_m<true>(aq, a_packed, a_scales, pt, wq, w_packed, w_scales, y, out_kind, m, n, k, out_scale,
                                   stream);
    return launch_gemm_m<false>(aq, a_packed, a_scales, pt, wq, w_packed, w_scales, y, out_kind, m, n, k, out_scale,
                                stream);
}

template <bool kFp8, int kOut, bool kWPacked, bool kAPacked>
static hipError_t launch_blockwise_t(const uint8_t* aq, const float* sa, const uint8_t* wq, const float* sw, void* y,
                                     int M, int N, int K, hipStream_t stream) {
    dim3 block(64 * SKINNY_KS);
    dim3 grid((unsigned)((N + 16 * SKINNY_NS - 1) / (16 * SKINNY_NS)));
    if (M <= 16) {
        gemm_skinny<kFp8, kOut, 1, SKINNY_NS, SKINNY_KS, SKINNY_DEPTH, kWPacked, kAPacked, true>
            <<<grid, block, 0, stream>>>(aq, sa, 1, wq, sw, y, M, N, K, nullptr);
    } else if (M <= 32) {
        gemm_skinny<kFp8, kOut, 2, SKINNY_NS, SKINNY_KS, SKINNY_DEPTH, kWPacked, kAPacked, true>
            <<<grid, block, 0, stream>>>(aq, sa, 1, wq, sw, y, M, N, K, nullptr);
    } else if (kFp8) {
        const int tiles = ((M + kBig - 1) / kBig) * ((N + kBig - 1) / kBig);
        const int per = (tiles + 7) / 8;
        gemm_big_blockwise<kOut, kWPacked, kAPacked>
            <<<dim3((unsigned)(per * 8)), dim3(512), 2 * kBwStage, stream>>>(aq, sa, wq, sw, y, M, N, K, per, nullptr);
    } else {
        return hipErrorInvalidValue;  // exact block-wise accumulation exists for M <= 32 only (checked by the ABI)
    }
    return hipGetLastError();
}

template <bool kFp8>
static hipError_t launch_blockwise_m(const uint8_t* aq, bool a_packed, const float* sa, const uint8_t* wq,
                                     bool w_packed, const float* sw, void* y, bool y_bf16, int M, int N, int K,
                                     hipStream_t stream) {
#define FP8SG_BW(YB, WP, AP) \
    launch_blockwise_t<kFp8, (YB) ? kOutBF16 : kOutF32, WP, AP>(aq, sa, wq, sw, y, M, N, K, stream)
    if (y_bf16) {
        if (a_packed) return w_packed ? FP8SG_BW(true, true, true) : FP8SG_BW(true, false, true);
        return w_packed ? FP8SG_BW(true, true, false) : FP8SG_BW(true, false, false);
    }
    if (a_packed) return w_packed ? FP8SG_BW(false, true, true) : FP8SG_BW(false, false, true);
    return w_packed ? FP8SG_BW(false, true, false) : FP8SG_BW(false, false, false);
#undef FP8SG_BW
}

hipError_t launch_gemm_blockwise(const uint8_t* aq, bool a_packed, const float* a_scales, const uint8_t* wq,
                                 bool w_packed, const float* w_scales, void* y, bool y_bf16, int64_t M, int64_t N,
                                 int64_t K, bool fp8_mfma, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const int m = (int)M, n = (int)N, k = (int)K;
    if (fp8_mfma)
        return launch_blockwise_m<true>(aq, a_packed, a_scales, wq, w_packed, w_scales, y, y_bf16, m, n, k, stream);
    return launch_blockwise_m<false>(aq, a_packed, a_scales, wq, w_packed, w_scales, y, y_bf16, m, n, k, stream);
}

// ---------------------------------------------------------------------------
// Decode GEMM with the per-token activation quantization fused in (bf16 X,
// M <= 4, K <= 4096): X [M, K] in, Y out, one launch.
//
// The dynamic per-token rule needs each row's maximum before any code, and
// every workgroup needs all of A, so each workgroup quantizes the few rows
// itself, while the weight stream is already under way: a wave first issues
// the loads of its X chunks (one chunk of 8 per thread and row), then the
// loads of ALL its W blocks (at most kFusedMaxPer, held in registers), and only
// then waits for X.  Loads complete in issue order, so X arrives first and the
// quantization (row maxima by wave shuffles and LDS, encode, codes to LDS with
// rows K + 16 bytes apart) runs while W is in flight.  Rows, chunks and blocks
// past the valid ones are clamped to valid addresses and masked, so the code
// between the loads has no branches.  8 waves of at most 128 registers each:
// the whole weight matrix of the decode shape is then requested at once by
// workgroups that all fit on the chip together (two per CU).  Workgroup 0
// also writes the scales for the caller.  The multiplies are the skinny
// kernel's: W fragments from registers, A fragments from LDS, k blocks split
// round-robin over the waves, partial sums added in fixed order.
constexpr int kFusedMaxM = 4;      // rows: with more, the X registers push the wave past 128 VGPRs
constexpr int kFusedKS = 8;         // waves per workgroup
constexpr int kFusedRowChunks = 1;  // chunks of 8 per thread and row: K <= 8 * 1 * 64 * kFusedKS
constexpr int kFusedMaxPer = 4;     // W blocks per wave: K <= 128 * 4 * kFusedKS

__device__ __forceinline__ Frag load_frag_lds(const uint8_t* p) {
    Frag f;
    f.lo = reinterpret_cast<const uint4*>(p)[0];
    f.hi = reinterpret_cast<const uint4*>(p)[1];
    return f;
}

template <bool kFp8, int kOut, bool kWPacked, int kNS, int kKS, int kM>
__global__ __launch_bounds__(64 * kKS) __attribute__((amdgpu_waves_per_eu(4))) void gemm_skinny_fused(
    const uint16_t* __restrict__ X, float* __restrict__ sa_out, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, const float* __restrict__ qs) {
    extern __shared__ __attribute__((aligned(16))) uint8_t a_lds[];  // [M][K + 16] codes
    __shared__ f32x4 red[kKS > 1 ? kKS - 1 : 1][kNS][64];
    __shared__ float row_max[kKS][kFusedMaxM];
    __shared__ float row_scale[kFusedMaxM];
    constexpr int T = 64 * kKS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n_base = (int64_t)blockIdx.x * (16 * kNS);
    const int nkb = K >> 7;
    const int r16 = lane & 15, kofs = (lane >> 4) * 32;
    const int pitch = K + 16;
    const int row_chunks = K >> 3;

    // 1. X: this thread's chunks of every row (clamped to valid rows / chunks)
    uint4 xr[kM][kFusedRowChunks];
#pragma unroll
    for (int r = 0; r < kM; ++r) {
        const int rr = r < M ? r : M - 1;
#pragma unroll
        for (int i = 0; i < kFusedRowChunks; ++i) {
            int c = threadIdx.x + i * T;
            c = c < row_chunks ? c : row_chunks - 1;
            xr[r][i] = *reinterpret_cast<const uint4*>(X + (int64_t)rr * K + (int64_t)c * 8);
        }
    }

    // 2. W: every block of this wave (wave + j * kKS, j < nper; clamped past the end)
    const int nper = nkb > wave ? (nkb - wave + kKS - 1) / kKS : 0;
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
    Frag wf[kFusedMaxPer][kNS];
#pragma unroll
    for (int j = 0; j < kFusedMaxPer; ++j) {
        int jj = j < nper ? j : nper - 1;
        jj = jj > 0 ? jj : 0;
        int kb = wave + jj * kKS;
        kb = kb < nkb ? kb : nkb - 1;  // a wave without blocks (nper == 0) loads block nkb - 1, unused
#pragma unroll
        for (int s = 0; s < kNS; ++s)
            wf[j][s] = kWPacked ? load_frag_packed_stream(wrow[s] + kb * kPackBlock, lane)
                                : load_frag_global(wrow[s] + ((int64_t)kb << 7));
    }

    // 3. row maxima and scales
#pragma unroll
    for (int r = 0; r < kM; ++r) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kFusedRowChunks; ++i) {
            const uint4 u = xr[r][i];
            const float a = fmaxf(fmaxf(fmaxf(__builtin_fabsf(bf16_lo(u.x)), __builtin_fabsf(bf16_hi(u.x))),
                                        fmaxf(__builtin_fabsf(bf16_lo(u.y)), __builtin_fabsf(bf16_hi(u.y)))),
                                  fmaxf(fmaxf(__builtin_fabsf(bf16_lo(u.z)), __builtin_fabsf(bf16_hi(u.z))),
                                        fmaxf(__builtin_fabsf(bf16_lo(u.w)), __builtin_fabsf(bf16_hi(u.w)))));
            const bool valid = (int)threadIdx.x + i * T < row_chunks;
            amax = valid ? fmaxf(amax, a) : amax;
        }
        amax = wave_max(amax);
        if (lane == 0) row_max[wave][r] = amax;
    }
    __syncthreads();
    if (threadIdx.x < kM) {
        float m = row_max[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kKS; ++w) m = fmaxf(m, row_max[w][threadIdx.x]);
        const float sc = dynamic_scale(m, kE4M3Max);
        row_scale[threadIdx.x] = sc;
        if (blockIdx.x == 0 && sa_out != nullptr && (int)threadIdx.x < M) sa_out[threadIdx.x] = sc;
    }
    __syncthreads();

    // 4. codes to LDS
#pragma unroll
    for (int r = 0; r < kM; ++r) {
        if (r < M) {
            const QScale p = make_qscale(row_scale[r], kE4M3Max);
#pragma unroll
            for (int i = 0; i < kFusedRowChunks; ++i) {
                const int c = threadIdx.x + i * T;
                if (c < row_chunks) {
                    float v[8];
                    const uint4 u = xr[r][i];
                    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
                    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
                    *reinterpret_cast<uint2*>(a_lds + r * pitch + c * 8) = encode_chunk_dynamic<uint16_t>(v, p);
                }
            }
        }
    }
    __syncthreads();

    // 5. the multiplies of this wave's blocks
    f32x4 acc[kNS];
#pragma unroll
    for (int s = 0; s < kNS; ++s) acc[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint8_t* arow = a_lds + (r16 < M ? r16 : M - 1) * pitch + kofs;
#pragma unroll
    for (int j = 0; j < kFusedMaxPer; ++j) {
        if (j < nper) {
            const Frag af = load_frag_lds(arow + (wave + j * kKS) * 128);
#pragma unroll
            for (int s = 0; s < kNS; ++s) acc[s] = mma<kFp8>(wf[j][s], af, acc[s]);
        }
    }

    if (kKS > 1) {
        if (wave > 0) {
#pragma unroll
            for (int s = 0; s < kNS; ++s) red[wave - 1][s][lane] = acc[s];
        }
        __syncthreads();
    }
    if (wave == 0) {
        const bool vec_ok = (N & 3) == 0;
        const QScale q = out_qscale<kOut>(qs);
        const int m = r16;
#pragma unroll
        for (int s = 0; s < kNS; ++s) {
            f32x4 a = acc[s];
#pragma unroll
            for (int w = 0; w < kKS - 1; ++w) a += red[w][s][lane];
            const int64_t n0 = n_base + 16 * s + 4 * (lane >> 4);
            if (m < M && n0 < N) store4<kOut>(Y, N, m, n0, a, row_scale[m], sw, vec_ok, q);
        }
    }
}

template <bool kFp8, int kOut, bool kWPacked>
static void launch_fused_t(const uint16_t* x, float* sa_out, const uint8_t* wq, const float* sw, void* y, int M,
                           int N, int K, const float* qs, hipStream_t stream) {
    dim3 grid((unsigned)((N + 16 * SKINNY_NS - 1) / (16 * SKINNY_NS))), block(64 * kFusedKS);
    const size_t lds = (size_t)M * (size_t)(K + 16);
#define FP8SG_FUSED_M(KM) \
    gemm_skinny_fused<kFp8, kOut, kWPacked, SKINNY_NS, kFusedKS, KM><<<grid, block, lds, stream>>>(x, sa_out, wq, sw, \
                                                                                                y, M, N, K, qs)
    if (M <= 1) FP8SG_FUSED_M(1);
    else if (M <= 2) FP8SG_FUSED_M(2);
    else FP8SG_FUSED_M(4);
#undef FP8SG_FUSED_M
}

template <bool kFp8, int kOut>
static void launch_fused_w(const uint16_t* x, float* sa_out, const uint8_t* wq, bool w_packed, const float* sw,
                           void* y, int M, int N, int K, const float* qs, hipStream_t stream) {
    if (w_packed) launch_fused_t<kFp8, kOut, true>(x, sa_out, wq, sw, y, M, N, K, qs, stream);
    else launch_fused_t<kFp8, kOut, false>(x, sa_out, wq, sw, y, M, N, K, qs, stream);
}

bool gemm_fused_quant_fits(bool x_is_bf16, int64_t M, int64_t K) {
    return x_is_bf16 && M >= 1 && M <= kFusedMaxM && K <= (int64_t)8 * kFusedRowChunks * 64 * kFusedKS &&
           K <= (int64_t)128 * kFusedMaxPer * kFusedKS;
}

hipError_t launch_gemm_fused_quant(const uint16_t* x, float* sa_out, const uint8_t* wq, bool w_packed,
                                   const float* w_scales, void* y, int out_kind, const float* out_scale, int64_t M,
                                   int64_t N, int64_t K, bool fp8_mfma, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const int m = (int)M, n = (int)N, k = (int)K;
#define FP8SG_FUSED(F8, OUT) launch_fused_w<F8, OUT>(x, sa_out, wq, w_packed, w_scales, y, m, n, k, out_scale, stream)
    if (fp8_mfma) {
        if (out_kind == kOutBF16) FP8SG_FUSED(true, kOutBF16);
        else if (out_kind == kOutE4M3) FP8SG_FUSED(true, kOutE4M3);
        else FP8SG_FUSED(true, kOutF32);
    } else {
        if (out_kind == kOutBF16) FP8SG_FUSED(false, kOutBF16);
        else if (out_kind == kOutE4M3) FP8SG_FUSED(false, kOutE4M3);
        else FP8SG_FUSED(false, kOutF32);
    }
#undef FP8SG_FUSED
    return hipGetLastError();
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
