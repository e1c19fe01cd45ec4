// Large-tile FP8 W8A8 GEMM kernels for gfx950 (M > 32): 256 x 256 tiles staged
// through LDS by direct global-to-LDS copies, in FP8 mode, exact mode and with
// block-wise scales.  Operand roles, the k assignment of a lane and the two
// accumulation modes are described at the top of gemm.hip.
#include <type_traits>

#include "gemm_common.h"

namespace fp8sg {

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
        auto stage = [&](auto fast_tag) __attribute__((always_inline)) {
            constexpr bool kFast = decltype(fast_tag)::value;
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
                    else epi_put4_q(wl, row, col, out_codes4_known<kFast>(v0, v1, v2, v3, q));
                }
            }
        };
        // the output scale's range test once per wave, not once per value
        if (kOut == kOutE4M3 && !q.fast) stage(std::false_type{});
        else stage(std::true_type{});
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

// Exact mode.  The FP8 codes are widened to bf16 (exact: every E4M3 value is a
// bf16 value) and multiplied by v_mfma_f32_32x32x16_bf16: each wave's 128 x 128
// share is 4 x 4 tiles of 32 x 32, with all 256 accumulator registers (one
// wave per SIMD).  With a single wave per SIMD nothing hides a stall, so the
// loop is software-pipelined by hand:
//
//  * The k range is walked in half blocks of 64 (the two 1 KB halves of each
//    16-row x 128-k fragment block).  LDS holds a ring of four half-block
//    slots of 32 KB (A 16 KB, W 16 KB).  The copies of half block h + 4 go
//    into slot h % 4 while half block h is multiplied, so each copy has three
//    half blocks (~6000 matrix-core cycles) to arrive.
//  * One barrier per half block.  Before it a wave waits for its own copies of
//    half block h + 1 (vmcnt: the copies of h + 2 and h + 3 stay in flight) and
//    for its own reads of half block h (lgkmcnt(0)); after it every copy of
//    h + 1 has landed and nobody reads slot h % 4 any more.
//  * The fragments of half block h + 1 are read from LDS into registers while
//    half block h is multiplied (two register sets of 64 VGPRs), and each
//    16-k step widens the operands of the next step between its own 16
//    multiplies (two sets of 32 VGPRs), so the matrix core never waits for a
//    read or a convert.
//
// Operand lane layout of the 32 x 32 x 16 instruction: lane l supplies row
// l % 32 and k 8 (l / 32) .. 8 (l / 32) + 7 of the step.  Within half block
// (kb, h) the 16-row subtile's lane slot s = (r % 16) + 16 q holds bytes
// [32 q + 16 h, 32 q + 16 h + 16) of row r's 128 k; step t (0..3) gives lane l
// the 8 bytes at offset 8 (t % 2) of slot q = 2 (l / 32) + t / 2 of row l % 32.
// A and W use the same assignment, so every product pairs matching k, and the
// 8 steps of a k block cover its 128 k once.  Output lane layout: acc[r] of
// lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] of the tile.
constexpr int kExSlot = 32 * 1024;   // one half-block slot: A 16 KB + W 16 KB
constexpr int kExSlots = 4;
static_assert(4 * kEpiWaveBytes <= kExSlots * kExSlot, "the staged output reuses the slots");

// s_waitcnt immediate for vmcnt(n) and lgkmcnt(0).
constexpr int wait_vmcnt_lgkm0(int n) {
    return 0x0070 | (n & 15) | ((n >> 4) << 14);
}

template <int kOut, bool kWPacked, bool kAPacked>
__global__ __launch_bounds__(256, 1) void gemm_big_exact(const uint8_t* __restrict__ A, const float* __restrict__ sa,
                                                         int sa_per_token, const uint8_t* __restrict__ W,
                                                         const float* __restrict__ sw, void* __restrict__ Y, int M,
                                                         int N, int K, int tiles_per_xcd,
                                                         const float* __restrict__ qs) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // kExSlots x kExSlot
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    int tile;
    int64_t m_base, n_base;
    tile_coords(M, N, tiles_per_xcd, tile, m_base, n_base);
    if (tile < 0) return;
    const int nkb = K >> 7;
    const int nhb = 2 * nkb;   // half blocks

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Copies: waves 0, 1 fill A subtiles 0-7 / 8-15 of every slot, waves 2, 3 the W
    // subtiles; 8 one-kilobyte copies per wave per half block.  o[j]: the lane's
    // source offset of subtile 8 (wave % 2) + j at k block 0, half 0.
    const bool cp_w = wave >= 2;
    const bool cp_packed = cp_w ? kWPacked : kAPacked;
    const int sub0 = 8 * (wave & 1);
    uint32_t o[8];
    {
        const int64_t base_row = cp_w ? n_base : m_base;
        const int rows = cp_w ? N : M;
        const int r16 = lane & 15, kq = (lane >> 4) * 32;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int js = sub0 + j;
            if (cp_packed) {
                int64_t t = (base_row >> 4) + js;
                const int64_t last_tile = ((int64_t)rows + 15) / 16 - 1;
                t = t < last_tile ? t : last_tile;
                o[j] = (uint32_t)((t - (base_row >> 4)) * (int64_t)nkb * kPackBlock + 16 * lane);
            } else {
                int64_t r = base_row + 16 * js + r16;
                r = r < rows ? r : rows - 1;
                o[j] = (uint32_t)((r - base_row) * K + kq);
            }
        }
    }
    const uint8_t* src = cp_w ? (kWPacked ? W + (n_base >> 4) * (int64_t)nkb * kPackBlock : W + n_base * K)
                              : (kAPacked ? A + (m_base >> 4) * (int64_t)nkb * kPackBlock : A + m_base * K);
    const int64_t src_kb = cp_packed ? kPackBlock : 128;   // bytes per k block
    const int64_t src_h = cp_packed ? 1024 : 16;           // bytes to the second half
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    const uint32_t dst_op = lds0 + (cp_w ? 16 * 1024u : 0u) + (uint32_t)sub0 * 1024u;

    // copy j (0..7) of half block hb (clamped to the last one) into its slot
    auto copy = [&](int j, int hb) __attribute__((always_inline)) {
        hb = hb < nhb ? hb : nhb - 1;
        const int64_t off = (int64_t)(hb >> 1) * src_kb + (int64_t)(hb & 1) * src_h;
        copy16_to_lds(src + off + o[j], dst_op + (uint32_t)((hb & (kExSlots - 1)) * kExSlot + j * 1024));
    };

    // Fragment reads: tile t of the wave's W (t = 0..3) or A (t = 4..7) rows, slot
    // part u (0, 1); the lane's 16 bytes of the half block.
    const int lane_off = ((lane & 31) >> 4) * 1024 + (lane & 15) * 16 + (lane >> 5) * 512;
    const uint8_t* rd_w = smem + 16 * 1024 + wn * 8 * 1024 + lane_off;
    const uint8_t* rd_a = smem + wm * 8 * 1024 + lane_off;
    uint4 raw[2][8][2];
    auto read = [&](int b, int t, int u, int hb) __attribute__((always_inline)) {
        const int slot = (hb & (kExSlots - 1)) * kExSlot;
        const uint8_t* p = (t < 4 ? rd_w + 2048 * t : rd_a + 2048 * (t - 4)) + slot + 256 * u;
        raw[b][t][u] = *reinterpret_cast<const uint4*>(p);
    };
    bf16x8 v[2][8];
    auto widen = [&](int vb, int b, int t) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const uint4 r = raw[b][f][t >> 1];
            v[vb][f] = (t & 1) ? widen8(r.z, r.w) : widen8(r.x, r.y);
        }
    };

    if (nhb > 0) {
#pragma unroll
        for (int h = 0; h < kExSlots; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) copy(j, h);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(24));   // this wave's copies of half block 0 have landed
        barrier_no_fence();                           // ... and every other wave's
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u) read(0, t, u, 0);
        widen(0, 0, 0);
    }

    // Half block hb, its fragments in raw[b]: four steps of 16 k.  Step t issues
    // two of the eight copies of hb + 4, steps 0 and 1 the reads of hb + 1 into
    // raw[b ^ 1]; each step widens the next step's operands between its
    // multiplies (step 3: step 0 of hb + 1).
    auto half_block = [&](int hb, int b) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(16));
        barrier_no_fence();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            copy(2 * t, hb + 4);
            copy(2 * t + 1, hb + 4);
            __builtin_amdgcn_sched_barrier(0);
            if (t < 2) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int u = 0; u < 2; ++u) read(b ^ 1, 4 * t + q, u, hb + 1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[t & 1][i], v[t & 1][4 + j], acc[i][j], 0,
                                                                        0, 0);
            if (t < 3) widen((t + 1) & 1, b, t + 1);
            else widen(0, b ^ 1, 0);
            // issue order: each multiply followed by two converts (the reads first, one per multiply)
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if (t < 2 && k < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    for (int hb = 0; hb < nhb; hb += 2) {
        half_block(hb, 0);
        half_block(hb + 1, 1);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // no copy into LDS may outlive the workgroup

    if (kOut == kOutBF16 || kOut == kOutE4M3) {
        __syncthreads();  // every wave is done with the slots: the LDS now holds the output tiles
        uint8_t* wl = smem + wave * kEpiWaveBytes;
        const QScale q = out_qscale<kOut>(qs);
        float sam[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t m = m_base + wm * 128 + 32 * j + (lane & 31);
            m = m < M ? m : M - 1;
            sam[j] = sa[sa_per_token ? m : 0];
        }
        auto stage = [&](auto fast_tag) __attribute__((always_inline)) {
            constexpr bool kFast = decltype(fast_tag)::value;
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
                        else epi_put4_q(wl, row, col, out_codes4_known<kFast>(v0, v1, v2, v3, q));
                    }
                }
        };
        // the output scale's range test once per wave, not once per value
        if (kOut == kOutE4M3 && !q.fast) stage(std::false_type{});
        else stage(std::true_type{});
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
// order, two stages, copies two k blocks ahead, fence-free barriers).  A stage
// is released in two parts, so its refill is spread over the k block instead
// of following its last read in one burst (a burst of copies holds up the
// multiplies queued behind it): the A tile, the scales and the W subtiles of
// rows 0-3 (each wave's W fragments 0-3) are read by row 3, and after a
// barrier there their copies for block kb + 2 are issued over rows 3-6; the W
// subtiles of rows 4-7 are read by row 7 and are copied after the barrier
// there.  Every wave makes 4 one-kilobyte A copies, 2 + 2 W copies and one
// 4-byte-per-lane copy of scales: waves 0-3 the s_a of tile rows 64 w + lane,
// waves 4-7 the s_w of the tile's two 128-column blocks (lane % 2).
constexpr int kBwOps = 32 * kPackBlock;       // A 32 KB + W 32 KB
constexpr int kBwStage = kBwOps + 2048;       // + s_a (256 floats) + s_w (4 x 64 floats)
constexpr int kBwCopies = 9;                  // copies per wave per stage

template <int kOut, bool kWPacked, bool kAPacked>
__global__ __launch_bounds__(512, 1) void gemm_big_blockwise(const uint8_t* __restrict__ A,
                                                             const float* __restrict__ sa, int sa_kmajor,
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

    // This wave's copies per stage: c = 0..3 the A (subtile, half) pairs 4 wave + c;
    // c = 4, 5 W pairs of rows 0-3 (subtiles 0-3 and 8-11), c = 6, 7 W pairs of
    // rows 4-7 (subtiles 4-7 and 12-15); c = 8 the scales.  o[c]: the lane's
    // source offset at k block 0; d[c]: the destination offset in a stage.
    const bool cp_a = wave < 4;
    uint32_t o[8], d[8];
    {
        auto pair = [&](int c, int& sub, int& half) __attribute__((always_inline)) {
            if (c < 4) {
                sub = (4 * wave + c) >> 1;
                half = c & 1;
            } else {
                const int q = 2 * wave + (c & 1);                    // 0..15 within the row half
                const int j = q >> 1;                                 // 0..7
                sub = (j & 3) + ((j >> 2) << 3) + (c >= 6 ? 4 : 0);   // {0-3, 8-11} or {4-7, 12-15}
                half = q & 1;
            }
        };
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            int sub, half;
            pair(c, sub, half);
            const bool is_a = c < 4;
            const bool packed = is_a ? kAPacked : kWPacked;
            const int64_t base_row = is_a ? m_base : n_base;
            const int rows = is_a ? M : N;
            if (packed) {
                int64_t t = (base_row >> 4) + sub;
                const int64_t last_tile = ((int64_t)rows + 15) / 16 - 1;
                t = t < last_tile ? t : last_tile;
                o[c] = (uint32_t)((t - (base_row >> 4)) * (int64_t)nkb * kPackBlock + 1024 * half + 16 * lane);
            } else {
                int64_t r = base_row + 16 * sub + (lane & 15);
                r = r < rows ? r : rows - 1;
                o[c] = (uint32_t)((r - base_row) * K + (lane >> 4) * 32 + 16 * half);
            }
            d[c] = (uint32_t)((is_a ? 0 : 16 * kPackBlock) + sub * kPackBlock + half * 1024);
        }
    }
    const uint8_t* a_src = kAPacked ? A + (m_base >> 4) * (int64_t)nkb * kPackBlock : A + m_base * K;
    const uint8_t* w_src = kWPacked ? W + (n_base >> 4) * (int64_t)nkb * kPackBlock : W + n_base * K;
    const int64_t a_kb = kAPacked ? kPackBlock : 128, w_kb = kWPacked ? kPackBlock : 128;
    // s_a [M, K/128] row-major, or k-block-major [K/128, M] (sa_kmajor): then the 64
    // scales a wave copies per k block are 256 contiguous bytes instead of 64 lines
    const float* ssrc;
    int64_t sstep = 1;
    if (cp_a) {
        int64_t m = m_base + 64 * wave + lane;
        m = m < M ? m : M - 1;
        ssrc = sa_kmajor ? sa + m : sa + m * nkb;
        sstep = sa_kmajor ? (int64_t)M : 1;
    } else {
        int64_t nb = (n_base >> 7) + (lane & 1);
        nb = nb < nbw ? nb : nbw - 1;
        ssrc = sw + nb * nkb;
    }
    const uint32_t dst_sc = (uint32_t)(kBwOps + 256 * wave);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

    // copy c (0..8) of block kb into the stage at LDS address `stage`
    auto issue_copy = [&](int c, uint32_t stage, int kb) __attribute__((always_inline)) {
        if (c < 4) copy16_to_lds(a_src + (int64_t)kb * a_kb + o[c], stage + d[c]);
        else if (c < 8) copy16_to_lds(w_src + (int64_t)kb * w_kb + o[c], stage + d[c]);
        else copy4_to_lds(ssrc + kb * sstep, stage + dst_sc);
    };
    // copies issued before rows 3..7 of a k block: [kBwSplit[i - 3], kBwSplit[i - 2]) -- rows 3-6 the
    // A, scale and first-half W copies (c = 0..5, 8), row 7 the second-half W copies (c = 6, 7)
    constexpr int kBwOrder[kBwCopies] = {0, 1, 4, 2, 3, 5, 8, 6, 7};
    constexpr int kBwSplit[6] = {0, 2, 4, 6, 7, 9};

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
        f32x4 p[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = load_frag_packed(cur + (4 * wm + j) * kPackBlock, lane);
        const uint8_t* lw = cur + (16 + 8 * wn) * kPackBlock;
        wf[0] = load_frag_packed(lw, lane);
        const int nxt = kb + 2 < nkb ? kb + 2 : nkb - 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i == 3 || i == 7) {
                // every wave's reads of the stage's A tile, scales and W rows 0-3 (row 3) or
                // of the rest of it (row 7) are done: that part may be refilled with block kb + 2
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads
                barrier_no_fence();                  // ... and every other wave's
            }
            if (i >= 3) {
#pragma unroll
                for (int c = kBwSplit[i - 3]; c < kBwSplit[i - 2]; ++c) issue_copy(kBwOrder[c], cur_lds, nxt);
            }
            if (i < 7) wf[(i + 1) & 1] = load_frag_packed(lw + (i + 1) * kPackBlock, lane);
            __builtin_amdgcn_sched_barrier(0);
            // the products of W fragment i, then the scaled adds of fragment i - 1, whose
            // products were issued a row earlier: no add waits for its multiply
#pragma unroll
            for (int j = 0; j < 4; ++j) p[i & 1][j] = mma_fp8(wf[i & 1], af[j], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            if (i > 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 q = p[(i - 1) & 1][j];
                    asm volatile("" : "+v"(q));  // keeps the adds in this row (plain arithmetic would be
                                                 // placed right behind its multiply, which then stalls)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i - 1][j][r] = __builtin_fmaf(q[r], f[j], acc[i - 1][j][r]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[7][j][r] = __builtin_fmaf(p[1][j][r], f[j], acc[7][j][r]);
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

// ---------------------------------------------------------------------------
// Block-wise scaled GEMM for M > 32 with exact partials: each 128-deep partial
// P_kb is formed on the bf16 matrix cores from the exactly widened codes (as in
// gemm_big_exact), then multiplied by its scale product and added to an fp32
// accumulator with vector FMAs (the same promotion as gemm_big_blockwise).  The
// FMAs read the partials and write the accumulators, so both live in the
// vector registers: a wave owns 64 x 64 outputs, 4 partials and 4 accumulators
// of 32 x 32 (128 registers), and two waves share each SIMD.
//
// 256 (m) x 128 (n) tile per workgroup of 8 waves.  Wave (wm, wn) = (wave % 4,
// wave / 4) owns tile rows 64 wm .. 64 wm + 63 (A fragments 2 wm, 2 wm + 1)
// and columns 64 wn .. 64 wn + 63 (W fragments 2 wn, 2 wn + 1); fragment and
// output lane layouts as in gemm_big_exact.  Half-block slots as there: the
// copies run four half blocks ahead, the next half block's fragments are read
// during the first two steps of the current one, and each slot holds the 16 A
// subtiles (16 KB), the 8 W subtiles (8 KB) and, in the slot of a k block's
// first half, the block's scales.  Per half block every wave copies A subtiles
// 2 w and 2 w + 1 and W subtile w; in a k block's first half also one
// 4-byte-per-lane copy of scales: waves 0-3 the s_a of tile rows 64 w + lane,
// waves 4-7 the tile's s_w (one value in every lane; each of these waves makes
// its own copy, so that every wave has the same number of copies in flight).
// A k block's scales are read with its first half block's fragments, before
// the barrier that lets that slot be refilled.
constexpr int kBxTileN = 128;
constexpr int kBxOps = 24 * 1024;          // A 16 KB + W 8 KB
constexpr int kBxSlot = kBxOps + 2048;     // + s_a (256 floats) + 4 copies of s_w (64 floats each)
constexpr int kBxSlots = 4;
constexpr int kBxEpiWaveBytes = 64 * 128;  // a wave's 64 x 64 bf16 outputs, staged
static_assert(8 * kBxEpiWaveBytes <= kBxSlots * kBxSlot, "the staged output reuses the slots");

template <int kOut, bool kWPacked, bool kAPacked>
__global__ __launch_bounds__(512, 1) void gemm_big_blockwise_exact(const uint8_t* __restrict__ A,
                                                                   const float* __restrict__ sa, int sa_kmajor,
                                                                   const uint8_t* __restrict__ W,
                                                                   const float* __restrict__ sw,
                                                                   void* __restrict__ Y, int M, int N, int K,
                                                                   int tiles_per_xcd) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // kBxSlots x kBxSlot
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    int tile;
    int64_t m_base, n_base;
    tile_coords<kBxTileN>(M, N, tiles_per_xcd, tile, m_base, n_base);
    if (tile < 0) return;
    const int nkb = K >> 7;
    const int nhb = 2 * nkb;

    f32x16 acc[2][2], p[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // copy c = 0, 1: A subtile 2 wave + c; c = 2: W subtile wave.  o[c]: the lane's
    // source offset at k block 0, half 0, relative to the tile's first row.
    uint32_t o[3];
    {
        const int r16 = lane & 15, kq = (lane >> 4) * 32;
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const bool is_a = c < 2;
            const int sub = is_a ? 2 * wave + c : wave;
            const bool packed = is_a ? kAPacked : kWPacked;
            const int64_t base_row = is_a ? m_base : n_base;
            const int rows = is_a ? M : N;
            if (packed) {
                int64_t t = (base_row >> 4) + sub;
                const int64_t last_tile = ((int64_t)rows + 15) / 16 - 1;
                t = t < last_tile ? t : last_tile;
                o[c] = (uint32_t)((t - (base_row >> 4)) * (int64_t)nkb * kPackBlock + 16 * lane);
            } else {
                int64_t r = base_row + 16 * sub + r16;
                r = r < rows ? r : rows - 1;
                o[c] = (uint32_t)((r - base_row) * K + kq);
            }
        }
    }
    const uint8_t* a_src = kAPacked ? A + (m_base >> 4) * (int64_t)nkb * kPackBlock : A + m_base * K;
    const uint8_t* w_src = kWPacked ? W + (n_base >> 4) * (int64_t)nkb * kPackBlock : W + n_base * K;
    const int64_t a_kb = kAPacked ? kPackBlock : 128, a_h = kAPacked ? 1024 : 16;
    const int64_t w_kb = kWPacked ? kPackBlock : 128, w_h = kWPacked ? 1024 : 16;
    // the scale this lane copies: s_a of tile row 64 wave + lane (waves 0-3) or the
    // tile's s_w (waves 4-7); s_a [M, K/128] row-major or k-block-major [K/128, M]
    const float* ssrc;
    int64_t sstep = 1;
    if (wave < 4) {
        int64_t m = m_base + 64 * wave + lane;
        m = m < M ? m : M - 1;
        ssrc = sa_kmajor ? sa + m : sa + m * nkb;
        sstep = sa_kmajor ? (int64_t)M : 1;
    } else {
        const int64_t nbw = ((int64_t)N + 127) >> 7;
        int64_t nb = n_base >> 7;
        nb = nb < nbw ? nb : nbw - 1;
        ssrc = sw + nb * nkb;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    const uint32_t dst_a = lds0 + (uint32_t)(2 * wave) * 1024u;
    const uint32_t dst_w = lds0 + 16 * 1024u + (uint32_t)wave * 1024u;
    const uint32_t dst_s = lds0 + (uint32_t)kBxOps + 256u * (uint32_t)wave;

    // copy c of half block hb (clamped to the last one) into slot hb % 4; the
    // scale copy of the k block whose first half hb is (hb even)
    auto copy = [&](int c, int hb) __attribute__((always_inline)) {
        const uint32_t slot = (uint32_t)((hb & (kBxSlots - 1)) * kBxSlot);
        hb = hb < nhb ? hb : nhb - 1;
        if (c < 2)
            copy16_to_lds(a_src + (int64_t)(hb >> 1) * a_kb + (int64_t)(hb & 1) * a_h + o[c],
                          dst_a + slot + (uint32_t)c * 1024u);
        else
            copy16_to_lds(w_src + (int64_t)(hb >> 1) * w_kb + (int64_t)(hb & 1) * w_h + o[2], dst_w + slot);
    };
    auto copy_scales = [&](int hb) __attribute__((always_inline)) {
        const uint32_t slot = (uint32_t)((hb & (kBxSlots - 1)) * kBxSlot);
        int kb = hb >> 1;
        kb = kb < nkb ? kb : nkb - 1;
        copy4_to_lds(ssrc + (int64_t)kb * sstep, dst_s + slot);
    };

    // Fragment reads: t = 0, 1 the wave's W fragments, t = 2, 3 its A fragments;
    // slot part u (0, 1): the lane's 16 bytes of the half block.
    const int lane_off = ((lane & 31) >> 4) * 1024 + (lane & 15) * 16 + (lane >> 5) * 512;
    const uint8_t* rd_w = smem + 16 * 1024 + wn * 4 * 1024 + lane_off;
    const uint8_t* rd_a = smem + wm * 4 * 1024 + lane_off;
    uint4 raw[2][4][2];
    auto read = [&](int b, int t, int u, int hb) __attribute__((always_inline)) {
        const int slot = (hb & (kBxSlots - 1)) * kBxSlot;
        const uint8_t* q = (t < 2 ? rd_w + 2048 * t : rd_a + 2048 * (t - 2)) + slot + 256 * u;
        raw[b][t][u] = *reinterpret_cast<const uint4*>(q);
    };
    // scales of the k block whose first half is hb: s_a of the lane's two rows, s_w
    float nsa[2], nsw;
    auto read_scales = [&](int hb) __attribute__((always_inline)) {
        const float* ls = reinterpret_cast<const float*>(smem + (hb & (kBxSlots - 1)) * kBxSlot + kBxOps);
#pragma unroll
        for (int j = 0; j < 2; ++j) nsa[j] = ls[64 * wm + 32 * j + (lane & 31)];
        nsw = ls[256];
    };
    bf16x8 v[2][4];
    auto widen = [&](int vb, int b, int t) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const uint4 r = raw[b][f][t >> 1];
            v[vb][f] = (t & 1) ? widen8(r.z, r.w) : widen8(r.x, r.y);
        }
    };

    if (nhb > 0) {
#pragma unroll
        for (int h = 0; h < kBxSlots; ++h) {
#pragma unroll
            for (int c = 0; c < 3; ++c) copy(c, h);
            if ((h & 1) == 0) copy_scales(h);
        }
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(10));   // this wave's copies of half block 0 have landed
        barrier_no_fence();                           // ... and every other wave's
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u) read(0, t, u, 0);
        read_scales(0);
        widen(0, 0, 0);
    }

    float f[2] = {0.0f, 0.0f};
    // Half block hb (b = hb % 2), its fragments in raw[b]: four steps of 16 k.
    // Steps 0-2 issue the three operand copies of hb + 4 (step 3 the scale copy
    // when hb + 4 starts a k block); steps 0 and 1 read hb + 1 into raw[b ^ 1]
    // (and, when hb + 1 starts a k block, its scales); each step widens the next
    // step's operands between its multiplies.  The first step of a k block starts
    // the partials from zero; after the last one they are promoted.
    auto half_block = [&](int hb, int b) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        // copies in flight after this wait: those of hb + 2 and hb + 3 (3 + 4 in some order)
        __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(7));
        barrier_no_fence();
        if (b == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j) f[j] = nsa[j] * nsw;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            if (t < 3) copy(t, hb + 4);
            else if (b == 0) copy_scales(hb + 4);
            __builtin_amdgcn_sched_barrier(0);
            if (b == 1 && t == 1) read_scales(hb + 1);
            if (t < 2) {
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int u = 0; u < 2; ++u) read(b ^ 1, 2 * t + q, u, hb + 1);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const f32x16 c = (b == 0 && t == 0) ? f32x16{} : p[i][j];
                    p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[t & 1][i], v[t & 1][2 + j], c, 0, 0, 0);
                }
            if (t < 3) widen((t + 1) & 1, b, t + 1);
            else widen(0, b ^ 1, 0);
            // issue order: each multiply followed by four converts (the reads first, one per multiply)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (t < 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (b == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(p[i][j][r], f[j], acc[i][j][r]);
        }
    };

    for (int hb = 0; hb < nhb; hb += 2) {
        half_block(hb, 0);
        half_block(hb + 1, 1);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // no copy into LDS may outlive the workgroup

    static_assert(kOut == kOutBF16 || kOut == kOutF32, "block-wise GEMMs write bf16 or fp32");
    if (kOut == kOutBF16) {
        // stage the wave's 64 x 64 outputs row-major (128-byte rows, 16-byte slots
        // XORed with the row's low three bits), then store 16 bytes per lane
        __syncthreads();  // every wave is done with the slots
        uint8_t* wl = smem + wave * kBxEpiWaveBytes;
        auto off = [](int row, int col_bytes) { return row * 128 + (col_bytes ^ ((row & 7) << 4)); };
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int row = 32 * j + (lane & 31);
                    const int col = 32 * i + 8 * g + 4 * (lane >> 5);
                    uint2 w2;
                    w2.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
                    w2.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                    *reinterpret_cast<uint2*>(wl + off(row, 2 * col)) = w2;
                }
        __syncthreads();
        const int c = lane & 7;
        const int64_t n = n_base + 64 * wn + 8 * c;
        const bool vec = (N & 7) == 0 && n + 8 <= N;
        uint16_t* Yb = (uint16_t*)Y;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int row = 8 * it + (lane >> 3);
            const int64_t m = m_base + 64 * wm + row;
            if (m >= M) continue;
            const uint4 val = *reinterpret_cast<const uint4*>(wl + off(row, 16 * c));
            uint16_t* yr = Yb + m * N;
            if (vec) {
                *reinterpret_cast<uint4*>(yr + n) = val;
            } else {
                const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n + e < N) yr[n + e] = (uint16_t)((w4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            }
        }
        return;
    }
    const bool vec_ok = (N & 3) == 0;
    const QScale q = out_qscale<kOut>(nullptr);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t m = m_base + 64 * wm + 32 * j + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t n0 = n_base + 64 * wn + 32 * i + 8 * g + 4 * (lane >> 5);
                const f32x4 a = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                if (n0 < N) store4_raw<kOut>(Y, N, m, n0, a, vec_ok, q);
            }
    }
}

// ---------------------------------------------------------------------------
// Launchers: tiles_per_xcd tiles for each of the 8 XCDs (tile_coords).
template <bool kFp8, int kOut, bool kWPacked, bool kAPacked>
static hipError_t launch_big_t(const uint8_t* aq, const float* sa, int sa_pt, const uint8_t* wq, const float* sw,
                               void* y, int M, int N, int K, const float* qs, hipStream_t stream) {
    const int tiles = ((M + kBig - 1) / kBig) * ((N + kBig - 1) / kBig);
    const int per = (tiles + 7) / 8;
    dim3 grid((unsigned)(per * 8)), block(256);
    if (kFp8)
        gemm_big_fp8<kOut, kWPacked, kAPacked>
            <<<grid, block, 2 * 32 * kPackBlock, stream>>>(aq, sa, sa_pt, wq, sw, y, M, N, K, per, qs);
    else
        gemm_big_exact<kOut, kWPacked, kAPacked>
            <<<grid, block, kExSlots * kExSlot, stream>>>(aq, sa, sa_pt, wq, sw, y, M, N, K, per, qs);
    return hipGetLastError();
}

template <bool kFp8, bool kWPacked, bool kAPacked>
static hipError_t launch_big_y(const uint8_t* aq, const float* sa, int pt, const uint8_t* wq, const float* sw, void* y,
                               int out_kind, int M, int N, int K, const float* qs, hipStream_t stream) {
    if (out_kind == kOutBF16)
        return launch_big_t<kFp8, kOutBF16, kWPacked, kAPacked>(aq, sa, pt, wq, sw, y, M, N, K, qs, stream);
    if (out_kind == kOutE4M3)
        return launch_big_t<kFp8, kOutE4M3, kWPacked, kAPacked>(aq, sa, pt, wq, sw, y, M, N, K, qs, stream);
    return launch_big_t<kFp8, kOutF32, kWPacked, kAPacked>(aq, sa, pt, wq, sw, y, M, N, K, qs, stream);
}

template <bool kFp8>
static hipError_t launch_big_m(const uint8_t* aq, bool a_packed, const float* sa, int pt, const uint8_t* wq,
                               bool w_packed, const float* sw, void* y, int out_kind, int M, int N, int K,
                               const float* qs, hipStream_t stream) {
    if (a_packed)
        return w_packed ? launch_big_y<kFp8, true, true>(aq, sa, pt, wq, sw, y, out_kind, M, N, K, qs, stream)
                        : launch_big_y<kFp8, false, true>(aq, sa, pt, wq, sw, y, out_kind, M, N, K, qs, stream);
    return w_packed ? launch_big_y<kFp8, true, false>(aq, sa, pt, wq, sw, y, out_kind, M, N, K, qs, stream)
                    : launch_big_y<kFp8, false, false>(aq, sa, pt, wq, sw, y, out_kind, M, N, K, qs, stream);
}

hipError_t launch_big_gemm(const uint8_t* aq, bool a_packed, const float* sa, int sa_per_token, const uint8_t* wq,
                           bool w_packed, const float* sw, void* y, int out_kind, const float* out_scale, int M, int N,
                           int K, bool fp8_mfma, hipStream_t stream) {
    if (fp8_mfma)
        return launch_big_m<true>(aq, a_packed, sa, sa_per_token, wq, w_packed, sw, y, out_kind, M, N, K, out_scale,
                                  stream);
    return launch_big_m<false>(aq, a_packed, sa, sa_per_token, wq, w_packed, sw, y, out_kind, M, N, K, out_scale,
                               stream);
}

template <int kOut, bool kWPacked, bool kAPacked>
static hipError_t launch_big_bw_t(const uint8_t* aq, const float* sa, int sa_kmajor, const uint8_t* wq,
                                  const float* sw, void* y, int M, int N, int K, bool fp8_mfma, hipStream_t stream) {
    if (fp8_mfma) {
        const int tiles = ((M + kBig - 1) / kBig) * ((N + kBig - 1) / kBig);
        const int per = (tiles + 7) / 8;
        gemm_big_blockwise<kOut, kWPacked, kAPacked><<<dim3((unsigned)(per * 8)), dim3(512), 2 * kBwStage, stream>>>(
            aq, sa, sa_kmajor, wq, sw, y, M, N, K, per, nullptr);
    } else {
        const int tiles = ((M + kBig - 1) / kBig) * ((N + kBxTileN - 1) / kBxTileN);
        const int per = (tiles + 7) / 8;
        gemm_big_blockwise_exact<kOut, kWPacked, kAPacked>
            <<<dim3((unsigned)(per * 8)), dim3(512), kBxSlots * kBxSlot, stream>>>(aq, sa, sa_kmajor, wq, sw, y, M,
                                                                                  N, K, per);
    }
    return hipGetLastError();
}

hipError_t launch_big_blockwise(const uint8_t* aq, bool a_packed, const float* sa, bool sa_kmajor, const uint8_t* wq,
                                bool w_packed, const float* sw, void* y, bool y_bf16, int M, int N, int K,
                                bool fp8_mfma, hipStream_t stream) {
    const int km = sa_kmajor ? 1 : 0;
#define FP8SG_BW(YB, WP, AP) \
    launch_big_bw_t<(YB) ? kOutBF16 : kOutF32, WP, AP>(aq, sa, km, wq, sw, y, M, N, K, fp8_mfma, stream)
    if (y_bf16) {
        if (a_packed) return w_packed ? FP8SG_BW(true, true, true) : FP8SG_BW(true, false, true);
        return w_packed ? FP8SG_BW(true, true, false) : FP8SG_BW(true, false, false);
    }
    if (a_packed) return w_packed ? FP8SG_BW(false, true, true) : FP8SG_BW(false, false, true);
    return w_packed ? FP8SG_BW(false, true, false) : FP8SG_BW(false, false, false);
#undef FP8SG_BW
}

}  // namespace fp8sg
