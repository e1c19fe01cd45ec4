// Decode attention over an FP8 KV cache for gfx950.
//
// One decode step: query q[b, h, :] (bf16) attends over the first L[b]
// positions of the cached keys and values of its kv head g = h / G (grouped
// query heads, G = Hq / Hkv).  The cache holds E4M3 or E5M2 codes with one
// scale per kv head, read back as code value times scale, and the attention is
// computed in higher precision (FP8 Inference Explained, in depth -- "FP8 KV
// cache": per-attention-head scales; backends that do not compute in FP8 read
// the cache back and compute in higher precision):
//     s_t = scale * q . K_t,   p = softmax(s),   o = sum_t p_t V_t.
// The softmax runs block by block with a running maximum and a running sum,
// the partial outputs rescaled by exp(m_old - m_new) ("FlashAttention
// v1/v2/v3/v4" post -- "The trick that made it all possible: online softmax":
// the recurrence gives exactly the standard result).
//
// Both scales are constant along their sums and are applied once: s_K with
// the softmax scale to the dot products, s_V to the final output.  Every FP8
// code is exactly a bf16 value, so the dot products q . dec(K_t) run on the
// bf16 matrix cores with exact products and fp32 sums; p.V runs on the vector
// ALU in fp32.
//
// Two kernels.  attn_split: one workgroup per (sequence, kv head, chunk of
// kChunk positions); its 4 waves take blocks of 64 positions round-robin and
// each keeps (m, l, o) for the G query heads of the kv head; the waves combine
// through LDS and the workgroup writes one partial (m, l, o) per query head to
// the workspace.  attn_combine: one workgroup per (sequence, query head) adds
// the chunks' partials in chunk order (deterministic), divides by the total
// sum, applies s_V and writes bf16 (round to nearest even) or fp32.
#include "fp8_device.h"
#include "launch.h"

namespace fp8sg {

typedef float f32x4a __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8a __attribute__((ext_vector_type(8)));

constexpr int kAttnD = 128;        // head dimension
constexpr int kChunk = 1024;       // positions per workgroup
constexpr int kBlk = 64;           // positions per wave step
constexpr int kPartFloats = kAttnD + 2;  // o[128], m, l

// Eight codes -> eight bf16 (exact), for the matrix cores.
template <int kFmt>
__device__ __forceinline__ bf16x8a codes8_to_bf16(uint32_t w0, uint32_t w1) {
    uint32_t u[4];
    if (kFmt == 0) {
        u[0] = e4m3x2_to_bf16x2(w0, false);
        u[1] = e4m3x2_to_bf16x2(w0, true);
        u[2] = e4m3x2_to_bf16x2(w1, false);
        u[3] = e4m3x2_to_bf16x2(w1, true);
    } else {
        bf16x2 h[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w0, 1.0f, false),
                       __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w0, 1.0f, true),
                       __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w1, 1.0f, false),
                       __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w1, 1.0f, true)};
        __builtin_memcpy(u, h, 16);
    }
    bf16x8a v;
    __builtin_memcpy(&v, u, 16);
    return v;
}

// Sixteen codes -> sixteen floats (exact).
template <int kFmt>
__device__ __forceinline__ void codes16_to_f32(uint4 c, float (&v)[16]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 a = unpack2<kFmt>(w[i], false), b = unpack2<kFmt>(w[i], true);
        v[4 * i] = a[0];
        v[4 * i + 1] = a[1];
        v[4 * i + 2] = b[0];
        v[4 * i + 3] = b[1];
    }
}

__device__ __forceinline__ float wave_max16(float v) {  // over lanes with the same lane % 16
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

__device__ __forceinline__ float wave_sum16(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}

// Workgroup (b, g, chunk c): grid x = c + nchunk * (g + Hkv * b).
template <int kFmt, int kG>
__global__ __launch_bounds__(256) void attn_split(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc,
                                                  const uint8_t* __restrict__ vc, const float* __restrict__ k_scales,
                                                  const int32_t* __restrict__ lengths, int S_cap, int Hkv,
                                                  int nchunk, float softmax_scale, float* __restrict__ part) {
    __shared__ float p_lds[4][kG][kBlk];
    __shared__ float w_m[4][kG], w_l[4][kG];
    __shared__ float w_o[4][kG][kAttnD];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = (int)(blockIdx.x % (unsigned)nchunk);
    const int bg = (int)(blockIdx.x / (unsigned)nchunk);
    const int g = bg % Hkv, b = bg / Hkv;
    int L = lengths[b];
    L = L < 0 ? 0 : (L > S_cap ? S_cap : L);
    const int t_begin = c * kChunk;
    const int t_end = t_begin + kChunk < L ? t_begin + kChunk : L;
    float* out = part + ((size_t)bg * nchunk + c) * kG * kPartFloats;
    if (t_begin >= t_end) {  // nothing here: a neutral partial
        for (int i = threadIdx.x; i < kG * kPartFloats; i += blockDim.x) {
            const int f = i % kPartFloats;
            out[i] = f == kAttnD ? -__builtin_inff() : 0.0f;
        }
        return;
    }
    const int Hq = Hkv * kG;
    const int64_t row_stride = (int64_t)Hkv * kAttnD;  // bytes between positions of one kv head
    const uint8_t* kb = kc + ((int64_t)b * S_cap * Hkv + g) * kAttnD;
    const uint8_t* vb = vc + ((int64_t)b * S_cap * Hkv + g) * kAttnD;
    const float xs = k_scales[g] * softmax_scale;

    // B operand of the score products: q^T, lane l = head l % 16 (zero past G),
    // dims 32 (l / 16) + 8 s .. + 8 in step s (the A operand uses the same dims).
    const int jh = lane & 15, kq = lane >> 4;
    bf16x8a qf[4];
    {
        const bool valid = jh < kG;
        const uint16_t* qr = q + ((int64_t)b * Hq + g * kG + (valid ? jh : 0)) * kAttnD + 32 * kq;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 u = *reinterpret_cast<const uint4*>(qr + 8 * s);
            if (!valid) u = make_uint4(0, 0, 0, 0);
            __builtin_memcpy(&qf[s], &u, 16);
        }
    }

    // p.V lane roles: dims 16 dg .. 16 dg + 15 of position slot ps of each 8.
    const int dg = lane & 7, ps = lane >> 3;
    float o[kG][16];
#pragma unroll
    for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int d = 0; d < 16; ++d) o[h][d] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;  // for head jh (lanes with jh < kG)

    // K slices for the 4 score tiles and V slices for the 8 p.V steps of the
    // block at t0, addressed from the block's uniform base with 32-bit per-lane
    // offsets; positions past t_end are clamped to the last valid one (their
    // scores are masked).  The row stride (Hkv * 128 < 2^23 bytes) and the
    // position within the block (< 64) multiply in 24 bits.
    const uint32_t rs = (uint32_t)row_stride;
    auto load_block = [&](uint4 (&kr)[4][2], uint4 (&vr)[8], int t0) __attribute__((always_inline)) {
        const int last = t_end - 1 - t0;   // the last valid position, relative to t0
        const uint8_t* kbase = kb + (int64_t)t0 * row_stride;
        const uint8_t* vbase = vb + (int64_t)t0 * row_stride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * i + jh < last ? 16 * i + jh : last;
            const uint32_t off = (uint32_t)__umul24((uint32_t)r, rs) + (uint32_t)(32 * kq);
            const uint4* p = reinterpret_cast<const uint4*>(kbase + (uint64_t)off);
            kr[i][0] = p[0];
            kr[i][1] = p[1];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = 8 * k + ps < last ? 8 * k + ps : last;
            const uint32_t off = (uint32_t)__umul24((uint32_t)r, rs) + (uint32_t)(16 * dg);
            vr[k] = *reinterpret_cast<const uint4*>(vbase + (uint64_t)off);
        }
    };
    // One block with its fragments in (kr, vr); the block four blocks on (this
    // wave's next one) is loaded into (kn, vn) first.
    auto block = [&](uint4 (&kr)[4][2], uint4 (&vr)[8], uint4 (&kn)[4][2], uint4 (&vn)[8], int t0)
        __attribute__((always_inline)) {
        if (t0 + 4 * kBlk < t_end) load_block(kn, vn, t0 + 4 * kBlk);
        // ---- scores: 4 tiles of 16 positions x 16 head columns
        float x[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4a acc = {0.0f, 0.0f, 0.0f, 0.0f};
            const uint32_t w[8] = {kr[i][0].x, kr[i][0].y, kr[i][0].z, kr[i][0].w,
                                   kr[i][1].x, kr[i][1].y, kr[i][1].z, kr[i][1].w};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes8_to_bf16<kFmt>(w[2 * s], w[2 * s + 1]), qf[s], acc,
                                                              0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 16 * i + 4 * kq + r;
                x[i][r] = t < t_end ? acc[r] * xs : -__builtin_inff();
            }
        }
        // ---- online softmax update for head jh
        float bm = x[0][0];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) bm = fmaxf(bm, x[i][r]);
        bm = wave_max16(bm);
        const float m_new = fmaxf(m_run, bm);  // finite: every block has a valid position
        const float alpha = __expf(m_run - m_new);
        // no head of the kv head raised its maximum: every rescale factor is 1 and o stays as it is
        const bool rescale = __builtin_amdgcn_ballot_w64(jh < kG && m_new != m_run) != 0;
        float bs = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float e[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                e[r] = __expf(x[i][r] - m_new);
                bs += e[r];
            }
            if (jh < kG)
                *reinterpret_cast<float4*>(&p_lds[wave][jh][16 * i + 4 * kq]) = make_float4(e[0], e[1], e[2], e[3]);
        }
        bs = wave_sum16(bs);
        l_run = alpha * l_run + bs;
        m_run = m_new;
        if (rescale) {
            // every lane needs each head's rescale factor: lane h holds it
            float al[kG];
#pragma unroll
            for (int h = 0; h < kG; ++h) al[h] = __shfl(alpha, h, 64);
#pragma unroll
            for (int h = 0; h < kG; ++h)
#pragma unroll
                for (int d = 0; d < 16; ++d) o[h][d] *= al[h];
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's p values are in LDS
        // ---- p.V for this wave's 64 positions
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float v[16];
            codes16_to_f32<kFmt>(vr[k], v);
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                const float ph = p_lds[wave][h][8 * k + ps];
#pragma unroll
                for (int d = 0; d < 16; ++d) o[h][d] = __builtin_fmaf(ph, v[d], o[h][d]);
            }
        }
        __builtin_amdgcn_wave_barrier();
    };
    uint4 kr[4][2], vr[8];
    if (t_begin + wave * kBlk < t_end) load_block(kr, vr, t_begin + wave * kBlk);
    for (int t0 = t_begin + wave * kBlk; t0 < t_end; t0 += 4 * kBlk) {
        uint4 kn[4][2], vn[8];
        block(kr, vr, kn, vn, t0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kr[i][0] = kn[i][0];
            kr[i][1] = kn[i][1];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) vr[k] = vn[k];
    }

    // ---- combine the 8 position slots of each dim group (xor over lane bits 3..5)
#pragma unroll
    for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int d = 0; d < 16; ++d) {
            float v = o[h][d];
            v += __shfl_xor(v, 8, 64);
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            o[h][d] = v;
        }
    // ---- combine the 4 waves through LDS (waves without a block contribute m = -inf, l = 0, o = 0)
    if (lane < kG) {
        w_m[wave][lane] = m_run;
        w_l[wave][lane] = l_run;
    }
    if (ps == 0) {
#pragma unroll
        for (int h = 0; h < kG; ++h)
#pragma unroll
            for (int d = 0; d < 16; ++d) w_o[wave][h][16 * dg + d] = o[h][d];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kG * kAttnD; i += blockDim.x) {
        const int h = i / kAttnD, d = i % kAttnD;
        float M = w_m[0][h];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, w_m[w][h]);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = w_m[w][h] == -__builtin_inff() ? 0.0f : __expf(w_m[w][h] - M);
            acc += f * w_o[w][h][d];
            lsum += f * w_l[w][h];
        }
        float* ph = out + h * kPartFloats;
        ph[d] = acc;
        if (d == 0) {
            ph[kAttnD] = M;
            ph[kAttnD + 1] = lsum;
        }
    }
}

// Workgroup (b, h), one thread per dimension: the chunks' partials in chunk
// order.  The chunk maxima and sums are read by all threads at once (one chunk
// per thread) and their weights exp(m_c - M) kept in LDS; each thread adds its
// dimension of the chunks' outputs, the first 32 chunks' values loaded together
// with the maxima and sums, any further chunks 8 per batch of loads.
constexpr int kMaxChunks = 1024;  // S_cap <= 2^20

template <bool kOutBf16>
__global__ __launch_bounds__(128) void attn_combine(const float* __restrict__ part, const float* __restrict__ v_scales,
                                                    const int32_t* __restrict__ lengths, int S_cap, int Hkv, int G,
                                                    int nchunk, void* __restrict__ out) {
    __shared__ float wgt[kMaxChunks];
    __shared__ float lsm[kMaxChunks];
    __shared__ float red[2];
    const int h = (int)(blockIdx.x % (unsigned)(Hkv * G));
    const int b = (int)(blockIdx.x / (unsigned)(Hkv * G));
    const int g = h / G, j = h % G;
    const int d = threadIdx.x;
    int L = lengths[b];
    L = L < 0 ? 0 : (L > S_cap ? S_cap : L);
    const int nc = (L + kChunk - 1) / kChunk;
    const size_t stride = (size_t)G * kPartFloats;
    const float* pb = part + ((size_t)(b * Hkv + g) * nchunk) * stride + (size_t)j * kPartFloats;
    // The loads go out together: this thread's dimension of the first kPre chunks'
    // outputs (they do not depend on the maxima) and the maximum and sum of chunk
    // d (and d + 128, ...), so the kernel waits for memory about once.
    constexpr int kPre = 32;
    float ov[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) ov[u] = u < nc ? pb[(size_t)u * stride + d] : 0.0f;
    float mx = -__builtin_inff();
    for (int c = d; c < nc; c += blockDim.x) {
        const float m = pb[(size_t)c * stride + kAttnD];
        wgt[c] = m;
        lsm[c] = pb[(size_t)c * stride + kAttnD + 1];
        mx = fmaxf(mx, m);
    }
    // chunk maxima -> M (every chunk c < nc holds at least one position, so its m is finite)
    mx = wave_max(mx);
    if ((d & 63) == 0) red[d >> 6] = mx;
    __syncthreads();
    const float M = fmaxf(red[0], red[1]);
    __syncthreads();
    float ls = 0.0f;
    for (int c = d; c < nc; c += blockDim.x) {
        const float f = __expf(wgt[c] - M);
        wgt[c] = f;
        ls += f * lsm[c];
    }
    ls = ls + __shfl_xor(ls, 32, 64);
    ls = ls + __shfl_xor(ls, 16, 64);
    ls = ls + __shfl_xor(ls, 8, 64);
    ls = ls + __shfl_xor(ls, 4, 64);
    ls = ls + __shfl_xor(ls, 2, 64);
    ls = ls + __shfl_xor(ls, 1, 64);
    if ((d & 63) == 0) red[d >> 6] = ls;
    __syncthreads();
    const float lsum = red[0] + red[1];
    // the weighted outputs in chunk order
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < kPre; ++u)
        if (u < nc) acc += wgt[u] * ov[u];
    int c = kPre;
    for (; c + 8 <= nc; c += 8) {
        float o8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o8[u] = pb[(size_t)(c + u) * stride + d];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += wgt[c + u] * o8[u];
    }
    for (; c < nc; ++c) acc += wgt[c] * pb[(size_t)c * stride + d];
    const float r = nc > 0 ? (acc / lsum) * v_scales[g] : 0.0f;
    const size_t o_idx = ((size_t)b * Hkv * G + h) * kAttnD + d;
    if (kOutBf16) ((uint16_t*)out)[o_idx] = (uint16_t)(pack_bf16x2(r, 0.0f) & 0xFFFFu);
    else ((float*)out)[o_idx] = r;
}

size_t attn_workspace_bytes(int64_t B, int64_t S_cap, int64_t Hq, int64_t Hkv) {
    const int64_t nchunk = (S_cap + kChunk - 1) / kChunk;
    const int64_t G = Hkv > 0 ? Hq / Hkv : 0;
    return (size_t)(B * Hkv * (nchunk > 0 ? nchunk : 1) * G * kPartFloats) * sizeof(float);
}

template <int kFmt, int kG>
static void launch_split(const uint16_t* q, const uint8_t* kc, const uint8_t* vc, const float* k_scales,
                         const int32_t* lengths, int B, int S_cap, int Hkv, int nchunk, float scale, float* part,
                         hipStream_t stream) {
    attn_split<kFmt, kG><<<dim3((unsigned)(B * Hkv * nchunk)), dim3(256), 0, stream>>>(
        q, kc, vc, k_scales, lengths, S_cap, Hkv, nchunk, scale, part);
}

template <int kFmt>
static void launch_split_g(int G, const uint16_t* q, const uint8_t* kc, const uint8_t* vc, const float* k_scales,
                           const int32_t* lengths, int B, int S_cap, int Hkv, int nchunk, float scale, float* part,
                           hipStream_t stream) {
    switch (G) {
        case 1: launch_split<kFmt, 1>(q, kc, vc, k_scales, lengths, B, S_cap, Hkv, nchunk, scale, part, stream); break;
        case 2: launch_split<kFmt, 2>(q, kc, vc, k_scales, lengths, B, S_cap, Hkv, nchunk, scale, part, stream); break;
        case 4: launch_split<kFmt, 4>(q, kc, vc, k_scales, lengths, B, S_cap, Hkv, nchunk, scale, part, stream); break;
        default: launch_split<kFmt, 8>(q, kc, vc, k_scales, lengths, B, S_cap, Hkv, nchunk, scale, part, stream); break;
    }
}

hipError_t launch_kv_decode_attention(const uint16_t* q, const uint8_t* kc, const uint8_t* vc, const float* k_scales,
                                      const float* v_scales, int fmt, const int32_t* lengths, int64_t B,
                                      int64_t S_cap, int64_t Hq, int64_t Hkv, float scale, void* out, bool out_bf16,
                                      float* part, hipStream_t stream) {
    if (B == 0 || Hq == 0) return hipSuccess;
    const int G = (int)(Hq / Hkv);
    const int nchunk = (int)((S_cap + kChunk - 1) / kChunk);
    if (nchunk > 0) {
        if (fmt == 0) launch_split_g<0>(G, q, kc, vc, k_scales, lengths, (int)B, (int)S_cap, (int)Hkv, nchunk, scale, part, stream);
        else launch_split_g<1>(G, q, kc, vc, k_scales, lengths, (int)B, (int)S_cap, (int)Hkv, nchunk, scale, part, stream);
    }
    const dim3 grid((unsigned)(B * Hq)), block(kAttnD);
    if (out_bf16)
        attn_combine<true><<<grid, block, 0, stream>>>(part, v_scales, lengths, (int)S_cap, (int)Hkv, G, nchunk, out);
    else
        attn_combine<false><<<grid, block, 0, stream>>>(part, v_scales, lengths, (int)S_cap, (int)Hkv, G, nchunk, out);
    return hipGetLastError();
}

}  // namespace fp8sg
