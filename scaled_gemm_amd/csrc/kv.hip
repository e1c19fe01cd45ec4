// FP8 KV-cache kernels for gfx950 (quantization itself is the grouped
// given-scale quantizer in quant.hip with inner = D, nscales = H).
//
// Cache layout [B, S, H, D], head dim contiguous; one fp32 scale per kv head
// (FP8 Inference Explained, in depth -- "FP8 KV cache": per-tensor or
// per-attention-head scales; Quantization: FP8 inference and KV-cache
// quantization -- "Turning it on in an engine": per-head scales need
// calibration, the default is 1.0).
//
//  * calibrate: s_h = RN32(amax_h / max), amax_h over (b, s, d).  Three small
//    launches: clear, a bandwidth-bound maximum pass (per-block maxima combined
//    with an integer atomic max on the float bit patterns -- the order of a max
//    does not matter, so the result is deterministic), and the scale rule.
//  * dequantize: bf16(RN32(dec(code) * s_h)), 16 codes -> 16 bf16 per step.
//  * append: one new token per sequence, written at cache[b, pos[b]].
#include "fp8_device.h"
#include "launch.h"

namespace fp8sg {

__global__ void kv_clear(uint32_t* bits, int H) {
    for (int h = threadIdx.x; h < H; h += blockDim.x) bits[h] = 0u;
}

// Units of 16 bf16 (never straddling a head since D % 16 == 0).  The grid
// stride is a multiple of the head period (H * D / 16 units) whenever the
// launcher can arrange it; then a thread's head is fixed and its running maximum
// needs one atomic at the end.  Otherwise each unit updates the LDS maxima.
constexpr int kMaxCalHeads = 256;

__global__ __launch_bounds__(256) void kv_amax(const uint16_t* __restrict__ kv, int64_t nunits, int64_t d_units,
                                               int H, uint32_t* __restrict__ amax_bits) {
    __shared__ uint32_t lmax_lds[kMaxCalHeads];
    // per-block maxima in LDS when they fit; otherwise straight to the global maxima
    const bool in_lds = H <= kMaxCalHeads;
    uint32_t* lmax = in_lds ? lmax_lds : amax_bits;
    if (in_lds) {
        for (int h = threadIdx.x; h < H; h += blockDim.x) lmax[h] = 0u;
        __syncthreads();
    }
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t period = d_units * H;
    int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (stride % period == 0) {
        const int h = (int)((u / d_units) % H);
        float m = 0.0f;
        for (; u < nunits; u += stride) {
            const uint4 a = reinterpret_cast<const uint4*>(kv + (u << 4))[0];
            const uint4 b = reinterpret_cast<const uint4*>(kv + (u << 4))[1];
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                m = fmaxf(m, fmaxf(__builtin_fabsf(bf16_lo(w[j])), __builtin_fabsf(bf16_hi(w[j]))));
        }
        if (m > 0.0f) atomicMax(&lmax[h], __float_as_uint(m));
    } else {
        for (; u < nunits; u += stride) {
            const int h = (int)((u / d_units) % H);
            const uint4 a = reinterpret_cast<const uint4*>(kv + (u << 4))[0];
            const uint4 b = reinterpret_cast<const uint4*>(kv + (u << 4))[1];
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                m = fmaxf(m, fmaxf(__builtin_fabsf(bf16_lo(w[j])), __builtin_fabsf(bf16_hi(w[j]))));
            if (m > 0.0f) atomicMax(&lmax[h], __float_as_uint(m));
        }
    }
    if (in_lds) {
        __syncthreads();
        for (int h = threadIdx.x; h < H; h += blockDim.x)
            if (lmax[h]) atomicMax(&amax_bits[h], lmax[h]);
    }
}

__global__ void kv_finalize(uint32_t* bits, int H, float fmax) {
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        const float s = dynamic_scale(__uint_as_float(bits[h]), fmax);
        reinterpret_cast<float*>(bits)[h] = s;
    }
}

hipError_t launch_kv_calibrate(const uint16_t* kv, int64_t B, int64_t S, int64_t H, int64_t D, int fmt,
                               float* head_scales, hipStream_t stream) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(head_scales);
    kv_clear<<<1, 256, 0, stream>>>(bits, (int)H);
    const int64_t numel = B * S * H * D;
    if (numel > 0) {
        const int64_t nunits = numel / 16, d_units = D / 16, period = d_units * H;
        int64_t blocks = (nunits + 255) / 256;
        // four workgroups per CU, each looping over its share: more workgroups
        // only add atomics at the end (measured: 1024 -> 90 us, 4096 -> 103 us,
        // 8192 -> 129 us for bf16 [8, 32768, 8, 128])
        const int64_t cap = 1024;
        if (blocks > cap) blocks = cap;
        // make the stride a multiple of the head period when possible
        const int64_t stride = blocks * 256;
        if (blocks > 1 && stride % period != 0 && period <= 256 * 256) {
            int64_t b2 = blocks;
            while (b2 > 1 && (b2 * 256) % period != 0) --b2;
            if ((b2 * 256) % period == 0) blocks = b2;
        }
        kv_amax<<<(unsigned)blocks, 256, 0, stream>>>(kv, nunits, d_units, (int)H, bits);
    }
    kv_finalize<<<1, 256, 0, stream>>>(bits, (int)H, fmt == 0 ? kE4M3Max : kE5M2Max);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One unit of 16 codes per thread.  The bf16 values leave with ordinary
// stores: with non-temporal ones this pass (1 byte read, 2 written per element)
// measured 1.55x slower, whereas the quantizers (2 read, 1 written) gain 5-11%.
template <int kFmt, int kSel>
__global__ __launch_bounds__(256) void kv_dequant(const uint8_t* __restrict__ q, int64_t nunits, int64_t d_units,
                                                  int H, int shift, const float* __restrict__ scales,
                                                  uint16_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nunits; u += stride) {
        const uint4 c = load16_stream(q + (u << 4));  // codes are read once
        const float s = scales[unit_group<kSel>(u, d_units, H, shift)];
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x2 lo = unpack2<kFmt>(w[j], false);
            const f32x2 hi = unpack2<kFmt>(w[j], true);
            o[2 * j] = pack_bf16x2(lo[0] * s, lo[1] * s);
            o[2 * j + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
        }
        uint4* dst = reinterpret_cast<uint4*>(out + (u << 4));
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

hipError_t launch_kv_dequant(const uint8_t* kvq, int64_t numel, int64_t H, int64_t D, const float* head_scales,
                             int fmt, uint16_t* out, hipStream_t stream) {
    if (numel == 0) return hipSuccess;
    const int64_t nunits = numel / 16;
    // one unit per thread (the loop only strides past 2^31 workgroups): a grid
    // capped at 16 workgroups per CU ran at 4.5 TB/s, the full grid at 5.9 TB/s
    int64_t blocks = (nunits + 255) / 256;
    if (blocks > ((int64_t)1 << 31) - 1) blocks = ((int64_t)1 << 31) - 1;
    int shift;
    const int sel = unit_group_select(D / 16, (int)H, &shift);
#define FP8SG_KVD(F, S) \
    kv_dequant<F, S><<<(unsigned)blocks, 256, 0, stream>>>(kvq, nunits, D / 16, (int)H, shift, head_scales, out)
    if (fmt == 0) {
        if (sel == 0) FP8SG_KVD(0, 0); else if (sel == 1) FP8SG_KVD(0, 1); else FP8SG_KVD(0, 2);
    } else {
        if (sel == 0) FP8SG_KVD(1, 0); else if (sel == 1) FP8SG_KVD(1, 1); else FP8SG_KVD(1, 2);
    }
#undef FP8SG_KVD
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <int kFmt>
__global__ __launch_bounds__(256) void kv_append(const uint16_t* __restrict__ kv_new, const int32_t* __restrict__ pos,
                                                 int64_t B, int64_t S_cap, int64_t H, int64_t D,
                                                 const float* __restrict__ scales, uint8_t* __restrict__ cache) {
    constexpr float fmax = kFmt == 0 ? kE4M3Max : kE5M2Max;
    const int64_t d_units = D / 16, per_b = H * d_units, nunits = B * per_b;
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= nunits) return;
    const int64_t b = u / per_b, rem = u % per_b, h = rem / d_units, du = rem % d_units;
    const int32_t p = pos[b];
    if (p < 0 || p >= S_cap) return;
    const QScale sc = make_qscale(scales[h], fmax);
    const uint16_t* src = kv_new + ((b * H + h) * D + du * 16);
    const uint4 a = reinterpret_cast<const uint4*>(src)[0];
    const uint4 c = reinterpret_cast<const uint4*>(src)[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = pack4<kFmt>(quotient_given<false>(bf16_lo(w[2 * j]), sc), quotient_given<false>(bf16_hi(w[2 * j]), sc),
                           quotient_given<false>(bf16_lo(w[2 * j + 1]), sc),
                           quotient_given<false>(bf16_hi(w[2 * j + 1]), sc));
    uint8_t* dst = cache + (((b * S_cap + p) * H + h) * D + du * 16);
    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_kv_append(const uint16_t* kv_new, const int32_t* pos, int64_t B, int64_t S_cap, int64_t H,
                            int64_t D, const float* head_scales, int fmt, uint8_t* cache, hipStream_t stream) {
    const int64_t nunits = B * H * (D / 16);
    if (nunits == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((nunits + 255) / 256);
    if (fmt == 0) kv_append<0><<<blocks, 256, 0, stream>>>(kv_new, pos, B, S_cap, H, D, head_scales, cache);
    else kv_append<1><<<blocks, 256, 0, stream>>>(kv_new, pos, B, S_cap, H, D, head_scales, cache);
    return hipGetLastError();
}

}  // namespace fp8sg
