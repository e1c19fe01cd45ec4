// Device helpers for the gfx950 FP8 kernels: exact float32 quotient, FP8
// packing/unpacking, bf16 conversion and reductions.
//
// Instruction facts these helpers rely on (checked on gfx950 against an
// independent CPU encoder over every float32 bit pattern):
//  * v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 round to nearest even into OCP E4M3 /
//    E5M2 exactly for every finite |t| below the format maximum, subnormals and
//    signed zero included.  They do NOT saturate (E4M3 turns values from 480 up
//    into NaN) and give the negative-NaN code for every NaN input, so callers
//    bound magnitudes first.
//  * v_cvt_pk_f32_fp8 / v_cvt_pk_f32_bf8 and v_cvt_scalef32_pk_bf16_fp8 with
//    scale 1.0 decode exactly; v_cvt_pk_bf16_f32 rounds to nearest even.
//  * The compiler's float division (v_div_scale/fmas/fixup) is correctly
//    rounded, and so is 1.0f / s.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp8sg {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Everything a thread needs to turn x into RN32(x / s) without a per-element
// division.  With r = RN32(1/s) (correctly rounded), q0 = RN(|x| r) is within
// two units in the last place of |x| / s, and each fused correction
// q <- RN(q + RN(|x| - q s) r) (Markstein's scheme) moves it to the correctly
// rounded quotient; one correction is exact for bf16 inputs (8 significant
// bits; checked exhaustively over every bf16 significand against every float32
// significand of s), two for float32 inputs.  The scheme needs s and 1/s to be
// normal with room to spare, so scales outside [2^-60, 2^60] fall back to the
// hardware-exact division.
struct QScale {
    float s;      // the stored scale
    float r;      // RN32(1 / s)
    float c;      // magnitude bound: RN32(fmax * s); |x| beyond it saturates anyway
    int fast;     // s in [2^-60, 2^60]
};

__device__ __forceinline__ QScale make_qscale(float s, float fmax) {
    QScale p;
    p.s = s;
    p.r = 1.0f / s;
    p.c = fmax * s;
    p.fast = (s >= 0x1p-60f) && (s <= 0x1p60f);
    return p;
}

// RN32(|x| / s) for |x| already bounded by the caller; kTwoCorrections for
// float32 inputs.
template <bool kTwoCorrections>
__device__ __forceinline__ float abs_quotient(float a, const QScale& p) {
    if (p.fast) {
        float q = a * p.r;
        float e = __builtin_fmaf(-q, p.s, a);
        q = __builtin_fmaf(e, p.r, q);
        if (kTwoCorrections) {
            e = __builtin_fmaf(-q, p.s, a);
            q = __builtin_fmaf(e, p.r, q);
        }
        return q;
    }
    return a / p.s;
}

// Signed quotient for the dynamic (amax-derived) path: |x| <= amax, so the
// quotient never exceeds fmax by more than a rounding, and stays far below the
// converter's overflow point.
template <bool kTwoCorrections>
__device__ __forceinline__ float quotient_dynamic(float x, const QScale& p) {
    return __builtin_copysignf(abs_quotient<kTwoCorrections>(__builtin_fabsf(x), p), x);
}

// abs_quotient with the range test already taken by the caller (kFast ==
// p.fast), so a loop over many values carries no branch per value.
template <bool kTwoCorrections, bool kFast>
__device__ __forceinline__ float abs_quotient_known(float a, const QScale& p) {
    if (kFast) {
        float q = a * p.r;
        float e = __builtin_fmaf(-q, p.s, a);
        q = __builtin_fmaf(e, p.r, q);
        if (kTwoCorrections) {
            e = __builtin_fmaf(-q, p.s, a);
            q = __builtin_fmaf(e, p.r, q);
        }
        return q;
    }
    return a / p.s;
}

// Signed quotient for the given-scale path: |x| is first bounded by
// c = RN32(fmax s) with a NaN-propagating minimum; every |x| >= c encodes to
// the maximum code, and the bounded quotient RN32(c / s) lies within a
// rounding of fmax, so it also encodes to the maximum.  +-inf saturates, NaN
// stays NaN.
template <bool kTwoCorrections>
__device__ __forceinline__ float quotient_given(float x, const QScale& p) {
    float a = __builtin_elementwise_minimum(__builtin_fabsf(x), p.c);
    return __builtin_copysignf(abs_quotient<kTwoCorrections>(a, p), x);
}

template <bool kTwoCorrections, bool kFast>
__device__ __forceinline__ float quotient_dynamic_known(float x, const QScale& p) {
    return __builtin_copysignf(abs_quotient_known<kTwoCorrections, kFast>(__builtin_fabsf(x), p), x);
}

template <bool kTwoCorrections, bool kFast>
__device__ __forceinline__ float quotient_given_known(float x, const QScale& p) {
    float a = __builtin_elementwise_minimum(__builtin_fabsf(x), p.c);
    return __builtin_copysignf(abs_quotient_known<kTwoCorrections, kFast>(a, p), x);
}

// Four quotients -> four codes in one dword (byte i = code of t_i).
template <int kFmt>  // 0 = E4M3, 1 = E5M2
__device__ __forceinline__ uint32_t pack4(float t0, float t1, float t2, float t3) {
    int w;
    if (kFmt == 0) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(t2, t3, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(t0, t1, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(t2, t3, w, true);
    }
    return (uint32_t)w;
}

// Two codes (bytes 0,1 or 2,3 of w) -> two floats, exact.
template <int kFmt>
__device__ __forceinline__ f32x2 unpack2(uint32_t w, bool hi) {
    if (kFmt == 0) return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    return hi ? __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
}

// Two floats -> two bf16 (round to nearest even) packed in a dword, low first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 h = __builtin_convertvector(v, bf16x2);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

// Two E4M3 codes (bytes 0,1 or 2,3 of w) -> two bf16 in a dword, exact.
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
    bf16x2 h = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Block-wide maximum of non-negative values; every thread gets the result.
// `red` must hold one float per wave of the block.
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = (blockDim.x + 63) >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
    for (int i = 1; i < nwaves; ++i) m = fmaxf(m, red[i]);
    __syncthreads();
    return m;
}

// Dynamic scale rule: s = RN32(amax / fmax), 1.0 when that is 0.
__device__ __forceinline__ float dynamic_scale(float amax, float fmax) {
    float s = amax / fmax;
    return s == 0.0f ? 1.0f : s;
}

// A 16-byte load with the non-temporal hint, for operands that a kernel
// streams through once (their lines need not stay in the caches).
__device__ __forceinline__ uint4 load16_stream(const void* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// A 16-byte store with the non-temporal hint, for results that the kernel
// writes once and does not read back (measured on a 2-byte-read / 1-byte-write
// stream of 100 MB: 17.0 us with these stores against 19.0 us with plain ones).
__device__ __forceinline__ void store16_stream(void* p, uint4 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
}

// The same for 8 bytes.
__device__ __forceinline__ void store8_stream(void* p, uint2 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
}

// Scale group of 16-element unit u when groups of inner_units units cycle over
// nscales scales: kSel 0 -- one scale for the tensor; 1 -- inner_units and
// nscales powers of two (a shift and a mask); 2 -- any (64-bit division).
template <int kSel>
__device__ __forceinline__ int unit_group(int64_t u, int64_t inner_units, int nscales, int shift) {
    if (kSel == 0) return 0;
    if (kSel == 1) return (int)(u >> shift) & (nscales - 1);
    return (int)((u / inner_units) % nscales);
}

// The kSel that fits (inner_units >= 1, nscales >= 1), and the shift for kSel 1.
inline int unit_group_select(int64_t inner_units, int nscales, int* shift) {
    const bool pow2 = (inner_units & (inner_units - 1)) == 0 && (nscales & (nscales - 1)) == 0;
    *shift = pow2 ? __builtin_ctzll((unsigned long long)inner_units) : 0;
    return nscales == 1 ? 0 : (pow2 ? 1 : 2);
}

// An empty asm statement that the compiler must assume rewrites the four
// words: values derived from them before it are not reused after it, which
// keeps a kernel from holding both raw words and their unpacked floats live.
__device__ __forceinline__ void opaque_words(uint4& v) {
    uint32_t a = v.x, b = v.y, c = v.z, d = v.w;
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
    v = make_uint4(a, b, c, d);
}

// A chunk is 8 consecutive elements: one 16-byte load for bf16, two for fp32.
template <typename InT>
__device__ __forceinline__ void load_chunk(const InT* p, float (&v)[8]);

// The same with streaming loads.
template <typename InT>
__device__ __forceinline__ void load_chunk_stream(const InT* p, float (&v)[8]) {
    const uint4 a = load16_stream(p);
    if constexpr (sizeof(InT) == 2) {
        v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
        v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
    } else {
        const uint4 b = load16_stream(p + 4);
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z);
        v[3] = __uint_as_float(a.w); v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    }
}

template <>
__device__ __forceinline__ void load_chunk<uint16_t>(const uint16_t* p, float (&v)[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}

template <>
__device__ __forceinline__ void load_chunk<float>(const float* p, float (&v)[8]) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Eight values -> eight E4M3 codes with the scale's range test taken once for
// the chunk (the scale is the row's).
template <typename InT>
__device__ __forceinline__ uint2 encode_chunk_dynamic(const float (&v)[8], const QScale& p) {
    constexpr bool kTwo = sizeof(InT) == 4;
    auto enc = [&](auto fast_tag) __attribute__((always_inline)) {
        constexpr bool kFast = decltype(fast_tag)::value;
        uint2 o;
        o.x = pack4<0>(quotient_dynamic_known<kTwo, kFast>(v[0], p), quotient_dynamic_known<kTwo, kFast>(v[1], p),
                       quotient_dynamic_known<kTwo, kFast>(v[2], p), quotient_dynamic_known<kTwo, kFast>(v[3], p));
        o.y = pack4<0>(quotient_dynamic_known<kTwo, kFast>(v[4], p), quotient_dynamic_known<kTwo, kFast>(v[5], p),
                       quotient_dynamic_known<kTwo, kFast>(v[6], p), quotient_dynamic_known<kTwo, kFast>(v[7], p));
        return o;
    };
    return p.fast ? enc(std::true_type{}) : enc(std::false_type{});
}

}  // namespace fp8sg
