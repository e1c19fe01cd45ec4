/*
 * fp8sg — FP8 W8A8 scaled GEMM, FP8 quantizers and FP8 KV-cache passes for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Every pointer argument is a DEVICE pointer (memory on the current HIP
 *   device), except where stated.  The caller allocates and frees every buffer;
 *   the library allocates no memory and keeps no per-call state.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *   work is enqueued asynchronously on it; results are visible after the caller
 *   synchronises the stream.  Scales live in device memory, so calls do not
 *   synchronise with the host.
 * - A call only launches kernels on `stream`: no allocation, no memset, no
 *   host synchronisation, no other stream.  Sequences of calls can therefore be
 *   captured into a HIP graph and replayed (the first call on a device queries
 *   its properties once; make it before capturing).
 * - Tensors are dense and row-major (last extent contiguous).  Data pointers
 *   must be 16-byte aligned; scale pointers 4-byte aligned.
 * - FP8 data travels as raw bytes (uint8): E4M3 is the OCP "fn" variant
 *   (bias 7, max 448, no infinities, S.1111.111 = NaN); E5M2 has bias 15,
 *   max 57344, infinities and NaNs.
 * - Quantization follows one rule everywhere: the stored scale s is the
 *   dequantization factor (value ~ s * code); a value x is encoded as
 *   FMT(RN32(x / s)), the IEEE-754 binary32 quotient rounded to the nearest FP8
 *   value, ties to even, saturating at +-max (also for +-inf); the sign of zero
 *   is kept; NaN gives a NaN code.  A dynamic scale is s = RN32(amax / max),
 *   or 1.0 when that is 0.  Quantized codes and scales are bit-exact with this
 *   rule.  (FP8 Inference Explained, in depth -- "The numbers in one byte",
 *   "Scales and their granularity"; Quantization: FP8 inference and KV-cache
 *   quantization -- "Dynamic scales or static scales".)
 * - Errors: arguments are checked synchronously, before any HIP call, and a
 *   non-OK status is returned with nothing enqueued.  No C++ exception crosses
 *   the ABI.  Work of size 0 (M == 0, numel == 0, ...) returns FP8SG_OK without
 *   launching.  Faults inside a kernel surface at the caller's stream
 *   synchronisation.
 * - Inputs containing NaN or infinity are out of contract for the dynamic
 *   (amax-based) paths, whose scale would itself be non-finite.
 */
#ifndef FP8SG_H
#define FP8SG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8sg_status {
    FP8SG_OK = 0,
    FP8SG_E_NULL = 1,       /* a required pointer is NULL                              */
    FP8SG_E_SHAPE = 2,      /* a size is negative, too large, or breaks a multiple-of rule */
    FP8SG_E_ALIGN = 3,      /* a pointer is not aligned as required                    */
    FP8SG_E_DTYPE = 4,      /* unsupported dtype / format / mode value                 */
    FP8SG_E_DEVICE = 5,     /* no HIP device, or the current device is not gfx950      */
    FP8SG_E_LAUNCH = 6,     /* a kernel launch failed (hipGetLastError)                */
    FP8SG_E_WORKSPACE = 7,  /* workspace missing or smaller than the size query says   */
    FP8SG_E_SCRATCH = 8     /* fp8_scaled_gemm_noalloc: the call needs more than
                               FP8SG_SCRATCH_BYTES of scratch                           */
} fp8sg_status;

/* Bytes of the static device scratch behind fp8_scaled_gemm_noalloc (16 MiB). */
#define FP8SG_SCRATCH_BYTES (16u << 20)

typedef enum fp8sg_dtype {
    FP8SG_F32 = 0,
    FP8SG_BF16 = 1,
    FP8SG_E4M3 = 2,
    FP8SG_E5M2 = 3
} fp8sg_dtype;

/* How the activation scale of fp8_scaled_gemm is organised. */
typedef enum fp8sg_scale_mode {
    FP8SG_SCALE_PER_TOKEN = 0,   /* one fp32 scale per row of A ([M])   */
    FP8SG_SCALE_PER_TENSOR = 1   /* one fp32 scale for all of A ([1])   */
} fp8sg_scale_mode;

/* How fp8_scaled_gemm accumulates the FP8 x FP8 products. */
typedef enum fp8sg_accum {
    /* Products formed exactly and summed in fp32 (the FP8 codes are widened
     * exactly to bf16 and multiplied on the bf16 matrix cores).  The
     * accumulator meets |acc - exact| <= 1e-5 * sum_k |a_k w_k|. */
    FP8SG_ACCUM_EXACT = 0,
    /* Native FP8 matrix cores.  On gfx950 each instruction sums its products in
     * groups of 8 consecutive k, aligning them to the group's largest product
     * and truncating below 2^(e_max - 13); group sums are then added in fp32.
     * Twice the peak rate of FP8SG_ACCUM_EXACT, with that error. */
    FP8SG_ACCUM_MFMA_FP8 = 1
} fp8sg_accum;

/* Memory layout of the E4M3 operands given to fp8_scaled_gemm: the `layout`
 * argument is FP8SG_W_ROW_MAJOR (0) or a bitwise OR of the flags below. */
typedef enum fp8sg_layout {
    /* Both operands row-major: A_q [M, K] and W_q [N, K], K contiguous (W_q^T is
     * the column-major "B"). */
    FP8SG_W_ROW_MAJOR = 0,
    /* W_q in matrix-core fragment order, produced by fp8_pack_weights: rows
     * padded to a multiple of 16 with zero codes; the 16-row x 128-k block
     * (t, kb) is 2048 contiguous bytes at offset (t * K/128 + kb) * 2048; inside
     * a block, byte j of lane l's first 16-byte half is at l * 16 + j and of its
     * second half at 1024 + l * 16 + j, where lane l covers row 16 t + l % 16
     * and the bytes [32 (l / 16), 32 (l / 16) + 32) of the block's 128 k. */
    FP8SG_W_PACKED = 1,
    /* A_q (a_dtype FP8SG_E4M3 only) in the same fragment order, e.g. from
     * fp8_pack_weights applied to [M, K] codes: ceil(M / 16) * 16 * K bytes.
     * Activations that fp8_scaled_gemm quantizes itself go to its workspace
     * in this order when M <= 32, when the activation scale is per-tensor, and
     * for per-token scales when K <= 8192 (bf16) or K <= 4096 (fp32). */
    FP8SG_A_PACKED = 2,
    /* fp8_quant_mx only: the E8M0 scales in the packed layout that
     * fp8_scaled_gemm_mx reads (see fp8_pack_mx_scales). */
    FP8SG_MX_SCALES_PACKED = 4,
    /* fp8_quant_per_token_group / fp8_scaled_gemm_blockwise only: the
     * activation scales k-block-major, [K / 128, M] (s[g, m] at g * M + m),
     * instead of [M, K / 128].  The large-tile block-wise GEMM then reads the
     * scales of 64 consecutive rows of one k block as one contiguous run. */
    FP8SG_SCALES_KMAJOR = 8
} fp8sg_layout;

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8sg_status_string(int status);

/* Library ABI version (incremented on any signature change). */
int fp8sg_version(void);

/*
 * Dynamic per-token activation quantization (one scale per row).
 * FP8 Inference Explained, in depth -- "Inside a quantized linear layer": a
 * small kernel finds each token's amax, divides and casts to E4M3; "Dynamic
 * scales or static scales" on the KV-cache page: each token's maximum lands on
 * 448.
 *   x       [M, K] input, x_dtype FP8SG_BF16 or FP8SG_F32
 *   q       [M, K] E4M3 codes (output)
 *   scales  [M] fp32, s_i = RN32(max_k |x_ik| / 448) or 1.0 (output)
 *   K % 16 == 0; M, K >= 0.
 */
fp8sg_status fp8_quant_per_token(const void* x, int x_dtype, int64_t M, int64_t K,
                                 uint8_t* q, float* scales, void* stream);

/*
 * Static per-tensor quantization with a given scale; values beyond max * s
 * saturate ("Dynamic scales or static scales": 180 / s = 672 clamps to 448).
 *   x      [numel] input, FP8SG_BF16 or FP8SG_F32
 *   scale  [1] fp32 (device), positive and finite
 *   fmt    FP8SG_E4M3 or FP8SG_E5M2
 *   q      [numel] codes (output)
 */
fp8sg_status fp8_quant_per_tensor_static(const void* x, int x_dtype, int64_t numel, const float* scale,
                                         int fmt, uint8_t* q, void* stream);

/*
 * Offline per-output-channel weight quantization: the dynamic row rule applied
 * to the rows of W (FP8 Inference Explained, in depth -- "Inside a quantized
 * linear layer": weights stored as E4M3 with one FP32 scale per output channel).
 *   w         [N, K] FP8SG_F32 or FP8SG_BF16
 *   wq        [N, K] E4M3 codes (output)
 *   w_scales  [N] fp32 (output)
 *   K % 16 == 0.
 */
fp8sg_status fp8_quant_weight_per_channel(const void* w, int w_dtype, int64_t N, int64_t K,
                                          uint8_t* wq, float* w_scales, void* stream);

/*
 * Bytes of a packed weight buffer for [N, K] codes: ceil(N / 16) * 16 * K.
 * Host-only; no HIP call.
 */
size_t fp8_packed_weight_bytes(int64_t N, int64_t K);

/*
 * Reorder row-major E4M3 codes [N, K] into the fragment order of
 * FP8SG_W_PACKED (for weights: once, offline, like the quantization itself).
 * Both GEMM operands share this order, so the same call packs activation
 * codes [M, K] for FP8SG_A_PACKED.  wq and wp are device pointers; wp holds
 * fp8_packed_weight_bytes(N, K) bytes; K % 128 == 0.
 */
fp8sg_status fp8_pack_weights(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wp, void* stream);

/*
 * Bytes of device workspace fp8_scaled_gemm needs for these arguments: the
 * codes it quantizes, in the fragment order with rows padded to a multiple of
 * 16 when M <= 32, when the scale is per-tensor, or when K <= 8192 (bf16) /
 * K <= 4096 (fp32), row-major otherwise, then (per-token mode without a
 * caller buffer) the scales.  0 when the activation arrives already quantized, and
 * for bf16 per-token activations with M <= 4 and K <= 4096, which the decode
 * kernel quantizes itself (in LDS, while its weight loads are in flight).
 * Host-only; no HIP call.
 */
size_t fp8_scaled_gemm_workspace_size(int a_dtype, int a_scale_mode, int64_t M, int64_t N, int64_t K);

/*
 * Scaled GEMM  Y = diag(s_a) (A_q W_q^T) diag(s_w), written as bf16 (or fp32).
 * Both scales are constant along k and leave the sum (FP8 Inference Explained,
 * in depth -- "Inside a quantized linear layer"); FP8 x FP8 products accumulate
 * in fp32 (FP8 Quantization notebook -- "How FP8 Matmul Works at the Hardware
 * Level").
 *   a             [M, K]: a_dtype FP8SG_E4M3 = codes already quantized;
 *                 FP8SG_BF16 / FP8SG_F32 = high-precision activations that this
 *                 call quantizes first (per token, or per tensor with the given
 *                 scale), writing the codes into the workspace.
 *   a_scales      per-token: [M] fp32; an input when a is E4M3, an output (the
 *                 computed dynamic scales) when a is BF16/F32 (may then be NULL).
 *                 per-tensor: [1] fp32 input in every case.
 *   a_scale_mode  FP8SG_SCALE_PER_TOKEN or FP8SG_SCALE_PER_TENSOR
 *   wq            [N, K] E4M3 weight codes, K contiguous (W_q is "B" column-major)
 *   w_scales      [N] fp32 per-output-channel scales
 *   y             [M, N] output, y_dtype FP8SG_BF16 (round to nearest even) or
 *                 FP8SG_F32 (the same epilogue without the bf16 rounding; with
 *                 unit scales this is the raw accumulator)
 *   layout        FP8SG_W_ROW_MAJOR (0), or an OR of FP8SG_W_PACKED and
 *                 FP8SG_A_PACKED (the latter only with a_dtype FP8SG_E4M3);
 *                 other bits: FP8SG_E_DTYPE
 *   accum         FP8SG_ACCUM_EXACT or FP8SG_ACCUM_MFMA_FP8
 *   workspace     device buffer of at least fp8_scaled_gemm_workspace_size(...)
 *                 bytes, 256-byte aligned (may be NULL when that size is 0)
 *   K % 128 == 0 and K < 2^24 (else FP8SG_E_SHAPE); M, N >= 0 arbitrary.
 */
fp8sg_status fp8_scaled_gemm(const void* a, int a_dtype, float* a_scales, int a_scale_mode,
                             const uint8_t* wq, int layout, const float* w_scales, void* y, int y_dtype,
                             int64_t M, int64_t N, int64_t K, int accum,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8_scaled_gemm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels and results as fp8_scaled_gemm with the same arguments, but
 * the workspace (the activation codes and per-token scales this call computes)
 * is a static device array of FP8SG_SCRATCH_BYTES inside the library, one
 * copy per device, held until the process ends.  The call allocates nothing;
 * the caller still provides a, a_scales, wq, w_scales and y as for
 * fp8_scaled_gemm.
 *   Arguments as for fp8_scaled_gemm, without workspace / workspace_bytes.
 *   A call whose fp8_scaled_gemm_workspace_size(...) exceeds
 *   FP8SG_SCRATCH_BYTES returns FP8SG_E_SCRATCH, with nothing enqueued (e.g.
 *   bf16 per-token activations of more than about 16.7 M elements).
 * Every call on a device shares that device's scratch, and nothing in it has
 * to start cleared (each call writes what it reads).  Calls that overlap on
 * one device -- on different streams, or from different threads -- race on
 * it: serialise them.  The first call on a device looks up the scratch's
 * device address; make it before capturing a graph.
 */
fp8sg_status fp8_scaled_gemm_noalloc(const void* a, int a_dtype, float* a_scales, int a_scale_mode,
                                     const uint8_t* wq, int layout, const float* w_scales, void* y, int y_dtype,
                                     int64_t M, int64_t N, int64_t K, int accum, void* stream);

/*
 * Scaled GEMM with an FP8 output epilogue: the result is written as the E4M3
 * input of a next layer that takes a static per-tensor activation scale, so no
 * separate quantization pass reads Y again (FP8 Inference Explained, in depth
 * -- "Scales and their granularity": engines fuse the activation quantization
 * work into the preceding kernel, and static activation scales cost nothing at
 * run time; Quantization: FP8 inference and KV-cache quantization -- "Dynamic
 * scales or static scales": values beyond a static scale saturate).
 *   All arguments as for fp8_scaled_gemm, except:
 *   out_scale  [1] fp32 (device), the per-tensor scale of the output codes,
 *              positive and finite
 *   y          [M, N] E4M3 codes (output): y_code = E4M3(RN32(y32 / out_scale)),
 *              saturating, where y32 is exactly the fp32 value fp8_scaled_gemm
 *              writes with y_dtype FP8SG_F32 for the same arguments.
 */
fp8sg_status fp8_scaled_gemm_fp8out(const void* a, int a_dtype, float* a_scales, int a_scale_mode,
                                    const uint8_t* wq, int layout, const float* w_scales,
                                    const float* out_scale, uint8_t* y, int64_t M, int64_t N, int64_t K,
                                    int accum, void* workspace, size_t workspace_bytes, void* stream);

/*
 * RMSNorm with the per-token activation quantization fused into it (FP8
 * Inference Explained, in depth -- "Scales and their granularity": engines
 * fuse the per-token amax reduction into the kernel that produces the
 * activations; here that producer is the RMS normalisation in front of a
 * transformer's linear layers).  For each row, in fp32:
 *   ss = sum_k x_k^2, r = 1 / sqrt(ss / K + eps), y_k = (x_k * r) * gamma_k,
 * then the dynamic per-token rule on y: s = RN32(max_k |y_k| / 448) (1.0 when
 * 0), q_k = E4M3(RN32(y_k / s)).  The codes and the scale are exactly those
 * rules applied to the fp32 y the call writes to y_out.
 *   x       [M, K] FP8SG_BF16 or FP8SG_F32;  gamma [K], the same dtype
 *   eps     finite, >= 0
 *   q       [M, K] E4M3 codes, or with layout FP8SG_A_PACKED the fragment
 *           order of fp8_pack_weights (padding rows unwritten)
 *   scales  [M] fp32 (output)
 *   y_out   [M, K] fp32 normalised rows (output), or NULL
 *   0 < K <= 16384, K % 16 == 0 (K % 128 == 0 when packed).
 */
fp8sg_status fp8_rmsnorm_quant_per_token(const void* x, int x_dtype, const void* gamma, float eps, int64_t M,
                                         int64_t K, uint8_t* q, float* scales, float* y_out, int layout,
                                         void* stream);

/*
 * Block-wise dynamic activation quantization: one scale per token and group of
 * 128 consecutive k, so an outlier widens the step of its own group only (FP8
 * Quantization notebook -- "Granularity"; FP8 Inference Explained, in depth --
 * "Scales and their granularity").  Each group's maximum lands on 448.
 *   x       [M, K] input, x_dtype FP8SG_BF16 or FP8SG_F32
 *   q       E4M3 codes (output): [M, K] row-major when layout is 0; with
 *           FP8SG_A_PACKED the fragment order of fp8_pack_weights
 *           (fp8_packed_weight_bytes(M, K) bytes; the padding rows of the last
 *           16-row tile are left unwritten)
 *   scales  [M, K / 128] fp32 (output), row-major:
 *           s[m, g] = RN32(max_{k in group g} |x[m, k]| / 448), or 1.0 when 0;
 *           with FP8SG_SCALES_KMAJOR the same values as [K / 128, M]
 *   layout  0 or an OR of FP8SG_A_PACKED and FP8SG_SCALES_KMAJOR; other bits:
 *           FP8SG_E_DTYPE
 *   K % 128 == 0.
 */
fp8sg_status fp8_quant_per_token_group(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* q,
                                       float* scales, int layout, void* stream);

/*
 * Offline block-wise weight quantization: one scale per 128 x 128 block of W
 * (FP8 Quantization notebook -- "Granularity": per-block scaling of weights).
 *   w         [N, K] FP8SG_F32 or FP8SG_BF16
 *   wq        [N, K] E4M3 codes (output)
 *   w_scales  [ceil(N / 128), K / 128] fp32 (output), row-major:
 *             s[b, g] = RN32(max |W[128 b .. 128 b + 127, 128 g .. 128 g + 127]| / 448),
 *             or 1.0 when 0; the last row block is short when N % 128 != 0
 *   K % 128 == 0.
 */
fp8sg_status fp8_quant_weight_blockwise(const void* w, int w_dtype, int64_t N, int64_t K, uint8_t* wq,
                                        float* w_scales, void* stream);

/*
 * Block-wise scaled GEMM.  The scales vary along k, so each 128-deep partial
 * product P_g is scaled on its own before the partials are summed in fp32
 * (FP8 Inference Explained, in depth -- "Inside a quantized linear layer", on
 * why finer-than-channel scales need a purpose-built GEMM; Quantization: FP8
 * inference and KV-cache quantization -- "Training in FP8 or lower", on
 * moving each 128-element partial sum to FP32):
 *   y[m, n] = sum_g s_a[m, g] * s_w[n / 128, g] * P_g[m, n],
 *   P_g[m, n] = sum_{k = 128 g}^{128 g + 127} a_q[m, k] * w_q[n, k].
 *   a_q       [M, K] E4M3 codes (row-major, or FP8SG_A_PACKED fragment order)
 *   a_scales  [M, K / 128] fp32, as written by fp8_quant_per_token_group
 *             ([K / 128, M] with FP8SG_SCALES_KMAJOR in layout)
 *   wq        [N, K] E4M3 codes (row-major, or FP8SG_W_PACKED fragment order)
 *   w_scales  [ceil(N / 128), K / 128] fp32, as written by fp8_quant_weight_blockwise
 *   y         [M, N] FP8SG_BF16 (y rounded to nearest even) or FP8SG_F32 (y)
 *   layout    0 or an OR of FP8SG_W_PACKED, FP8SG_A_PACKED and FP8SG_SCALES_KMAJOR
 *   accum     FP8SG_ACCUM_MFMA_FP8: each P_g is one FP8 matrix-core product
 *             (with that hardware's in-instruction alignment, see fp8sg_accum);
 *             FP8SG_ACCUM_EXACT: P_g formed exactly on the bf16 matrix cores
 *             (every M).
 *   K % 128 == 0 and K < 2^24; M, N >= 0 arbitrary.
 */
fp8sg_status fp8_scaled_gemm_blockwise(const uint8_t* a_q, const float* a_scales, const uint8_t* wq, int layout,
                                       const float* w_scales, void* y, int y_dtype, int64_t M, int64_t N,
                                       int64_t K, int accum, void* stream);

/*
 * MXFP8 (microscaling): every 32 consecutive k of a row share one power-of-two
 * scale, stored as an E8M0 byte e with the value 2^(e - 127) (e = 255, NaN, is
 * never written).  Small blocks with an 8-bit scale each ("Quantization for LLM
 * inference: FP8, INT4 (GPTQ, AWQ) and GGUF", blog.lo0.es -- "Microscaling:
 * NVFP4 and MXFP4"), contiguous along the reduction dimension ("Quantization:
 * FP8 inference and KV-cache quantization" -- "Training in FP8 or lower").
 * The scale of a block is the smallest 2^k with amax <= FMAX * 2^k (the
 * dynamic rule s = amax / FMAX rounded up to a power of two, so no element
 * saturates), k clamped to [-127, 127], and 2^0 for a block of zeros; a value
 * is encoded as FMT(RN32(x / 2^k)) with the library's rounding rule.
 *
 * MX fragment order of packed codes: the 2048-byte block of (16-row tile t,
 * 128-k block kb) sits at (t * K/128 + kb) * 2048, as for FP8SG_W_PACKED, but
 * lane l's first 16 bytes (at 16 l) are k 128 kb + 16 (l / 16) + [0, 16) of
 * row 16 t + l % 16 and its second 16 bytes (at 1024 + 16 l) are
 * k 128 kb + 64 + 16 (l / 16) + [0, 16): the k order of gfx950's scaled matrix
 * cores, which apply scale l / 16 of the block to k [32 (l / 16), +32).  Codes
 * packed by fp8_pack_weights are NOT in this order.
 *
 * Packed scale layout (what fp8_scaled_gemm_mx reads): for 128-deep k block
 * kb and group g of four 16-row tiles, 256 bytes at (kb * T4 + g) * 256 with
 * T4 = ceil(rows / 64); inside, byte 4 l + j is the scale of row
 * 16 (4 g + j) + l % 16 for the 32-k group l / 16 of block kb (l = 0..63,
 * j = 0..3).  Rows past `rows` hold 127 when written by fp8_pack_mx_scales and
 * are left unwritten by fp8_quant_mx.
 */

/* Bytes of a packed MX scale buffer for [rows, K] codes: ceil(rows / 64) * 256
 * * (K / 128).  Host-only; no HIP call. */
size_t fp8_mx_packed_scale_bytes(int64_t rows, int64_t K);

/*
 * MXFP8 quantization of the rows of x (activations or, offline, weights).
 *   x       [rows, K] FP8SG_BF16 or FP8SG_F32
 *   fmt     element format: FP8SG_E4M3 (FMAX 448) or FP8SG_E5M2 (FMAX 57344)
 *   q       codes (output): [rows, K] row-major, or with FP8SG_A_PACKED in
 *           layout the MX fragment order above (fp8_packed_weight_bytes(rows, K)
 *           bytes; padding rows unwritten) -- for weights, quantize straight
 *           into this order offline
 *   scales  E8M0 bytes (output): [rows, K / 32] row-major, or with
 *           FP8SG_MX_SCALES_PACKED the packed layout above
 *           (fp8_mx_packed_scale_bytes(rows, K) bytes)
 *   layout  0 or an OR of FP8SG_A_PACKED and FP8SG_MX_SCALES_PACKED
 *   K % 32 == 0 (K % 128 == 0 with either packed flag).
 */
fp8sg_status fp8_quant_mx(const void* x, int x_dtype, int64_t rows, int64_t K, int fmt, uint8_t* q,
                          uint8_t* scales, int layout, void* stream);

/*
 * Row-major E8M0 scales [rows, K / 32] -> the packed layout above (for
 * weights: once, offline).  packed holds fp8_mx_packed_scale_bytes(rows, K)
 * bytes; K % 128 == 0.
 */
fp8sg_status fp8_pack_mx_scales(const uint8_t* scales, int64_t rows, int64_t K, uint8_t* packed, void* stream);

/*
 * MXFP8 GEMM on the gfx950 scaled matrix cores: each 32-deep partial product
 * is scaled by its two block scales and the results accumulate in fp32:
 *   y[m, n] = sum_b 2^(ka[m, b] + kw[n, b]) sum_{k = 32 b}^{32 b + 31} a[m, k] w[n, k].
 * The matrix cores sum each group of 8 consecutive products with the in-
 * instruction alignment described at fp8sg_accum (FP8SG_ACCUM_MFMA_FP8).
 *   a_q       [M, K] codes of format a_fmt (FP8SG_E4M3 or FP8SG_E5M2),
 *             row-major, or with FP8SG_A_PACKED the MX fragment order
 *   a_scales  packed E8M0 scales of a (fp8_mx_packed_scale_bytes(M, K) bytes)
 *   wq        [N, K] E4M3 codes, row-major, or with FP8SG_W_PACKED the MX fragment order
 *   w_scales  packed E8M0 scales of W (fp8_mx_packed_scale_bytes(N, K) bytes)
 *   y         [M, N] FP8SG_BF16 (round to nearest even) or FP8SG_F32
 *   layout    0 or an OR of FP8SG_W_PACKED and FP8SG_A_PACKED
 *   K % 128 == 0 and K < 2^24; M, N >= 0 arbitrary.
 */
fp8sg_status fp8_scaled_gemm_mx(const uint8_t* a_q, const uint8_t* a_scales, int a_fmt, const uint8_t* wq,
                                const uint8_t* w_scales, int layout, void* y, int y_dtype, int64_t M, int64_t N,
                                int64_t K, void* stream);

/*
 * The MXFP8 decode GEMM on bf16 activations: every 32-element block of each
 * row of x is quantized inside the GEMM kernel by the rule above (the codes and
 * scales fp8_quant_mx writes for the same x), in registers, and multiplied as
 * in fp8_scaled_gemm_mx -- the same products in the same order, so the result
 * equals fp8_quant_mx followed by fp8_scaled_gemm_mx bit for bit.  One launch,
 * no quantized copy of x (the pages' point that engines fuse the activation
 * quantization into the kernels around it: FP8 Inference Explained, in depth --
 * "Inside a quantized linear layer").
 *   x         [M, K] bf16 (uint16 bit patterns), row-major
 *   a_fmt     format of the activation codes: FP8SG_E4M3 or FP8SG_E5M2
 *   wq, w_scales, y, y_dtype: as for fp8_scaled_gemm_mx
 *   layout    0 or FP8SG_W_PACKED (the weights' layout)
 *   K % 128 == 0, K < 2^24; 0 <= M <= 16 (decode shapes).  A larger M returns
 *   FP8SG_E_SHAPE: every workgroup reads all of x, twice the bytes of its
 *   codes, so there fp8_quant_mx followed by fp8_scaled_gemm_mx is faster.
 */
fp8sg_status fp8_scaled_gemm_mx_bf16(const uint16_t* x, int a_fmt, const uint8_t* wq, const uint8_t* w_scales,
                                     int layout, void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                     void* stream);

/*
 * KV-cache calibration: one scale per kv head, s_h = RN32(amax_h / max) over
 * all (b, s, d) of head h, or 1.0 when that is 0 (per-head KV scales require
 * calibration -- Quantization: FP8 inference and KV-cache quantization,
 * "Turning it on in an engine").
 *   kv           [B, S, H, D] bf16 (uint16 bit patterns)
 *   fmt          FP8SG_E4M3 (max 448) or FP8SG_E5M2 (max 57344)
 *   head_scales  [H] fp32 (output; also used as scratch during the call)
 *   D % 16 == 0.
 */
fp8sg_status fp8_kv_calibrate(const uint16_t* kv, int64_t B, int64_t S, int64_t H, int64_t D, int fmt,
                              float* head_scales, void* stream);

/*
 * KV-cache quantization with per-head scales (FP8 Inference Explained, in
 * depth -- "FP8 KV cache": stored FP8 halves the cache).
 *   kv [B, S, H, D] bf16 -> out [B, S, H, D] codes; code = FMT(RN32(x / s_h)).
 *   D % 16 == 0.
 */
fp8sg_status fp8_kv_quant(const uint16_t* kv, int64_t B, int64_t S, int64_t H, int64_t D,
                          const float* head_scales, int fmt, uint8_t* out, void* stream);

/*
 * KV-cache dequantization: a stored code reads back as the head's scale times
 * the code's value (FP8 Inference Explained, in depth -- "Scales and their
 * granularity": x is approximately s times x_fp8; "FP8 KV cache": backends
 * that do not compute in FP8 read the cache back and compute in higher
 * precision; Quantization: FP8 inference and KV-cache quantization -- "Turning
 * it on in an engine": one scale per attention head).
 *   kvq          [B, S, H, D] codes of format fmt (FP8SG_E4M3 or FP8SG_E5M2)
 *   head_scales  [H] fp32, the scales the codes were quantized with
 *   out          [B, S, H, D] bf16 (output): bf16(RN32(dec(code) * s_h)),
 *                round to nearest even; a NaN code gives a bf16 NaN
 *   D % 16 == 0.  The caller owns every buffer; nothing else is written.
 */
fp8sg_status fp8_kv_dequant(const uint8_t* kvq, int64_t B, int64_t S, int64_t H, int64_t D,
                            const float* head_scales, int fmt, uint16_t* out, void* stream);

/*
 * Append one token per sequence to an FP8 KV cache.  The new keys or values
 * are quantized with the head scales the cache already holds: the static
 * scales of a calibrated cache (Quantization: FP8 inference and KV-cache
 * quantization -- "Turning it on in an engine": per-head scales come from
 * calibration), so a new value beyond max * s_h saturates to the format's
 * maximum ("Dynamic scales or static scales": static scales clip inputs more
 * extreme than the calibration set; FP8 Inference Explained, in depth -- "FP8
 * KV cache").
 *   kv_new       [B, H, D] bf16 (uint16 bit patterns)
 *   pos          [B] int32 (device): the position each sequence writes; a
 *                sequence whose pos[b] lies outside [0, S_cap) is skipped
 *   head_scales  [H] fp32 per-head scales of the cache
 *   fmt          FP8SG_E4M3 or FP8SG_E5M2
 *   cache        [B, S_cap, H, D] codes: cache[b, pos[b], h, :] =
 *                FMT(RN32(kv_new[b, h, :] / s_h)); nothing else is written
 *   D % 16 == 0.
 */
fp8sg_status fp8_kv_append(const uint16_t* kv_new, const int32_t* pos, int64_t B, int64_t S_cap,
                           int64_t H, int64_t D, const float* head_scales, int fmt,
                           uint8_t* cache, void* stream);

/*
 * Bytes of device workspace fp8_kv_decode_attention needs (the per-chunk
 * partial results).  Host-only; no HIP call.
 */
size_t fp8_kv_decode_attention_workspace_size(int64_t B, int64_t S_cap, int64_t Hq, int64_t Hkv, int64_t D);

/*
 * One decode step of attention over an FP8 KV cache: query q[b, h, :] attends
 * over positions 0 .. lengths[b] - 1 of kv head g = h / (Hq / Hkv) (grouped
 * query heads).  The cache is read back as code value times the head's scale
 * and the attention is computed in fp32 (FP8 Inference Explained, in depth --
 * "FP8 KV cache": per-attention-head scales; backends that do not compute in
 * FP8 read the cache back and compute in higher precision), with the softmax
 * taken block by block by the online recurrence ("FlashAttention v1/v2/v3/v4"
 * post -- "The trick that made it all possible: online softmax"):
 *     s_t = scale * q . (dec(K_t) s_K[g]),  p = softmax(s),  o = sum_t p_t dec(V_t) s_V[g].
 *   q           [B, Hq, D] bf16
 *   k_cache,
 *   v_cache     [B, S_cap, Hkv, D] codes of format fmt (FP8SG_E4M3 or FP8SG_E5M2),
 *               as written by fp8_kv_quant / fp8_kv_append
 *   k_scales,
 *   v_scales    [Hkv] fp32 per-head scales
 *   lengths     [B] int32 (device): positions attended per sequence; values are
 *               clamped to [0, S_cap]; a sequence of length 0 gets output 0
 *   scale       softmax scale; 0 or negative means 1 / sqrt(D)
 *   out         [B, Hq, D], out_dtype FP8SG_BF16 (round to nearest even) or FP8SG_F32
 *   workspace   at least fp8_kv_decode_attention_workspace_size(...) bytes, 16-byte aligned
 *   D == 128; Hq % Hkv == 0 with Hq / Hkv in {1, 2, 4, 8}; S_cap <= 2^20.
 * The result does not depend on timing: chunk partials are combined in a fixed order.
 */
fp8sg_status fp8_kv_decode_attention(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                     const float* k_scales, const float* v_scales, int fmt,
                                     const int32_t* lengths, int64_t B, int64_t S_cap, int64_t Hq,
                                     int64_t Hkv, int64_t D, float scale, void* out, int out_dtype,
                                     void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8SG_H */
