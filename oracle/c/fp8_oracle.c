/*
 * FP8 (E4M3 "fn" and E5M2) saturating round-to-nearest-even encoder, in plain C.
 *
 * TEST INFRASTRUCTURE ONLY (CPU oracle).  It serves sweeps over every float32
 * bit pattern, which the numpy oracle is too slow for.  It follows the same
 * definition as oracle/fp8.py and is checked against it; it shares nothing with
 * the HIP library.
 *
 * Definition (FP8 Inference Explained, in depth -- "The numbers in one byte";
 * FP8 Quantization notebook -- "FP8 Representation", "E4M3 vs E5M2"):
 *   E4M3fn: bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, max 448.
 *   E5M2:   bias 15, 2 mantissa bits, infinities and NaNs at exponent 31,
 *           max 57344 (IEEE-style reading of the pages' maximum).
 *   encode(t): the finite grid value nearest to t; ties go to the even code;
 *   |t| >= max (including infinity) saturates to max; the sign is kept;
 *   NaN -> 0x7F with the input's sign bit.
 *
 * The grid is built by decoding each code from its bit fields; a value is
 * placed on the grid by binary search over the midpoints between neighbours
 * (exact in double).  Built with -O2 -ffp-contract=off, no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int ncodes;            /* finite non-negative codes 0 .. ncodes-1 */
    double grid[128];
    double mid[127];
} grid_t;

static grid_t g_e4m3, g_e5m2;
static int g_ready = 0;

static double decode_fields(int code, int ebits, int mbits, int bias) {
    int e = (code >> mbits) & ((1 << ebits) - 1);
    int m = code & ((1 << mbits) - 1);
    double frac = (double)m / (double)(1 << mbits);
    if (e == 0) return frac * ldexp(1.0, 1 - bias);
    return (1.0 + frac) * ldexp(1.0, e - bias);
}

static void build(grid_t* g, int ebits, int mbits, int bias, int max_code) {
    g->ncodes = max_code + 1;
    for (int c = 0; c <= max_code; ++c) g->grid[c] = decode_fields(c, ebits, mbits, bias);
    for (int c = 0; c < max_code; ++c) g->mid[c] = 0.5 * (g->grid[c] + g->grid[c + 1]);
}

static void ensure_ready(void) {
    if (g_ready) return;
    build(&g_e4m3, 4, 3, 7, 0x7E);   /* 0x7F is NaN in the fn variant */
    build(&g_e5m2, 5, 2, 15, 0x7B);  /* 0x7C is +Inf, 0x7D..0x7F NaN */
    g_ready = 1;
}

int fp8o_init(void) { ensure_ready(); return 0; }

static inline uint8_t encode_one(const grid_t* g, float t) {
    uint32_t bits;
    memcpy(&bits, &t, 4);
    uint8_t sign = (uint8_t)((bits >> 31) << 7);
    if (isnan(t)) return (uint8_t)(0x7F | sign);
    double a = fabs((double)t);
    int maxc = g->ncodes - 1;
    if (a >= g->grid[maxc]) return (uint8_t)(maxc | sign);
    /* first midpoint index i with mid[i] >= a */
    int lo = 0, hi = maxc; /* search in mid[0 .. maxc-1]; result in [0, maxc] */
    while (lo < hi) {
        int md = (lo + hi) >> 1;
        if (g->mid[md] >= a) hi = md; else lo = md + 1;
    }
    int code = lo;
    if (code < maxc && a == g->mid[code] && (code & 1)) code += 1;
    return (uint8_t)(code | sign);
}

/* fmt: 0 = E4M3, 1 = E5M2 */
static const grid_t* pick(int fmt) { ensure_ready(); return fmt == 1 ? &g_e5m2 : &g_e4m3; }

void fp8o_encode_f32(const float* t, int64_t n, int fmt, uint8_t* out) {
    const grid_t* g = pick(fmt);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = encode_one(g, t[i]);
}

/* Encode the float32 values whose bit patterns are start, start+1, ..., start+n-1. */
void fp8o_encode_bit_patterns(uint32_t start, int64_t n, int fmt, uint8_t* out) {
    const grid_t* g = pick(fmt);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b = start + (uint32_t)i;
        float t;
        memcpy(&t, &b, 4);
        out[i] = encode_one(g, t);
    }
}

/* code = FMT(RN32(x / s)) for float32 x and a float32 scale s (IEEE division). */
void fp8o_quant_given_scale_f32(const float* x, int64_t n, float s, int fmt, uint8_t* out) {
    const grid_t* g = pick(fmt);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        volatile float q = x[i] / s;
        out[i] = encode_one(g, q);
    }
}

/* Same with a per-element-group scale: scale index = (i / inner) % nscales. */
void fp8o_quant_grouped_scale_f32(const float* x, int64_t n, const float* s, int64_t inner, int64_t nscales,
                                  int fmt, uint8_t* out) {
    const grid_t* g = pick(fmt);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        volatile float q = x[i] / s[(i / inner) % nscales];
        out[i] = encode_one(g, q);
    }
}

/* Count threads an OpenMP region actually uses (for reporting). */
int fp8o_num_threads(void) {
    int nt = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            nt = omp_get_num_threads();
#endif
        }
    }
    return nt;
}
