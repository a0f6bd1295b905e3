/*
 * CPU oracle for blockwise 4-bit weight quantization and the dequantize-and-
 * multiply products that consume it.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain definition that the
 * HIP library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the library never does.  It shares
 * no code, header or table with the HIP sources.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (contraction off: every float operation below is one IEEE binary32 operation
 * with round-to-nearest-even, in exactly the order written).
 *
 * Sources (the pages this follows):
 *  [P2] gsantana.dev, "Quantizing LLMs Without Guesswork: What 4 Bits Really
 *       Cost": section "Scale and zero point" (symmetric and asymmetric
 *       formulas), "Granularity: who shares a scale" (groups are runs of
 *       consecutive weights inside a row), "Quantize, then dequantize" (the
 *       NumPy fake-quant: half-to-even rounding, zero scale replaced by 1, the
 *       relative-error metric), "Number formats" (FP8 E4M3: max 448, no inf).
 *  [P3] gowda.ai, "LLM fast inference" (Tahoma): "The naive symmetric
 *       baseline", "Achievement 1: asymmetric W4 that uses the code space"
 *       (codes 0..15, integer zero point, 16-bit scale and zero per group of
 *       128 along K), "MSE clipping: do not let one outlier price the whole
 *       block" (11 contracted ranges from the observed midpoint, strict
 *       improvement over the plain quantizer, clipped values count in the
 *       error), "Achievement 2: 8-bit activations without a calibration set"
 *       (per-row FP8 E4M3 scale from the row maximum over 448, 1e-8 floor).
 *  [P5] nebelwolfi.xyz, "The outlier problem that reshaped how we quantize
 *       LLMs": "The Basic Arithmetic and Why It Breaks", "Block Quantization".
 *
 * Readings where the pages are silent or their formulas were lost (each also
 * listed in the design notes):
 *  - rounding is half-to-even everywhere (P2's code uses NumPy round);
 *  - symmetric INT4: scale = f*amax/7 as on P2/P5, codes clamped to the full
 *    signed range -8..7 (at f = 1 no value reaches -8, as P3 notes);
 *  - asymmetric: P2's formulas with 2^bits - 1 levels; the zero point is an
 *    integer and is NOT clamped to the code range;
 *  - the scale is rounded to fp16 first and the zero point, codes and error
 *    are computed with that rounded scale (the stored triple reproduces the
 *    error the search measured);
 *  - clip candidate f: asym range [mid - f*h, mid + f*h] about the observed
 *    midpoint (f = 1 uses [min, max] directly); sym range [-f*amax, f*amax];
 *  - block error: a fixed pairwise halving sum of squared errors (the mean
 *    differs only by the constant 1/G, so the argmin is the same);
 *  - activation codes: e4m3(fl32(x / s_m)), round to nearest even, saturating.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define W4O_SYM 0
#define W4O_ASYM 1
#define W4O_MAX_FRACS 64
#define W4O_MAX_GROUP (1 << 26)

/* ------------------------------------------------------------------ formats */

/* binary32 -> binary16, round to nearest even, from the IEEE 754 definition:
 * the value is rounded to the multiple of the binary16 quantum at its binade
 * (2^-24 below the smallest normal 2^-14, else 2^(e-10)), and the rounded value
 * is then encoded.  Overflow rounds to infinity (65520 and up). */
uint16_t w4o_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int ex;
    (void)frexp(a, &ex);              /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;                   /* a in [2^e, 2^(e+1)) */
    if (e < -14) {                    /* subnormal binade: quantum 2^-24 */
        double r = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)r);       /* r == 1024 encodes 2^-14 */
    }
    double r = nearbyint(ldexp(a, 10 - e));          /* in [1024, 2048] */
    uint32_t enc = ((uint32_t)(e + 15) << 10) + (uint32_t)r - 1024u;
    if (enc >= 0x7C00u) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | enc);
}

float w4o_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

float w4o_bf16_to_f32(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* OCP FP8 E4M3 ("fn": no infinities, one NaN pattern per sign).  Exponent bias
 * 7, 3 mantissa bits; normal values (8 + m) * 2^(e - 10) for e = 1..15, except
 * e = 15, m = 7 which is NaN; subnormals m * 2^-9.  Largest finite 448. */
float w4o_e4m3_to_f32(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xF;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return (float)(sign ? -v : v);
}

/* binary32 -> E4M3, round to nearest even, saturating to +-448. */
uint8_t w4o_f32_to_e4m3(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint8_t sign = (uint8_t)((bits >> 24) & 0x80u);
    if (isnan(f)) return (uint8_t)(sign | 0x7Fu);
    double a = fabs((double)f);
    if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);   /* e = 15, m = 6 */
    if (a == 0.0) return sign;
    int ex;
    (void)frexp(a, &ex);
    int e = ex - 1;
    if (e < -6) {                                    /* subnormal: quantum 2^-9 */
        double r = nearbyint(ldexp(a, 9));           /* 0..8; 8 encodes 2^-6 */
        return (uint8_t)(sign | (uint8_t)r);
    }
    double r = nearbyint(ldexp(a, 3 - e));           /* in [8, 16] */
    uint32_t enc = ((uint32_t)(e + 7) << 3) + (uint32_t)r - 8u;
    return (uint8_t)(sign | enc);                    /* a < 448 keeps enc <= 0x7E */
}

/* --------------------------------------------------------------- quantizer */

static float round_half_even(float x) { return nearbyintf(x); }

/* The integer grid of a mode: codes lie in [qlo, qhi]. */
static void code_range(int bits, int mode, int64_t *qlo, int64_t *qhi)
{
    if (mode == W4O_ASYM) { *qlo = 0; *qhi = ((int64_t)1 << bits) - 1; }
    else { *qlo = -((int64_t)1 << (bits - 1)); *qhi = ((int64_t)1 << (bits - 1)) - 1; }
}

/* One candidate range for one group: the fp16 scale (as bits and as the float
 * used afterwards), the integer zero point, the codes and the squared-error
 * sum.  Returns the SSE.  `a` is scratch of length `pow2`. */
static float eval_candidate(const float *w, int64_t G, int64_t pow2, int bits, int mode,
                            float f, float wmin, float wmax, float amax,
                            int64_t *q, uint16_t *s_bits, float *s_out, int64_t *z_out,
                            float *a)
{
    int64_t qlo, qhi;
    code_range(bits, mode, &qlo, &qhi);
    float s32;
    if (mode == W4O_ASYM) {
        float lo, hi;
        if (f == 1.0f) {
            lo = wmin;                       /* plain min/max quantizer */
            hi = wmax;
        } else {
            float mid = (wmax + wmin) * 0.5f;  /* observed midpoint */
            float h = (wmax - wmin) * 0.5f;    /* half range */
            float fh = f * h;
            lo = mid - fh;
            hi = mid + fh;
        }
        s32 = (hi - lo) / (float)(qhi - qlo);        /* (max - min) / (2^bits - 1) */
        uint16_t sb = w4o_f32_to_f16(s32);
        float s = w4o_f16_to_f32(sb);
        if (s == 0.0f) { s = 1.0f; sb = w4o_f32_to_f16(1.0f); }
        float zf = round_half_even(-lo / s);         /* zero = round(-min / scale) */
        int64_t z = (int64_t)zf;
        for (int64_t j = 0; j < G; ++j) {
            int64_t t = (int64_t)round_half_even(w[j] / s);
            int64_t c = t + z;
            if (c < qlo) c = qlo;
            if (c > qhi) c = qhi;
            q[j] = c;
        }
        *s_bits = sb; *s_out = s; *z_out = z;
    } else {
        float r = f * amax;
        s32 = r / (float)qhi;                        /* amax / qmax, qmax = 2^(bits-1) - 1 */
        uint16_t sb = w4o_f32_to_f16(s32);
        float s = w4o_f16_to_f32(sb);
        if (s == 0.0f) { s = 1.0f; sb = w4o_f32_to_f16(1.0f); }
        for (int64_t j = 0; j < G; ++j) {
            int64_t c = (int64_t)round_half_even(w[j] / s);
            if (c < qlo) c = qlo;
            if (c > qhi) c = qhi;
            q[j] = c;
        }
        *s_bits = sb; *s_out = s; *z_out = 0;
    }
    /* reconstruction error, clipped values included, summed by halving */
    float s = *s_out;
    int64_t z = *z_out;
    for (int64_t j = 0; j < G; ++j) {
        float xr = (float)(q[j] - z) * s;            /* x' = (q - zero) * scale */
        float e = w[j] - xr;
        a[j] = e * e;
    }
    for (int64_t j = G; j < pow2; ++j) a[j] = 0.0f;
    for (int64_t len = pow2 / 2; len >= 1; len /= 2)
        for (int64_t j = 0; j < len; ++j) a[j] = a[j] + a[j + len];
    return a[0];
}

/*
 * Quantize W[N, K] (fp32, row-major, row = output channel) in groups of G
 * consecutive weights along K.
 *   bits  : 4 (the library's format) or 8 (worked examples only)
 *   mode  : 0 symmetric, 1 asymmetric
 *   fracs : n_fracs clip fractions, fracs[0] == 1, descending (n_fracs == 1:
 *           no search, the plain quantizer)
 * Outputs (all [N, K/G] unless noted; NULL skips):
 *   q       [N, K] int16 codes (sym: signed, asym: 0..2^bits-1)
 *   scale   fp16 bits;  zero  fp16 bits of the integer zero point (asym only)
 *   clip    index of the winning fraction
 *   sse     [N, K/G, n_fracs] squared-error sum of every candidate
 * Returns 0, or a negative number for bad arguments.
 */
int w4o_quantize(const float *W, int64_t N, int64_t K, int64_t G, int bits, int mode,
                 const float *fracs, int n_fracs, int16_t *q, uint16_t *scale,
                 uint16_t *zero, uint8_t *clip, float *sse)
{
    if (!W || N < 0 || K <= 0 || G <= 0 || K % G != 0 || G > W4O_MAX_GROUP) return -1;
    if (bits != 4 && bits != 8) return -2;
    if (mode != W4O_SYM && mode != W4O_ASYM) return -3;
    if (!fracs || n_fracs < 1 || n_fracs > W4O_MAX_FRACS || fracs[0] != 1.0f) return -4;
    int64_t pow2 = 1;
    while (pow2 < G) pow2 *= 2;
    int64_t ng = K / G;
    int bad = 0;
#pragma omp parallel
    {
        int64_t *qc = (int64_t *)malloc(sizeof(int64_t) * (size_t)G);
        int64_t *qb = (int64_t *)malloc(sizeof(int64_t) * (size_t)G);
        float *a = (float *)malloc(sizeof(float) * (size_t)pow2);
        if (!qc || !qb || !a) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                for (int64_t g = 0; g < ng; ++g) {
                    const float *w = W + n * K + g * G;
                    float wmin = w[0], wmax = w[0], amax = fabsf(w[0]);
                    for (int64_t j = 1; j < G; ++j) {
                        if (w[j] < wmin) wmin = w[j];
                        if (w[j] > wmax) wmax = w[j];
                        if (fabsf(w[j]) > amax) amax = fabsf(w[j]);
                    }
                    int best = 0;
                    float best_sse = 0.0f, best_s = 0.0f;
                    uint16_t best_sb = 0;
                    int64_t best_z = 0;
                    for (int i = 0; i < n_fracs; ++i) {
                        uint16_t sb; float s; int64_t z;
                        float e = eval_candidate(w, G, pow2, bits, mode, fracs[i], wmin, wmax,
                                                 amax, qc, &sb, &s, &z, a);
                        if (sse) sse[(n * ng + g) * n_fracs + i] = e;
                        if (i == 0 || e < best_sse) {        /* strictly better only */
                            best = i; best_sse = e; best_sb = sb; best_s = s; best_z = z;
                            memcpy(qb, qc, sizeof(int64_t) * (size_t)G);
                        }
                    }
                    (void)best_s;
                    if (q) for (int64_t j = 0; j < G; ++j) q[n * K + g * G + j] = (int16_t)qb[j];
                    if (scale) scale[n * ng + g] = best_sb;
                    if (zero && mode == W4O_ASYM) zero[n * ng + g] = w4o_f32_to_f16((float)best_z);
                    if (clip) clip[n * ng + g] = (uint8_t)best;
                }
            }
        }
        free(qc); free(qb); free(a);
    }
    return bad ? -5 : 0;
}

/* Canonical packing of 4-bit codes: byte [n, k/2] holds code k (even) in its
 * low nibble and code k+1 in its high nibble; symmetric codes are stored as
 * two's-complement nibbles, asymmetric codes as unsigned 0..15. */
int w4o_pack(const int16_t *q, int64_t N, int64_t K, uint8_t *packed)
{
    if (K % 2) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < K / 2; ++b) {
            uint8_t lo = (uint8_t)(q[n * K + 2 * b] & 0xF);
            uint8_t hi = (uint8_t)(q[n * K + 2 * b + 1] & 0xF);
            packed[n * (K / 2) + b] = (uint8_t)(lo | (hi << 4));
        }
    return 0;
}

/* Code of weight (n, k) read back from the canonical packing. */
static int64_t unpack_code(const uint8_t *packed, int64_t K, int64_t n, int64_t k, int mode)
{
    uint8_t byte = packed[n * (K / 2) + k / 2];
    int v = (k & 1) ? (byte >> 4) : (byte & 0xF);
    if (mode == W4O_SYM && v >= 8) v -= 16;
    return v;
}

/* Dequantized weight W'[n, k] = (q - zero) * scale, exact in float64. */
static double dequant_one(const uint8_t *packed, const uint16_t *scale, const uint16_t *zero,
                          int64_t K, int64_t G, int mode, int64_t n, int64_t k)
{
    int64_t ng = K / G;
    double s = (double)w4o_f16_to_f32(scale[n * ng + k / G]);
    double z = (mode == W4O_ASYM) ? (double)w4o_f16_to_f32(zero[n * ng + k / G]) : 0.0;
    return ((double)unpack_code(packed, K, n, k, mode) - z) * s;
}

int w4o_dequant(const uint8_t *packed, const uint16_t *scale, const uint16_t *zero, int64_t N,
                int64_t K, int64_t G, int mode, double *Wd)
{
    if (K % G || K % 2) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) Wd[n * K + k] = dequant_one(packed, scale, zero, K, G, mode, n, k);
    return 0;
}

/* ------------------------------------------------------------ activations */

/* Per-row dynamic FP8: amax over the row, s_m = max(amax / 448, 1e-8),
 * xq = e4m3(fl32(x / s_m)).  X is bf16 bits [M, K]. */
int w4o_row_quant_e4m3(const uint16_t *X, int64_t M, int64_t K, uint8_t *xq, float *s_m)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(w4o_bf16_to_f32(X[m * K + k]));
            if (v > amax) amax = v;
        }
        float s = amax / 448.0f;
        if (s < 1e-8f) s = 1e-8f;
        s_m[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float x = w4o_bf16_to_f32(X[m * K + k]);
            xq[m * K + k] = w4o_f32_to_e4m3(x / s);
        }
    }
    return 0;
}

/* --------------------------------------------------------------- products */

/*
 * Reference product in float64, Y = X . W'^T, over a chosen subset of rows of X
 * and rows of W (output columns):
 *   Y[i, j] = a_scale[rows[i]] * sum_k x[rows[i], k] * W'[cols[j], k]
 * X is float64 [M, K] (bf16 activations or decoded E4M3 codes, both exact in
 * float64); W' is rebuilt from the packed codes, fp16 scales and zeros.
 * a_scale may be NULL (taken as 1): the W4A8 product passes the row scales.
 */
int w4o_gemm_ref(const double *X, int64_t M, const uint8_t *packed, const uint16_t *scale,
                 const uint16_t *zero, int64_t N, int64_t K, int64_t G, int mode,
                 const float *a_scale, const int64_t *rows, int64_t n_rows, const int64_t *cols,
                 int64_t n_cols, double *Y)
{
    if (K % G || K % 2) return -1;
    for (int64_t i = 0; i < n_rows; ++i) if (rows[i] < 0 || rows[i] >= M) return -2;
    for (int64_t j = 0; j < n_cols; ++j) if (cols[j] < 0 || cols[j] >= N) return -3;
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
        for (int64_t j = 0; j < n_cols; ++j) {
            int64_t n = cols[j];
            for (int64_t k = 0; k < K; ++k) wcol[k] = dequant_one(packed, scale, zero, K, G, mode, n, k);
            for (int64_t i = 0; i < n_rows; ++i) {
                const double *x = X + rows[i] * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += x[k] * wcol[k];
                if (a_scale) acc *= (double)a_scale[rows[i]];
                Y[i * n_cols + j] = acc;
            }
        }
        free(wcol);
    }
    return 0;
}

int w4o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------- array forms (for tests) */

void w4o_f32_to_f16_n(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = w4o_f32_to_f16(x[i]);
}

void w4o_f16_to_f32_n(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = w4o_f16_to_f32(h[i]);
}

void w4o_f32_to_e4m3_n(const float *x, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = w4o_f32_to_e4m3(x[i]);
}

void w4o_bf16_to_f32_n(const uint16_t *b, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = w4o_bf16_to_f32(b[i]);
}
