/*
 * fp4_oracle.c -- plain CPU oracle for block-scaled 4-bit weights (NVFP4, MXFP4)
 * and the weight-only (W4A16) linear.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the GPU library must compute.
 * It is built and called by the tests, by the package's smoke check and by the
 * CPU-baseline leg of the benchmark.  The product path never links or calls it,
 * and it shares no code, header, table or constant with the GPU sources.
 *
 * What the pages fix and what is a stated reading:
 *  - A weight in NVFP4 / MXFP4 is a 4-bit E2M1 code plus a scale shared by its
 *    block (Scale-QLoRA page, rit.work "scale-qlora-merge-native-4bit-models",
 *    paragraph on the NVFP4 and MXFP4 formats).
 *  - The quantization is weight-only; activations stay 16-bit (Telegram post
 *    tggo.me/sberlogasci/42740, section "Metod"; QATFactory page, section on
 *    NVFP4 vs MXFP4 strategies, where W4A16 is defined).
 *  - "Max" calibration recomputes dynamic scales from the current tensors; frozen
 *    scales keep calibrated scales and recompute only the codes (Nemotron 3.5
 *    Lightning NVFP4 via QAD, section 03 "Dynamic vs Frozen").
 *  - A scale-only merge writes trained scale bytes on the format's scale grid and
 *    copies the code plane verbatim (Scale-QLoRA page, merge paragraph).
 *  - The linear multiplies in bf16-representable values with a parallel LoRA
 *    branch (Telegram post, section "Metod"; QATFactory page, section on how
 *    training repeats the engine's arithmetic).
 *  Bit layouts, block sizes, scale formulas and rounding are not on the pages;
 *  the readings used are the OCP Microscaling v1.0 definitions of E2M1 and E8M0,
 *  the OCP 8-bit float E4M3 ("FN": max 448, no infinities), 16-element NVFP4
 *  blocks with an E4M3 scale and an fp32 tensor scale amax/(6*448), 32-element
 *  MXFP4 blocks with scale 2^(floor(log2 amax) - 2), blocks laid along K, and
 *  round-to-nearest-even on the exact real quotient with saturation.
 *
 * Arithmetic: every rounding decision compares exact values.  Grid values and
 * midpoints have at most 5 significant bits, the block scale at most 28, so each
 * product compared below has at most 33 significant bits and is exact in binary64.
 * Sums (merge) are kept exact as a TwoSum pair.  Dot products are accumulated in
 * binary64 with k ascending.
 *
 * Layout (shared with the C-ABI by convention only): W is (n, k) row-major;
 * codes are (n, k/2) bytes with element k in the low nibble when k is even;
 * NVFP4 scales are (n, k/16) E4M3 bytes, MXFP4 scales are (n, k/32) E8M0 bytes.
 * bf16 values are passed as their uint16 bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Scalar decoders (OCP definitions)                                          */
/* ------------------------------------------------------------------------- */

/* bf16 bit pattern -> exact value (bf16 is the top half of a binary32). */
static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; no inf/nan. */
double orc_e2m1_decode(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return s ? -mag : mag;
}

/* E4M3 "FN": sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
 * exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities. */
double orc_e4m3_decode(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    mag = (e == 0) ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0: unsigned power of two 2^(code-127); 0xFF is NaN; there is no zero. */
double orc_e8m0_decode(int code) {
    if (code == 0xFF) return NAN;
    return ldexp(1.0, code - 127);
}

/* ------------------------------------------------------------------------- */
/* Value grids: the non-negative values of each format, ascending by code.    */
/* The index into the grid is the (magnitude) code, so "ties to the even      */
/* code" is "ties to the even index".                                         */
/* ------------------------------------------------------------------------- */

static double E2M1_GRID[8];     /* codes 0..7           : 0 .. 6     */
static double E4M3_GRID[127];   /* codes 0x00..0x7E     : 0 .. 448   */
static double E8M0_GRID[255];   /* codes 0x00..0xFE     : 2^-127 .. 2^127 */
static int grids_ready = 0;

static void init_grids(void) {
    int i;
    if (grids_ready) return;
    for (i = 0; i < 8; i++) E2M1_GRID[i] = orc_e2m1_decode(i);
    for (i = 0; i < 127; i++) E4M3_GRID[i] = orc_e4m3_decode(i);
    for (i = 0; i < 255; i++) E8M0_GRID[i] = orc_e8m0_decode(i);
    grids_ready = 1;
}

void orc_init(void) { init_grids(); }

/* Sign of (a/D - g) for D > 0, decided exactly as the sign of a - g*D. */
static int cmp_quot(double a, double D, double g) {
    double p = g * D;
    return (a > p) - (a < p);
}

/* Round the exact quotient a/D (a >= 0, D > 0) to the nearest value of an
 * ascending grid: ties go to the even index, values at or above the top
 * saturate to the top, values below the bottom go to the bottom. */
static int rne_sat_quot(double a, double D, const double *grid, int n) {
    int i = 0, c;
    double mid;
    if (cmp_quot(a, D, grid[n - 1]) >= 0) return n - 1;
    while (i + 1 < n && cmp_quot(a, D, grid[i + 1]) >= 0) i++;
    /* now grid[i] <= a/D < grid[i+1], or a/D < grid[0] with i == 0 */
    mid = 0.5 * (grid[i] + grid[i + 1]);
    c = cmp_quot(a, D, mid);
    if (c > 0) return i + 1;
    if (c < 0) return i;
    return (i % 2 == 0) ? i : i + 1;
}

/* Sign of (hi + lo - g) where (hi, lo) is an exact TwoSum pair and g is a
 * binary64 value: if hi != g the rounded sum already decides, else lo does. */
static int cmp_pair(double hi, double lo, double g) {
    if (hi != g) return (hi > g) - (hi < g);
    return (lo > 0) - (lo < 0);
}

/* Same rounding as rne_sat_quot, for the exact value hi + lo. */
static int rne_sat_pair(double hi, double lo, const double *grid, int n) {
    int i = 0, c;
    double mid;
    if (cmp_pair(hi, lo, grid[n - 1]) >= 0) return n - 1;
    while (i + 1 < n && cmp_pair(hi, lo, grid[i + 1]) >= 0) i++;
    mid = 0.5 * (grid[i] + grid[i + 1]);
    c = cmp_pair(hi, lo, mid);
    if (c > 0) return i + 1;
    if (c < 0) return i;
    return (i % 2 == 0) ? i : i + 1;
}

/* Knuth's TwoSum: hi = fl(a + b), lo = (a + b) - hi exactly. */
static void two_sum(double a, double b, double *hi, double *lo) {
    double s = a + b;
    double bb = s - a;
    double err = (a - (s - bb)) + (b - bb);
    *hi = s;
    *lo = err;
}

/* Exposed for the format tests: magnitude codes for the exact quotient a/D. */
int orc_e2m1_rne_quot(double a, double D) { init_grids(); return rne_sat_quot(a, D, E2M1_GRID, 8); }
int orc_e4m3_rne_quot(double a, double D) { init_grids(); return rne_sat_quot(a, D, E4M3_GRID, 127); }

/* Round an exact binary64 value once, to nearest even, to bf16 (returns the
 * bit pattern).  bf16 has 8 significant bits and binary32's exponent range:
 * quantum 2^(e-7) for |v| in [2^e, 2^(e+1)), 2^-133 below 2^-126, and values
 * that round past the largest finite bf16 become infinity. */
uint16_t orc_round_bf16(double v) {
    double a = fabs(v), q, r;
    int ex;
    float f;
    uint32_t u;
    if (isnan(v)) return 0x7FC0;
    if (a == 0.0 || isinf(a)) {
        f = (float)v;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    frexp(a, &ex);                 /* a in [2^(ex-1), 2^ex) */
    q = (ex - 1 < -126) ? ldexp(1.0, -133) : ldexp(1.0, ex - 8);
    r = nearbyint(a / q) * q;      /* a/q is exact; nearbyint rounds half to even */
    if (r > ldexp(255.0, 120)) r = INFINITY;   /* largest finite bf16 is 255 * 2^120 */
    f = (float)(v < 0 ? -r : r);
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------- */
/* Quantize                                                                    */
/* ------------------------------------------------------------------------- */

static void put_code(uint8_t *codes_row, int64_t kk, int code) {
    uint8_t *b = &codes_row[kk >> 1];
    if ((kk & 1) == 0) *b = (uint8_t)((*b & 0xF0) | (code & 0xF));
    else               *b = (uint8_t)((*b & 0x0F) | ((code & 0xF) << 4));
}

static int get_code(const uint8_t *codes_row, int64_t kk) {
    uint8_t b = codes_row[kk >> 1];
    return (kk & 1) ? (b >> 4) : (b & 0xF);
}

/* NVFP4 tensor scale: A = max |w| over the tensor, s_t = fl32(A / (6*448)).
 * Correctly rounded binary32 division.  A non-finite input gives a
 * non-finite s_t (NaN if any NaN, else +inf). */
float orc_nvfp4_tensor_scale(const uint16_t *w, int64_t count) {
    double A = 0.0;
    int has_nan = 0;
    int64_t i;
    for (i = 0; i < count; i++) {
        double a = fabs(bf16_value(w[i]));
        if (isnan(a)) has_nan = 1;
        else if (a > A) A = a;
    }
    if (has_nan) return NAN;
    {
        volatile float Af = (float)A;     /* exact: A is a bf16 value */
        volatile float den = 2688.0f;     /* 6 * 448, exact */
        return Af / den;
    }
}

/* NVFP4 codes of one row given its block scales and the tensor scale
 * (also the frozen-scale quantize).  Per element: S_b = dec(sb)*s_t exactly;
 * S_b == 0 flushes to a signed zero code; otherwise the magnitude code is
 * RNE_sat(|w| / S_b) on the E2M1 grid. */
static void nvfp4_codes_row(const uint16_t *wrow, int64_t k, const uint8_t *srow,
                            float st, uint8_t *crow) {
    int64_t b, j;
    for (b = 0; b < k / 16; b++) {
        double Sb = orc_e4m3_decode(srow[b]) * (double)st;
        for (j = 0; j < 16; j++) {
            int64_t kk = b * 16 + j;
            double v = bf16_value(wrow[kk]);
            int sign = signbit(v) ? 8 : 0;
            int mag = 0;
            if (Sb != 0.0 && !isnan(Sb)) mag = rne_sat_quot(fabs(v), Sb, E2M1_GRID, 8);
            put_code(crow, kk, sign | mag);
        }
    }
}

/* NVFP4 quantize: tensor scale, then per 16-block along K the E4M3 block
 * scale sb = RNE_sat(a_b / (6 s_t)) (0 when s_t == 0), then the codes. */
/* Steps after the tensor scale, for rows of a tensor whose s_t is given (the
 * tests use it to check sampled rows of large tensors). */
void orc_nvfp4_quantize_with_tensor_scale(const uint16_t *w, int64_t n, int64_t k, float st,
                                          uint8_t *codes, uint8_t *scales) {
    int64_t r;
    init_grids();
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; r++) {
        const uint16_t *wrow = w + r * k;
        uint8_t *srow = scales + r * (k / 16);
        int64_t b, j;
        for (b = 0; b < k / 16; b++) {
            double ab = 0.0;
            for (j = 0; j < 16; j++) {
                double a = fabs(bf16_value(wrow[b * 16 + j]));
                if (a > ab) ab = a;
            }
            if (st == 0.0f || !isfinite(st)) srow[b] = 0;
            else srow[b] = (uint8_t)rne_sat_quot(ab, 6.0 * (double)st, E4M3_GRID, 127);
        }
        nvfp4_codes_row(wrow, k, srow, st, codes + r * (k / 2));
    }
}

void orc_nvfp4_quantize(const uint16_t *w, int64_t n, int64_t k,
                        uint8_t *codes, uint8_t *scales, float *tensor_scale) {
    float st = orc_nvfp4_tensor_scale(w, n * k);
    *tensor_scale = st;
    orc_nvfp4_quantize_with_tensor_scale(w, n, k, st, codes, scales);
}

void orc_nvfp4_quantize_frozen(const uint16_t *w, int64_t n, int64_t k,
                               const uint8_t *scales, float tensor_scale, uint8_t *codes) {
    int64_t r;
    init_grids();
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; r++)
        nvfp4_codes_row(w + r * k, k, scales + r * (k / 16), tensor_scale, codes + r * (k / 2));
}

/* MXFP4 codes of one row given its E8M0 block scales: RNE_sat(|w| / 2^e). */
static void mxfp4_codes_row(const uint16_t *wrow, int64_t k, const uint8_t *srow, uint8_t *crow) {
    int64_t b, j;
    for (b = 0; b < k / 32; b++) {
        double D = orc_e8m0_decode(srow[b]);
        for (j = 0; j < 32; j++) {
            int64_t kk = b * 32 + j;
            double v = bf16_value(wrow[kk]);
            int sign = signbit(v) ? 8 : 0;
            int mag = isnan(D) ? 0 : rne_sat_quot(fabs(v), D, E2M1_GRID, 8);
            put_code(crow, kk, sign | mag);
        }
    }
}

/* MXFP4 block scale exponent: e = floor(log2 a_b) - 2 (2 is E2M1's largest
 * exponent), taken exactly from the binary exponent; a_b == 0 gives -127;
 * e is clamped to [-127, 127]; the stored byte is e + 127.  A block holding
 * inf or NaN gets the NaN scale 0xFF. */
int orc_mxfp4_scale_code(double ab) {
    int ex, e;
    if (!isfinite(ab)) return 0xFF;
    if (ab == 0.0) return 0;
    frexp(ab, &ex);            /* ab in [2^(ex-1), 2^ex): floor(log2 ab) = ex - 1 */
    e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e + 127;
}

void orc_mxfp4_quantize(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales) {
    int64_t r;
    init_grids();
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; r++) {
        const uint16_t *wrow = w + r * k;
        uint8_t *srow = scales + r * (k / 32);
        int64_t b, j;
        for (b = 0; b < k / 32; b++) {
            double ab = 0.0;
            int nonfinite = 0;
            for (j = 0; j < 32; j++) {
                double a = fabs(bf16_value(wrow[b * 32 + j]));
                if (!isfinite(a)) nonfinite = 1;
                else if (a > ab) ab = a;
            }
            srow[b] = (uint8_t)(nonfinite ? 0xFF : orc_mxfp4_scale_code(ab));
        }
        mxfp4_codes_row(wrow, k, srow, codes + r * (k / 2));
    }
}

void orc_mxfp4_quantize_frozen(const uint16_t *w, int64_t n, int64_t k,
                               const uint8_t *scales, uint8_t *codes) {
    int64_t r;
    init_grids();
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; r++)
        mxfp4_codes_row(w + r * k, k, scales + r * (k / 32), codes + r * (k / 2));
}

/* ------------------------------------------------------------------------- */
/* Dequantize                                                                  */
/* ------------------------------------------------------------------------- */

/* Exact decoded value of element (row, kk): e2m1(c) * dec(sb) * s_t (NVFP4, at
 * most 30 significant bits) or e2m1(c) * 2^(sb-127) (MXFP4). fmt 0 = NVFP4. */
static double weight_value(int fmt, const uint8_t *crow, const uint8_t *srow, float st, int64_t kk) {
    double q = orc_e2m1_decode(get_code(crow, kk));
    if (fmt == 0) return q * orc_e4m3_decode(srow[kk / 16]) * (double)st;
    return q * orc_e8m0_decode(srow[kk / 32]);
}

/* Exact values as binary64 (used by tests and by the linear below). */
void orc_dequantize_f64(int fmt, const uint8_t *codes, const uint8_t *scales, float st,
                        int64_t n, int64_t k, double *out) {
    int64_t r, kk;
    int64_t sb_per_row = (fmt == 0) ? k / 16 : k / 32;
    init_grids();
#pragma omp parallel for schedule(static) private(kk)
    for (r = 0; r < n; r++)
        for (kk = 0; kk < k; kk++)
            out[r * k + kk] = weight_value(fmt, codes + r * (k / 2), scales + r * sb_per_row, st, kk);
}

/* Rounded once to binary32 (RNE). */
void orc_dequantize_f32(int fmt, const uint8_t *codes, const uint8_t *scales, float st,
                        int64_t n, int64_t k, float *out) {
    int64_t r, kk;
    int64_t sb_per_row = (fmt == 0) ? k / 16 : k / 32;
    init_grids();
#pragma omp parallel for schedule(static) private(kk)
    for (r = 0; r < n; r++)
        for (kk = 0; kk < k; kk++) {
            double v = weight_value(fmt, codes + r * (k / 2), scales + r * sb_per_row, st, kk);
            out[r * k + kk] = isnan(v) ? NAN : (float)v;    /* one canonical quiet NaN */
        }
}

/* Rounded once to bf16 (RNE), returned as bit patterns. */
void orc_dequantize_bf16(int fmt, const uint8_t *codes, const uint8_t *scales, float st,
                         int64_t n, int64_t k, uint16_t *out) {
    int64_t r, kk;
    int64_t sb_per_row = (fmt == 0) ? k / 16 : k / 32;
    init_grids();
#pragma omp parallel for schedule(static) private(kk)
    for (r = 0; r < n; r++)
        for (kk = 0; kk < k; kk++)
            out[r * k + kk] = orc_round_bf16(weight_value(fmt, codes + r * (k / 2), scales + r * sb_per_row, st, kk));
}

/* ------------------------------------------------------------------------- */
/* Scale-only merge                                                            */
/* ------------------------------------------------------------------------- */

/* New scale byte from a stored scale byte and an additive delta in the decoded
 * scale domain: v = dec(S) + delta exactly; v <= 0 gives the smallest code
 * (E4M3 0x00 = 0, E8M0 0x00 = 2^-127); otherwise v is rounded to the nearest
 * value of the format's scale grid, ties to the even code, saturating at the
 * top (E4M3 448 = 0x7E, E8M0 2^127 = 0xFE).  dec(S) is the signed E4M3 value,
 * as in dequantize.  A NaN scale or delta gives the
 * format's NaN code (0x7F, 0xFF). */
int orc_merge_scale(int fmt, int code, float delta) {
    double base = (fmt == 0) ? orc_e4m3_decode(code) : orc_e8m0_decode(code);
    double hi, lo;
    init_grids();
    if (isnan(base) || isnan(delta)) return (fmt == 0) ? 0x7F : 0xFF;
    two_sum(base, (double)delta, &hi, &lo);
    if (hi < 0.0 || (hi == 0.0 && lo <= 0.0)) return 0;
    if (isinf(hi)) return (fmt == 0) ? 0x7E : 0xFE;
    if (fmt == 0) return rne_sat_pair(hi, lo, E4M3_GRID, 127);
    return rne_sat_pair(hi, lo, E8M0_GRID, 255);
}

void orc_merge_scales(int fmt, const uint8_t *scales_in, const float *deltas, int64_t num_blocks,
                      uint8_t *scales_out, const uint8_t *codes_in, uint8_t *codes_out, int64_t code_bytes) {
    int64_t i;
    init_grids();
    for (i = 0; i < num_blocks; i++) scales_out[i] = (uint8_t)orc_merge_scale(fmt, scales_in[i], deltas[i]);
    if (codes_out && codes_in && codes_out != codes_in) memcpy(codes_out, codes_in, (size_t)code_bytes);
}

/* ------------------------------------------------------------------------- */
/* W4A16 linear: y = x deq(W)^T + (x A^T) B^T, binary64, k ascending           */
/* ------------------------------------------------------------------------- */

/* One output y[m, n] with an already computed LoRA row t[m, :] (may be NULL). */
static double linear_one(int fmt, const uint16_t *x_row, int64_t k,
                         const uint8_t *crow, const uint8_t *srow, float st,
                         const double *t_row, const uint16_t *b_row, int r) {
    double acc = 0.0;
    int64_t kk;
    int j;
    for (kk = 0; kk < k; kk++) acc += bf16_value(x_row[kk]) * weight_value(fmt, crow, srow, st, kk);
    if (t_row && b_row)
        for (j = 0; j < r; j++) acc += t_row[j] * bf16_value(b_row[j]);
    return acc;
}

/* t[m, j] = sum_k x[m, k] A[j, k] */
static void lora_down(const uint16_t *x, int64_t m, int64_t k, const uint16_t *a, int r, double *t) {
    int64_t i, kk;
    int j;
    for (i = 0; i < m; i++)
        for (j = 0; j < r; j++) {
            double acc = 0.0;
            for (kk = 0; kk < k; kk++) acc += bf16_value(x[i * k + kk]) * bf16_value(a[(int64_t)j * k + kk]);
            t[i * r + j] = acc;
        }
}

/* Full (m, n) output.  lora_a (r, k) and lora_b (n, r) may be NULL (r ignored). */
void orc_linear(int fmt, const uint16_t *x, int64_t m, int64_t k,
                const uint8_t *codes, const uint8_t *scales, float st, int64_t n,
                const uint16_t *lora_a, const uint16_t *lora_b, int r, double *y) {
    int64_t sb_per_row = (fmt == 0) ? k / 16 : k / 32;
    double *t = NULL;
    int64_t idx;
    init_grids();
    if (lora_a && lora_b && r > 0) {
        t = (double *)malloc(sizeof(double) * (size_t)(m * r));
        lora_down(x, m, k, lora_a, r, t);
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (idx = 0; idx < m * n; idx++) {
        int64_t i = idx / n, nn = idx % n;
        y[idx] = linear_one(fmt, x + i * k, k, codes + nn * (k / 2), scales + nn * sb_per_row, st,
                            t ? t + i * r : NULL, t ? lora_b + nn * r : NULL, r);
    }
    free(t);
}

/* Selected outputs only: y[s] = y_full[rows[s], cols[s]]. */
void orc_linear_sampled(int fmt, const uint16_t *x, int64_t m, int64_t k,
                        const uint8_t *codes, const uint8_t *scales, float st, int64_t n,
                        const uint16_t *lora_a, const uint16_t *lora_b, int r,
                        const int64_t *rows, const int64_t *cols, int64_t count, double *y) {
    int64_t sb_per_row = (fmt == 0) ? k / 16 : k / 32;
    double *t = NULL;
    int64_t s;
    init_grids();
    (void)n;
    if (lora_a && lora_b && r > 0) {
        t = (double *)malloc(sizeof(double) * (size_t)(m * r));
        lora_down(x, m, k, lora_a, r, t);
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (s = 0; s < count; s++) {
        int64_t i = rows[s], nn = cols[s];
        y[s] = linear_one(fmt, x + i * k, k, codes + nn * (k / 2), scales + nn * sb_per_row, st,
                          t ? t + i * r : NULL, t ? lora_b + nn * r : NULL, r);
    }
    free(t);
}

/* Grouped (MoE) linear without LoRA: for expert e and each row q in
 * [offsets[e], offsets[e+1]), y[q, :] = x[row_index[q], :] deq(W_e)^T.
 * codes is (E, n, k/2), scales (E, n, k/blk), tensor_scales (E) (NVFP4). */
void orc_grouped_linear(int fmt, const uint16_t *x, const int32_t *row_index, const int32_t *offsets,
                        int64_t num_experts, int64_t n, int64_t k,
                        const uint8_t *codes, const uint8_t *scales, const float *tensor_scales,
                        double *y) {
    int64_t sb_per_row = (fmt == 0) ? k / 16 : k / 32;
    int64_t e;
    init_grids();
    for (e = 0; e < num_experts; e++) {
        int64_t q0 = offsets[e], q1 = offsets[e + 1], idx;
        const uint8_t *ce = codes + e * n * (k / 2);
        const uint8_t *se = scales + e * n * sb_per_row;
        float st = (fmt == 0) ? tensor_scales[e] : 1.0f;
#pragma omp parallel for schedule(static)
        for (idx = 0; idx < (q1 - q0) * n; idx++) {
            int64_t q = q0 + idx / n, nn = idx % n;
            y[q * n + nn] = linear_one(fmt, x + (int64_t)row_index[q] * k, k, ce + nn * (k / 2),
                                       se + nn * sb_per_row, st, NULL, NULL, 0);
        }
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
