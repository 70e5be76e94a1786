/*
 * intlora_oracle.c -- plain, slow, obviously-correct CPU oracle for the IntLoRA
 * integer merge and the W8A8/W4A8 integer linear layer that consumes it.
 *
 * THIS FILE IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant generator with the GPU library; both sides implement the
 * same written definitions independently.
 *
 * Sources (the pages):
 *   [IntLoRA notes]  "IntLoRA: Integral Low-rank Adaptation of Quantized
 *                    Diffusion Models" (Paper-Notes, ICML 2025), sections
 *                    "1. AQS" (eq. W' = Q[W - sg(R)] + sg(R) + AB),
 *                    "2. MLA" (eq. W' = [s*I + (R+AB)/(W_round - z)] (.) (W_round - z)),
 *                    "3. VMC" (eq. R* = r^alpha R, r = sigma_W / sigma_R),
 *                    "two implementation variants" (MUL eq. and SHIFT eq.).
 *   [IntLoRA summary] atlas.scime.ai summary: Laplace auxiliary matrix ablation,
 *                    alpha -> 1.5 ablation.
 *   [SVDQuant notes] "Implementation details": per-token dynamic activation
 *                    quantization with per-channel weight quantization (8-bit).
 *   Philox4x32-10:   Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *                    Easy as 1, 2, 3", SC'11 (the published generator).
 *
 * Where floating point decides an integer (a quantized code) the oracle takes
 * the decision in IEEE binary32 with round-to-nearest-even, one operation at a
 * time, in the order written below; this file must be compiled with
 * -ffp-contract=off and without -ffast-math.  Continuous quantities with no
 * integer consequence (sigma_W, the VMC pow) are computed in binary64.
 *
 * Readings of points the pages leave open are listed in the header of each
 * function.  Layouts: W, A, B, R*, U are row-major fp32; W is d x n (out x in);
 * A is d x r, B is r x n; codes (W_round) are one uint8 per element here
 * (no nibble packing: packing is a GPU storage detail).
 *
 * OpenMP is used only to run independent rows / tokens concurrently; it never
 * changes the order of operations inside one output.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 as published (SC'11): 10 rounds; each round multiplies two   */
/* counter words by the two round multipliers, XORs the high halves with the  */
/* other two words and the round key, and the key is advanced by the two      */
/* Weyl constants between rounds.                                             */
/* ------------------------------------------------------------------------- */
ORA_API void ora_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)x0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)x2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Batch form, for the statistics / known-answer tests. */
ORA_API void ora_philox_batch(int64_t count, const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
    for (int64_t i = 0; i < count; ++i) ora_philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i);
}

/* The random word of matrix element (i, j) of layer `layer_id`.
 * Reading (AQS: R is regenerated from statistics and a fixed seed, so it need
 * not be stored): the element's linear index q = i*n + j selects counter
 * (q >> 2 low 32 bits, q >> 34, layer_id, 0) and output word q & 3; the key is
 * (seed low 32 bits, seed high 32 bits).  R is then a pure function of
 * (seed, layer_id, i, j). */
static uint32_t element_word(uint64_t seed, uint32_t layer_id, uint64_t q) {
    uint32_t ctr[4] = {(uint32_t)(q >> 2), (uint32_t)(q >> 34), layer_id, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    ora_philox4x32_10(ctr, key, out);
    return out[q & 3];
}

/* ------------------------------------------------------------------------- */
/* Natural log, correctly rounded to binary32.                                */
/* Definition: RN32(ln g).  Computed as the binary64 log rounded to binary32.  */
/* That equals RN32(ln g) unless ln g sits within the binary64 error of a      */
/* binary32 rounding midpoint; the test suite checks every g this oracle ever  */
/* feeds it (the 2^22 odd multiples of 2^-23 in (0,1)) against a 40-digit      */
/* decimal logarithm, so on that domain this is the exact definition.          */
/* ------------------------------------------------------------------------- */
ORA_API float ora_ln_rn32(float g) { return (float)log((double)g); }

/* Laplace(0, b = 1) sample from one 32-bit word, by the inverse CDF
 * L = -sign(v) * ln(1 - 2|v|) with v = u - 1/2 and
 * u = (2 * floor(x / 2^9) + 1) / 2^24, an exact binary32 in (0,1) that is never
 * 1/2.  v, |v| and g = 1 - 2|v| are exact in binary32 (g is an odd multiple of
 * 2^-23).  Laplace is the distribution the ablation retains for R. */
ORA_API float ora_laplace(uint32_t x) {
    uint32_t a = x >> 9;
    float u = (float)(2u * a + 1u) * 0x1p-24f;
    float v = u - 0.5f;
    float g = 1.0f - 2.0f * fabsf(v);
    float lg = ora_ln_rn32(g);
    return (v < 0.0f) ? lg : -lg;
}

ORA_API void ora_ln_batch(int64_t count, const float* g, float* out) {
    for (int64_t i = 0; i < count; ++i) out[i] = ora_ln_rn32(g[i]);
}

ORA_API void ora_laplace_batch(int64_t count, const uint32_t* words, float* out) {
    for (int64_t i = 0; i < count; ++i) out[i] = ora_laplace(words[i]);
}

/* ------------------------------------------------------------------------- */
/* The other laws of the auxiliary-matrix ablation (IntLoRA summary table,    */
/* "Measured effects": Gaussian, Cauchy and Student-t samples against the     */
/* Laplace one).  The pages name the laws only; readings:                     */
/*  - every law takes the Laplace sampler's uniform u = (2 floor(x/2^9)+1)2^-24 */
/*    of the element's word x;                                                 */
/*  - Gaussian: the Box-Muller transform on the word pairs (0, 1) and (2, 3)   */
/*    of the element's Philox block (u1 from the first word, u2 from the       */
/*    second; element 2p takes the cosine, 2p + 1 the sine):                   */
/*      L = RN32(ln u1), S = RN32(sqrt(-2 L)), C = RN32(cos(2 pi u2)) or       */
/*      RN32(sin(2 pi u2)), sample = RN32(S C);                                */
/*  - Cauchy(0, 1): RN32(tan(pi (u - 1/2)));                                   */
/*  - Student-t with 2 degrees of freedom (its inverse distribution function   */
/*    is algebraic): RN32((2u - 1) / sqrt(2 u (1 - u))).                       */
/* Each RN32(f) is the binary64 value rounded once; the arguments are reduced  */
/* exactly (v has at most 24 significant bits) to [0, 1/4] before libm's sin,  */
/* cos or tan, so the binary64 value is within a few units of 2^-53 and the    */
/* test suite decides every point near a binary32 midpoint with 40 digits.     */
/* ------------------------------------------------------------------------- */
static double sinpi_small(double a) { return sin(M_PI * a); } /* 0 <= a <= 1/4 */
static double cospi_small(double a) { return cos(M_PI * a); } /* 0 <= a <= 1/4 */

/* cos(pi v), sin(pi v) for 0 < v < 2 */
ORA_API double ora_cospi(double v) {
    double a = v > 1.0 ? 2.0 - v : v; /* cos(pi v) = cos(pi (2 - v)) */
    double sign = 1.0;
    if (a > 0.5) { a = 1.0 - a; sign = -1.0; } /* cos(pi a) = -cos(pi (1 - a)) */
    return sign * (a <= 0.25 ? cospi_small(a) : sinpi_small(0.5 - a));
}
ORA_API double ora_sinpi(double v) {
    double sign = 1.0, a = v;
    if (a > 1.0) { a = a - 1.0; sign = -1.0; } /* sin(pi v) = -sin(pi (v - 1)) */
    if (a > 0.5) a = 1.0 - a;                  /* sin(pi a) = sin(pi (1 - a)) */
    return sign * (a <= 0.25 ? sinpi_small(a) : cospi_small(0.5 - a));
}
/* tan(pi v) for |v| < 1/2 */
ORA_API double ora_tanpi(double v) {
    double a = fabs(v), t;
    if (a <= 0.25) t = tan(M_PI * a);
    else t = cospi_small(0.5 - a) / sinpi_small(0.5 - a); /* cot(pi (1/2 - a)) */
    return v < 0.0 ? -t : t;
}

ORA_API void ora_trig_batch(int64_t count, const double* v, int kind, double* out) {
    for (int64_t i = 0; i < count; ++i)
        out[i] = kind == 0 ? ora_cospi(v[i]) : kind == 1 ? ora_sinpi(v[i]) : ora_tanpi(v[i]);
}

static double uniform24(uint32_t x) { return (double)(2u * (x >> 9) + 1u) * 0x1p-24; }

/* element e (0..3) of the block of four words w under law `dist` (0 Laplace,
 * 1 Gaussian, 2 Cauchy, 3 Student-t(2)), before the VMC scale */
ORA_API float ora_aux(const uint32_t w[4], int e, int dist) {
    if (dist == 0) return ora_laplace(w[e]);
    if (dist == 1) {
        double u1 = uniform24(w[e & 2]), u2 = uniform24(w[(e & 2) | 1]);
        float L = (float)log(u1);
        float S = sqrtf(-2.0f * L);
        float C = (float)((e & 1) ? ora_sinpi(2.0 * u2) : ora_cospi(2.0 * u2));
        return S * C;
    }
    double v = uniform24(w[e]) - 0.5; /* exact */
    if (dist == 2) return (float)ora_tanpi(v);
    double u = uniform24(w[e]);
    return (float)((2.0 * u - 1.0) / sqrt(2.0 * u * (1.0 - u)));
}

ORA_API void ora_aux_batch(int64_t blocks, const uint32_t* words, int dist, float* out) {
    for (int64_t t = 0; t < blocks; ++t)
        for (int e = 0; e < 4; ++e) out[4 * t + e] = ora_aux(words + 4 * t, e, dist);
}

/* R*_ij = c_i * L_ij  (VMC: R* = r^alpha R with c_i = r_i^alpha passed in). */
ORA_API void ora_gen_r(int64_t d, int64_t n, uint64_t seed, uint32_t layer_id, const float* c, float* r_out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            uint64_t q = (uint64_t)i * (uint64_t)n + (uint64_t)j;
            float L = ora_laplace(element_word(seed, layer_id, q));
            r_out[i * n + j] = c[i] * L;
        }
    }
}

/* Rows [row0, row0 + rows) of R* under law `dist`: the element's whole Philox block
 * (the Gaussian pairs two of its words). */
ORA_API void ora_gen_r_dist(int64_t row0, int64_t rows, int64_t n, uint64_t seed, uint32_t layer_id, int dist,
                            const float* c, float* r_out) {
#pragma omp parallel for schedule(static)
    for (int64_t ii = 0; ii < rows; ++ii) {
        int64_t i = row0 + ii;
        for (int64_t j = 0; j < n; ++j) {
            uint64_t q = (uint64_t)i * (uint64_t)n + (uint64_t)j;
            uint32_t ctr[4] = {(uint32_t)(q >> 2), (uint32_t)(q >> 34), layer_id, 0u};
            uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
            uint32_t w[4];
            ora_philox4x32_10(ctr, key, w);
            r_out[ii * n + j] = c[ii] * ora_aux(w, (int)(q & 3), dist);
        }
    }
}

/* Rows [row0, row0 + rows) only: the same values as the full matrix, because R
 * depends on (seed, layer_id, i, j) alone. */
ORA_API void ora_gen_r_rows(int64_t row0, int64_t rows, int64_t n, uint64_t seed, uint32_t layer_id,
                            const float* c, float* r_out) {
#pragma omp parallel for schedule(static)
    for (int64_t ii = 0; ii < rows; ++ii) {
        int64_t i = row0 + ii;
        for (int64_t j = 0; j < n; ++j) {
            uint64_t q = (uint64_t)i * (uint64_t)n + (uint64_t)j;
            r_out[ii * n + j] = c[ii] * ora_laplace(element_word(seed, layer_id, q));
        }
    }
}

/* ------------------------------------------------------------------------- */
/* VMC statistics.  sigma_W,i = population standard deviation of row i of the */
/* original weight (per output channel), in binary64, rounded to binary32.     */
/* c_i = RN32((sigma_W,i / sigma_R)^alpha) with sigma_R = sqrt(2), the         */
/* standard deviation of the unit Laplace distribution.                        */
/*                                                                             */
/* Reading: the pages fix no summation order, and binary64 sums of a row's     */
/* binary32 values are not exact in general, so the order is part of the      */
/* definition here.  Each of the two row sums (the values, for the mean; the   */
/* squared deviations e*e, e = x - mean, for the variance) is formed as        */
/*   (1) 256 partial sums: partial t adds x_j for j = t, t + 256, t + 512, ... */
/*       in increasing j, starting from 0;                                      */
/*   (2) in each group of 64 consecutive partials, a halving tree: entry k     */
/*       becomes entry k plus entry k + h, for h = 32, 16, 8, 4, 2, 1;          */
/*   (3) the four group results added in order: ((g0 + g1) + g2) + g3.         */
/* mean = sum / n; sigma = RN32(sqrt(sum of squares / n)).                     */
/* ------------------------------------------------------------------------- */
static double ordered_row_sum(const double* v, int64_t n) {
    double part[256];
    for (int t = 0; t < 256; ++t) {
        double a = 0.0;
        for (int64_t j = t; j < n; j += 256) a += v[j];
        part[t] = a;
    }
    double g[4];
    for (int w = 0; w < 4; ++w) {
        double* p = part + 64 * w;
        for (int h = 32; h >= 1; h >>= 1)
            for (int k = 0; k < h; ++k) p[k] = p[k] + p[k + h];
        g[w] = p[0];
    }
    return ((g[0] + g[1]) + g[2]) + g[3];
}

ORA_API void ora_sigma_w(int64_t d, int64_t n, const float* W, float* sigma_out) {
#pragma omp parallel
    {
        double* v = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < d; ++i) {
            const float* row = W + i * n;
            for (int64_t j = 0; j < n; ++j) v[j] = (double)row[j];
            const double mean = ordered_row_sum(v, n) / (double)n;
            for (int64_t j = 0; j < n; ++j) {
                const double e = (double)row[j] - mean;
                v[j] = e * e;
            }
            sigma_out[i] = (float)sqrt(ordered_row_sum(v, n) / (double)n);
        }
        free(v);
    }
}

ORA_API void ora_vmc_scale(int64_t d, const float* sigma_w, double alpha, float* c_out) {
    for (int64_t i = 0; i < d; ++i) c_out[i] = (float)pow((double)sigma_w[i] / sqrt(2.0), alpha);
}

/* sigma_R = 1 for the other laws: the Gaussian's standard deviation, and the unit scale
 * of the Cauchy and Student-t(2) laws, whose variance is not finite (a reading). */
ORA_API void ora_vmc_scale_dist(int64_t d, const float* sigma_w, double alpha, int dist, float* c_out) {
    if (dist == 0) {
        ora_vmc_scale(d, sigma_w, alpha, c_out);
        return;
    }
    for (int64_t i = 0; i < d; ++i) c_out[i] = (float)pow((double)sigma_w[i], alpha);
}

/* ------------------------------------------------------------------------- */
/* Uniform affine quantizer Q[.] of the AQS base term W - R*, per output row.  */
/* Reading: asymmetric min/max quantizer whose range always contains 0,        */
/*   lo = min(0, min_j x), hi = max(0, max_j x), s = (hi - lo) / (2^b - 1)     */
/*   (s := 1 if that is 0), z = clamp(rint(-lo / s), 0, 2^b - 1),              */
/*   W_round = clamp(rint(x / s) + z, 0, 2^b - 1), rint = half to even.        */
/* ------------------------------------------------------------------------- */
ORA_API void ora_base_quant(int64_t d, int64_t n, int bits, const float* W, const float* rstar,
                            uint8_t* wround_out, int32_t* z_out, float* s_out) {
    const int qmax = (1 << bits) - 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d; ++i) {
        float lo = 0.0f, hi = 0.0f;
        for (int64_t j = 0; j < n; ++j) {
            float x = W[i * n + j] - rstar[i * n + j];
            if (x < lo) lo = x;
            if (x > hi) hi = x;
        }
        float s = (hi - lo) / (float)qmax;
        if (!(s > 0.0f)) s = 1.0f;
        float zf = rintf(-lo / s);
        int z = (int)zf;
        if (z < 0) z = 0;
        if (z > qmax) z = qmax;
        z_out[i] = z;
        s_out[i] = s;
        for (int64_t j = 0; j < n; ++j) {
            float x = W[i * n + j] - rstar[i * n + j];
            double code = (double)rintf(x / s) + (double)z;   /* exact: an integer plus a small integer */
            if (code < 0.0) code = 0.0;
            if (code > (double)qmax) code = (double)qmax;
            wround_out[i * n + j] = (uint8_t)code;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* MLA adaptation term.  The functions below take a block of `rows` rows:     */
/* wround, rstar, u (rows x n), z, s (rows), A (rows x r) are that block's    */
/* slices; B is the whole r x n matrix.                                       */
/*   w = W_round - z  (the signed pretrained integer); valid iff w != 0.       */
/*   acc = sum_k A[i,k] * B[k,j] as a binary32 fused multiply-add chain in     */
/*   increasing k starting from +0;  t = R*_ij + acc;  q = t / w (IEEE);       */
/*   U = s_i + q.                                                              */
/* Reading for w == 0 (the MLA quotient has a zero denominator): the element   */
/* is excluded from the U range and merges to 0.                               */
/* ------------------------------------------------------------------------- */
static int u_element(int64_t i, int64_t j, int64_t n, int r, const uint8_t* wround, const int32_t* z,
                     const float* s, const float* rstar, const float* A, const float* B, float* u_out) {
    int w = (int)wround[i * n + j] - z[i];
    if (w == 0) return 0;
    float acc = 0.0f;
    for (int k = 0; k < r; ++k) acc = fmaf(A[i * r + k], B[(int64_t)k * n + j], acc);
    float t = rstar[i * n + j] + acc;
    float q = t / (float)w;
    *u_out = s[i] + q;
    return 1;
}

/* a < b in the IEEE total order (-0 below +0); operands are never NaN. */
static int total_less(float a, float b) {
    if (a < b) return 1;
    return a == b && signbit(a) && !signbit(b);
}

/* U for every element (NaN marks w == 0, when u_out is given) and the row
 * range over valid elements: the least and greatest U in the IEEE total order
 * (so a zero extreme is -0 if any valid U is -0); U_min = +inf, U_max = -inf for
 * a row with no valid element. */
ORA_API void ora_adaptation(int64_t rows, int64_t n, int r, const uint8_t* wround, const int32_t* z, const float* s,
                            const float* rstar, const float* A, const float* B, float* u_out, float* umin_out,
                            float* umax_out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        float umin = INFINITY, umax = -INFINITY;
        for (int64_t j = 0; j < n; ++j) {
            float u;
            if (!u_element(i, j, n, r, wround, z, s, rstar, A, B, &u)) {
                if (u_out) u_out[i * n + j] = NAN;
                continue;
            }
            if (u_out) u_out[i * n + j] = u;
            if (total_less(u, umin)) umin = u;
            if (total_less(umax, u)) umax = u;
        }
        umin_out[i] = umin;
        umax_out[i] = umax;
    }
}

/* ------------------------------------------------------------------------- */
/* IntLoRA_MUL merge:  W' = s_bar * (U_round - z_bar) (.) (W_round - z).       */
/* Reading: per row, uniform affine quantization of U over the range          */
/*   lo = min(U_min, 0), hi = max(U_max, 0);  s_bar = (hi - lo) / (2^bU - 1)   */
/*   (s_bar := 1 unless positive);  z_bar = clamp(rint(-lo / s_bar), 0, 2^bU-1)*/
/*   U_round = clamp(rint(U / s_bar) + z_bar, 0, 2^bU - 1)  (IEEE division);   */
/*   m = (U_round - z_bar) * w exactly, stored as int16 with saturation       */
/*   (counted).  w == 0: U_round = z_bar, m = 0.                               */
/* The range is the row's own (U_min, U_max) unless range_given is nonzero:    */
/* then umin_out / umax_out hold a caller's range on entry and are used as it  */
/* is (s_bar and z_bar only need some range of U; the MUL equation does not   */
/* say where it comes from).                                                  */
/* Returns the number of saturated elements.                                  */
/* ------------------------------------------------------------------------- */
ORA_API void ora_mul_params(int64_t rows, int u_bits, const float* umin, const float* umax, float* sbar_out,
                            int32_t* zbar_out) {
    const int qmax = (1 << u_bits) - 1;
    for (int64_t i = 0; i < rows; ++i) {
        float lo = fminf(umin[i], 0.0f);
        float hi = fmaxf(umax[i], 0.0f);
        float sbar = (hi - lo) / (float)qmax;
        if (!(sbar > 0.0f)) sbar = 1.0f;
        float zf = rintf(-lo / sbar);
        int zbar = zf < 0.0f ? 0 : (zf > (float)qmax ? qmax : (int)zf);
        sbar_out[i] = sbar;
        zbar_out[i] = zbar;
    }
}

ORA_API int64_t ora_merge_mul(int64_t rows, int64_t n, int r, int u_bits, const uint8_t* wround, const int32_t* z,
                              const float* s, const float* rstar, const float* A, const float* B, int16_t* m_out,
                              uint8_t* uround_out, float* sbar_out, int32_t* zbar_out, float* umin_out,
                              float* umax_out, int range_given) {
    const int qmax = (1 << u_bits) - 1;
    int64_t sat_total = 0;
    if (!range_given) ora_adaptation(rows, n, r, wround, z, s, rstar, A, B, NULL, umin_out, umax_out);
    ora_mul_params(rows, u_bits, umin_out, umax_out, sbar_out, zbar_out);
#pragma omp parallel for schedule(static) reduction(+ : sat_total)
    for (int64_t i = 0; i < rows; ++i) {
        const float sbar = sbar_out[i];
        const int zbar = zbar_out[i];
        for (int64_t j = 0; j < n; ++j) {
            int w = (int)wround[i * n + j] - z[i];
            float u;
            int ur, mm;
            if (!u_element(i, j, n, r, wround, z, s, rstar, A, B, &u)) {
                ur = zbar;
                mm = 0;
            } else {
                double code = (double)rintf(u / sbar) + (double)zbar;
                if (code < 0.0) code = 0.0;
                if (code > (double)qmax) code = (double)qmax;
                ur = (int)code;
                mm = (ur - zbar) * w;
            }
            if (mm > 32767) { mm = 32767; ++sat_total; }
            if (mm < -32768) { mm = -32768; ++sat_total; }
            m_out[i * n + j] = (int16_t)mm;
            if (uround_out) uround_out[i * n + j] = (uint8_t)ur;
        }
    }
    return sat_total;
}

/* ------------------------------------------------------------------------- */
/* QLoRA-style comparison path (the flow IntLoRA removes, [IntLoRA notes]      */
/* research background): dequantize the base, add the auxiliary matrix and    */
/* the adapter in floating point, then re-quantize each row post-training.    */
/* Reading (binary32, round to nearest even, in this order):                  */
/*   deq = s_i * (W_round - z_i);  t = deq + R*_ij;                           */
/*   acc = the fused multiply-add chain of A[i,k] B[k,j] over k from +0 (the  */
/*   same product as the MLA term);  x = t + acc;                             */
/* then the base quantizer of "1. AQS" (ora_base_quant's reading) on x at     */
/* `bits`: lo = min(0, min x), hi = max(0, max x), s' = (hi - lo)/(2^b - 1)   */
/* (1 if 0), z' = clamp(rint(-lo / s')), code = clamp(rint(x / s') + z').     */
/* Every element takes part (no zero-denominator exclusion: there is none).   */
/* x_out (optional) receives x.                                               */
/* ------------------------------------------------------------------------- */
static float ptq_element(int64_t i, int64_t j, int64_t n, int r, const uint8_t* wround, const int32_t* z,
                         const float* s, const float* rstar, const float* A, const float* B) {
    int w = (int)wround[i * n + j] - z[i];
    float deq = s[i] * (float)w;
    float t = deq + rstar[i * n + j];
    float acc = 0.0f;
    for (int k = 0; k < r; ++k) acc = fmaf(A[i * r + k], B[(int64_t)k * n + j], acc);
    return t + acc;
}

ORA_API void ora_ptq_merge(int64_t rows, int64_t n, int r, int bits, const uint8_t* wround, const int32_t* z,
                           const float* s, const float* rstar, const float* A, const float* B, uint8_t* code_out,
                           float* s_out, int32_t* z_out, float* x_out) {
    const int qmax = (1 << bits) - 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        float lo = 0.0f, hi = 0.0f;
        for (int64_t j = 0; j < n; ++j) {
            float x = ptq_element(i, j, n, r, wround, z, s, rstar, A, B);
            if (x_out) x_out[i * n + j] = x;
            if (x < lo) lo = x;
            if (x > hi) hi = x;
        }
        float sq = (hi - lo) / (float)qmax;
        if (!(sq > 0.0f)) sq = 1.0f;
        float zf = rintf(-lo / sq);
        int zq = (int)zf;
        if (zq < 0) zq = 0;
        if (zq > qmax) zq = qmax;
        s_out[i] = sq;
        z_out[i] = zq;
        for (int64_t j = 0; j < n; ++j) {
            float x = ptq_element(i, j, n, r, wround, z, s, rstar, A, B);
            double code = (double)rintf(x / sq) + (double)zq;
            if (code < 0.0) code = 0.0;
            if (code > (double)qmax) code = (double)qmax;
            code_out[i * n + j] = (uint8_t)code;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* IntLoRA_SHIFT merge:  W' = sign(V) (.) [(W_round - z) >> shift].           */
/* Reading: V = U / s_bar with s_bar = max |U| over the row's valid elements  */
/*   (s_bar := 1 for an empty or all-zero row), so |V| <= 1 and only right     */
/*   shifts occur;  shift = clamp(-round(log2 |V|), 0, 2^bV - 1) (round to     */
/*   nearest; no ties exist since sqrt(2) is irrational);  ">>" is the         */
/*   arithmetic shift, i.e. floor(w / 2^shift);  V == 0 gives m = 0 and the    */
/*   largest shift code; m saturates to the signed bW-bit range (counted).    */
/*   w == 0: m = 0, shift code 255 (marker).                                    */
/* range_given: as for ora_merge_mul (s_bar = max(|U_min|, |U_max|) of the     */
/* caller's range).                                                           */
/* ------------------------------------------------------------------------- */
ORA_API int ora_log2_round(float a) {
    /* round(log2 a) for finite a > 0, in binary64: the binary32 nearest to a
     * half-integer power of two is more than 1e-8 away from it in log2, far
     * above the binary64 error. */
    double l = log2((double)a);
    return (int)floor(l + 0.5);
}

ORA_API void ora_log2_round_batch(int64_t count, const float* a, int32_t* out) {
    for (int64_t i = 0; i < count; ++i) out[i] = ora_log2_round(a[i]);
}

ORA_API float ora_shift_scale(float umin, float umax) {
    float sbar = fmaxf(fabsf(umin), fabsf(umax));
    if (!(sbar > 0.0f) || isinf(sbar)) sbar = 1.0f;
    return sbar;
}

ORA_API int64_t ora_merge_shift(int64_t rows, int64_t n, int r, int w_bits, int v_bits, const uint8_t* wround,
                                const int32_t* z, const float* s, const float* rstar, const float* A, const float* B,
                                int8_t* m_out, uint8_t* shift_out, float* sbar_out, float* umin_out,
                                float* umax_out, int range_given) {
    const int smax = (1 << v_bits) - 1;
    const int mhi = (1 << (w_bits - 1)) - 1, mlo = -(1 << (w_bits - 1));
    int64_t sat_total = 0;
    if (!range_given) ora_adaptation(rows, n, r, wround, z, s, rstar, A, B, NULL, umin_out, umax_out);
    for (int64_t i = 0; i < rows; ++i) sbar_out[i] = ora_shift_scale(umin_out[i], umax_out[i]);
#pragma omp parallel for schedule(static) reduction(+ : sat_total)
    for (int64_t i = 0; i < rows; ++i) {
        const float sbar = sbar_out[i];
        for (int64_t j = 0; j < n; ++j) {
            int w = (int)wround[i * n + j] - z[i];
            float u;
            int mm, sh;
            if (!u_element(i, j, n, r, wround, z, s, rstar, A, B, &u)) {
                mm = 0;
                sh = 255;
            } else {
                float v = u / sbar;
                if (v == 0.0f) {
                    mm = 0;
                    sh = smax;
                } else {
                    int k = ora_log2_round(fabsf(v));
                    sh = -k;
                    if (sh < 0) sh = 0;
                    if (sh > smax) sh = smax;
                    int sg = (v > 0.0f) ? 1 : -1;
                    int fl = (int)floor((double)w / ldexp(1.0, sh));
                    mm = sg * fl;
                }
            }
            if (mm > mhi) { mm = mhi; ++sat_total; }
            if (mm < mlo) { mm = mlo; ++sat_total; }
            m_out[i * n + j] = (int8_t)mm;
            if (shift_out) shift_out[i * n + j] = (uint8_t)sh;
        }
    }
    return sat_total;
}

/* ------------------------------------------------------------------------- */
/* Per-token symmetric int8 activation quantization (the activations stay     */
/* conventionally quantized; 8-bit setting uses per-token dynamic scales):    */
/*   s_x = max_j |x_tj| / 127 (1 for an all-zero token);                       */
/*   X_q = clamp(rint(x / s_x), -127, 127);  rowsum = sum_j X_q.               */
/* ------------------------------------------------------------------------- */
ORA_API void ora_quant_act(int64_t M, int64_t n, const float* X, int8_t* xq_out, float* sx_out, int32_t* rowsum_out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < M; ++t) {
        float amax = 0.0f;
        for (int64_t j = 0; j < n; ++j) {
            float a = fabsf(X[t * n + j]);
            if (a > amax) amax = a;
        }
        float sx = amax / 127.0f;
        if (!(sx > 0.0f)) sx = 1.0f;
        sx_out[t] = sx;
        int32_t sum = 0;
        for (int64_t j = 0; j < n; ++j) {
            float qv = rintf(X[t * n + j] / sx);
            if (qv > 127.0f) qv = 127.0f;
            if (qv < -127.0f) qv = -127.0f;
            xq_out[t * n + j] = (int8_t)qv;
            sum += (int32_t)qv;
        }
        rowsum_out[t] = sum;
    }
}

/* ------------------------------------------------------------------------- */
/* Integer linear layer on the merged integers, Y = X_q . m^T, dequantized.   */
/*   exact = sum_j X_q[t,j] * m[i,j]  (integer, no overflow in int64);         */
/*   y = RN32(RN32(float(exact) * s_x[t]) * s_bar[i]);  Y = bf16 RNE of y.     */
/* m is given as int32 values (int16 MUL or int8/int4 SHIFT merged integers).  */
/* ------------------------------------------------------------------------- */
static uint16_t bf16_rne(float y) {
    uint32_t b;
    memcpy(&b, &y, 4);
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7FFFu + lsb;
    return (uint16_t)(b >> 16);
}

ORA_API uint16_t ora_bf16_rne(float y) { return bf16_rne(y); }

static float dequant(int64_t exact, float sx, float sbar) {
    float y = (float)exact;
    y = y * sx;
    y = y * sbar;
    return y;
}

ORA_API void ora_linear(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx, const int32_t* m,
                        const float* sbar, int64_t* exact_out, float* y32_out, uint16_t* y_out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < M; ++t) {
        for (int64_t i = 0; i < d; ++i) {
            int64_t acc = 0;
            for (int64_t j = 0; j < n; ++j) acc += (int64_t)xq[t * n + j] * (int64_t)m[i * n + j];
            float y = dequant(acc, sx[t], sbar[i]);
            if (exact_out) exact_out[t * d + i] = acc;
            if (y32_out) y32_out[t * d + i] = y;
            y_out[t * d + i] = bf16_rne(y);
        }
    }
}

/* The same, for a list of (t, i) output positions only (full-size sampling). */
ORA_API void ora_linear_sampled(int64_t count, const int64_t* ts, const int64_t* is, int64_t n, const int8_t* xq,
                                const float* sx, const int32_t* m, const float* sbar, int64_t* exact_out,
                                uint16_t* y_out) {
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < count; ++p) {
        int64_t t = ts[p], i = is[p];
        int64_t acc = 0;
        for (int64_t j = 0; j < n; ++j) acc += (int64_t)xq[t * n + j] * (int64_t)m[i * n + j];
        exact_out[p] = acc;
        y_out[p] = bf16_rne(dequant(acc, sx[t], sbar[i]));
    }
}

ORA_API int ora_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the row / token loops from now on (the CPU-baseline timing runs the
 * oracle on one thread as well as on all host cores). */
ORA_API void ora_set_threads(int t) {
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}
