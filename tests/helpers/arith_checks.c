/*
 * arith_checks.c -- test helper (CPU): binary32 emulations of the arithmetic the GPU
 * kernels substitute for an IEEE division, checked against the division itself, and
 * a plain fmaf chain for the matrix-core product pins.
 *
 * Built by the tests with gcc -O2 -ffp-contract=off (every operation below is the
 * IEEE binary32 operation written; fmaf is the correctly rounded fused multiply-add).
 * It shares nothing with the library or the oracle: each substitution is restated here
 * from its definition.
 *
 * (1) Division by a small integer (the MLA term's (R* + AB) / (W_round - z), IntLoRA
 *     notes, "2. MLA"): for an integer 1 <= |w| <= 255 and y = RN(1/w),
 *         q0 = RN(t y),  r = fma(-q0, w, t),  q = fma(r, y, q0)
 *     is claimed to equal RN(t / w) for every binary32 t with 2^-100 <= |t| <= 2^100.
 * (2) The MUL quantizer's code (IntLoRA notes, "two implementation variants", MUL):
 *     with rs = RN(1/s) a normal number, qt = RN(u rs) is claimed to round (rint, half
 *     to even) to the same integer as RN(u / s) whenever |qt| < 512 and qt lies more
 *     than 2^-11 from every half-integer, tested as |qt - rint(qt)| < 1/2 - 2^-11.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float from_bits(uint32_t b) {
    float f;
    memcpy(&f, &b, 4);
    return f;
}

static uint32_t to_bits(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    return b;
}

static float div_small_int(float t, float wf, float y) {
    const float q0 = t * y;
    const float r = fmaf(-q0, wf, t);
    return fmaf(r, y, q0);
}

/* Every w in [w_lo, w_hi] \ {0}, every biased exponent in [eb_lo, eb_hi], both signs,
 * every significand m with m % stride == phase: the number of t where the emulation
 * differs from t / w in any bit.  *checked receives the number of quotients compared. */
int64_t count_div_mismatches(int w_lo, int w_hi, int eb_lo, int eb_hi, uint32_t stride, uint32_t phase,
                             int64_t* checked) {
    int64_t bad = 0, cnt = 0;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad, cnt) collapse(2)
    for (int w = w_lo; w <= w_hi; ++w) {
        for (int eb = eb_lo; eb <= eb_hi; ++eb) {
            if (w == 0) continue;
            const float wf = (float)w;
            const float y = 1.0f / wf;
            for (uint32_t m = phase; m < (1u << 23); m += stride) {
                for (uint32_t sg = 0; sg < 2; ++sg) {
                    const float t = from_bits((sg << 31) | ((uint32_t)eb << 23) | m);
                    const float q = div_small_int(t, wf, y);
                    const float ref = t / wf;
                    bad += to_bits(q) != to_bits(ref);
                    ++cnt;
                }
            }
        }
    }
    *checked = cnt;
    return bad;
}

/* The exact power of two 2^e as a binary32 t (and -t): mismatches of the emulation. */
int64_t count_div_mismatches_pow2(int e) {
    int64_t bad = 0;
    for (int w = -255; w <= 255; ++w) {
        if (w == 0) continue;
        const float wf = (float)w, y = 1.0f / wf;
        for (int sg = 0; sg < 2; ++sg) {
            const float t = sg ? -ldexpf(1.0f, e) : ldexpf(1.0f, e);
            bad += to_bits(div_small_int(t, wf, y)) != to_bits(t / wf);
        }
    }
    return bad;
}

/* (2) For each scale s[k] (k < ns) and every half-integer h = c + 1/2 with
 * -256 <= c <= 255, every u within `span` ulps of RN(h s): where the fast rule says
 * "exact", compare its integer with rint(RN(u / s)).  Returns the mismatches;
 * *fast receives how often the rule applied and *total how many u were tried. */
int64_t count_code_mismatches(int64_t ns, const float* s, int span, int64_t* fast, int64_t* total) {
    int64_t bad = 0, nf = 0, nt = 0;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad, nf, nt)
    for (int64_t k = 0; k < ns; ++k) {
        const float sb = s[k];
        const float rs = 1.0f / sb;
        if (!(fabsf(rs) >= 0x1p-126f) || isinf(rs)) continue;  /* the rule needs a normal reciprocal */
        for (int c = -256; c <= 255; ++c) {
            const float centre = ((float)c + 0.5f) * sb;
            const uint32_t cb = to_bits(centre);
            for (int dlt = -span; dlt <= span; ++dlt) {
                const float u = from_bits((uint32_t)((int64_t)cb + dlt));
                if (!isfinite(u)) continue;
                const float qt = u * rs;
                const int ok = fabsf(qt) < 512.0f && fabsf(qt - rintf(qt)) < 0.5f - 0x1p-11f;
                ++nt;
                if (!ok) continue;
                ++nf;
                const float qd = u / sb;
                bad += rintf(qt) != rintf(qd);
            }
        }
    }
    *fast = nf;
    *total = nt;
    return bad;
}

/* Random u in the range the quantizer sees (|u / s| <= 2^bits - 1) for each scale:
 * the same comparison on `per` values per scale drawn from a counter-based hash. */
static uint32_t mix32(uint64_t x) {
    x ^= x >> 33;
    x *= 0xff51afd7ed558ccdull;
    x ^= x >> 33;
    x *= 0xc4ceb9fe1a85ec53ull;
    x ^= x >> 33;
    return (uint32_t)x;
}

int64_t count_code_mismatches_random(int64_t ns, const float* s, int bits, int64_t per, int64_t* fast) {
    int64_t bad = 0, nf = 0;
    const float qmax = (float)((1 << bits) - 1);
#pragma omp parallel for schedule(dynamic) reduction(+ : bad, nf)
    for (int64_t k = 0; k < ns; ++k) {
        const float sb = s[k];
        const float rs = 1.0f / sb;
        if (!(fabsf(rs) >= 0x1p-126f) || isinf(rs)) continue;
        for (int64_t t = 0; t < per; ++t) {
            const uint32_t h = mix32(((uint64_t)k << 32) ^ (uint64_t)t);
            const float x = ((float)(h >> 8) * 0x1p-24f * 2.0f - 1.0f) * qmax;  /* in [-qmax, qmax) */
            const float u = x * sb;
            const float qt = u * rs;
            if (!(fabsf(qt) < 512.0f && fabsf(qt - rintf(qt)) < 0.5f - 0x1p-11f)) continue;
            ++nf;
            bad += rintf(qt) != rintf(u / sb);
        }
    }
    *fast = nf;
    return bad;
}

/* acc[i][j] = the fmaf chain of A[i][k] B[k][j] over k = 0..r-1 from +0 (d x r, r x n,
 * row-major). */
void fmaf_chain(int64_t d, int64_t n, int r, const float* A, const float* B, float* acc) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d; ++i)
        for (int64_t j = 0; j < n; ++j) {
            float a = 0.0f;
            for (int k = 0; k < r; ++k) a = fmaf(A[i * r + k], B[(int64_t)k * n + j], a);
            acc[i * n + j] = a;
        }
}
