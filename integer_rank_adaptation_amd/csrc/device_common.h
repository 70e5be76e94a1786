// Device helpers shared by the IntLoRA kernels (gfx950, wave64).
//
// Every floating-point step that decides an integer code is a single IEEE binary32
// operation with round-to-nearest-even; the library is compiled with
// -ffp-contract=off so that no multiply-add is fused behind our back, and fused
// multiply-adds appear only where written as fmaf().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace intlora {

constexpr int kWave = 64;

// --------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64
// multiplies; the high halves are XORed with the other two counter words and the
// round key; the key advances by the two Weyl constants between rounds.
// --------------------------------------------------------------------------------
struct U4 {
  uint32_t x, y, z, w;
};

// a ^ b ^ k in one instruction: v_bitop3_b32 with truth table 0x96 (three-input
// parity), which the compiler does not form by itself here; k is a round key, uniform
// over the wave.
__device__ __forceinline__ uint32_t xor3_key(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  __asm__("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    U4 n;
    n.x = xor3_key((uint32_t)(p1 >> 32), c.y, k0);
    n.y = (uint32_t)p1;
    n.z = xor3_key((uint32_t)(p0 >> 32), c.w, k1);
    n.w = (uint32_t)p0;
    c = n;
  }
  return c;
}

// Counter block of linear element index q (q >> 2), layer id in word 2; the element
// uses output word q & 3.  Key = (seed low, seed high).
__device__ __forceinline__ U4 philox_block(uint64_t q4, uint32_t layer_id, uint64_t seed) {
  U4 c{(uint32_t)q4, (uint32_t)(q4 >> 32), layer_id, 0u};
  return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t pick_word(const U4& v, unsigned idx) {
  return idx == 0 ? v.x : idx == 1 ? v.y : idx == 2 ? v.z : v.w;
}

// --------------------------------------------------------------------------------
// Natural logarithm of g = G * 2^-23 (G odd, 1 <= G < 2^23) rounded to binary32.
// Evaluated in binary64: g = m * 2^e with m in [0.75, 1.5); ln m = -ln(r_k) +
// log1p(m r_k - 1) with a 96-entry table (r_k short enough that m r_k is exact) and
// a degree-7 series for log1p on |f| <= 2^-7.  The binary64 result is within a few
// units of 2^-53 relative of ln g, far inside the distance of every ln g on this
// domain from a binary32 rounding midpoint, so the final conversion gives RN32(ln g).
// --------------------------------------------------------------------------------
struct LnEntry {  // as stored (generated table)
  double neg_ln_r_hi;
  float neg_ln_r_lo;
  float r;
};

struct __attribute__((aligned(16))) LnLds {  // as used, in LDS: 16 bytes, one ds_read_b128;
  double hi;                                 // r pre-scaled by 2^-24 (exact in binary32)
  float lo, r24;
};

__device__ __forceinline__ LnLds ln_lds_entry(const LnEntry& e) {
  return LnLds{e.neg_ln_r_hi, e.neg_ln_r_lo, e.r * 0x1p-24f};
}

// The integer part of the logarithm below: g = (F 2^-24) 2^e with F 2^-24 in
// [0.75, 1.5), and the table entry k of F.
struct LnPrep {
  uint32_t F;
  int e;
  int k;
};

__device__ __forceinline__ LnPrep ln_prep(uint32_t G, int bias) {
  // leading-bit position p (0..22); m24 = G << (23 - p) in [2^23, 2^24)
  const int p = 31 - __clz(G);
  const uint32_t m24 = G << (23 - p);
  LnPrep r;
  r.e = p - bias;                  // g = (m24 * 2^-23) * 2^e
  if (m24 >= 0xC00000u) {          // m >= 1.5: halve
    r.F = m24;                     // (m/2) * 2^24 = m24
    r.e += 1;
  } else {
    r.F = m24 << 1;
  }
  r.k = (int)((r.F - 0xC00000u) >> 17);
  return r;
}

// ln(G 2^-bias) for odd G < 2^bias, bias 23 or 24, as the binary64 value before the
// final rounding (the Gaussian sampler takes its logarithm at bias 24), from its
// integer part and table entry t = tab[P.k].
template <bool ESTRIN = true>
__device__ __forceinline__ double ln_finish(const LnPrep& P, const LnLds& t) {
  const uint32_t F = P.F;
  const int e = P.e;
  const double f = fma((double)F, (double)t.r24, -1.0);  // m r_k - 1, exact
  // log1p(f) = f - f^2/2 + ... - f^8/8 truncated after f^7: |f| <= 2^-7 leaves a
  // relative error below 2^-52, far under the 2^-47.6 the rounding needs.  The
  // polynomial p(f) = -1/2 + f/3 - f^2/4 + ... + f^5/7 in log1p(f) = f + f^2 p(f) is
  // evaluated in Estrin's pairs (three dependent steps instead of Horner's five: in
  // the adaptation kernel the chain, not the operation count, sets the pace), or by
  // Horner's rule where registers are short (the Gaussian sampler); either way its
  // rounding errors are scaled by f^2 <= 2^-14 in the result.
  const double f2 = f * f;
  double p7;
  if (ESTRIN) {
    const double p01 = fma(1.0 / 3.0, f, -0.5);
    const double p23 = fma(1.0 / 5.0, f, -0.25);
    const double p45 = fma(1.0 / 7.0, f, -1.0 / 6.0);
    p7 = fma(f2, fma(f2, p45, p23), p01);
  } else {
    p7 = 1.0 / 7.0;
    p7 = fma(p7, f, -1.0 / 6.0);
    p7 = fma(p7, f, 1.0 / 5.0);
    p7 = fma(p7, f, -0.25);
    p7 = fma(p7, f, 1.0 / 3.0);
    p7 = fma(p7, f, -0.5);
  }
  const double lp = fma(f2, p7, f);
  // e*ln2 as a head with trailing zeros (exact product) plus a tail
  const double LN2_HI = 0x1.62e42fefa3800p-1;
  const double LN2_LO = 0x1.ef35793c76730p-45;
  const double ed = (double)e;
  const double head = fma(ed, LN2_HI, t.hi);
  const double tail = fma(ed, LN2_LO, (double)t.lo);
  return head + (lp + tail);
}

template <bool ESTRIN = true>
__device__ __forceinline__ double ln_odd_d(uint32_t G, int bias, const LnLds* __restrict__ tab) {
  const LnPrep P = ln_prep(G, bias);
  return ln_finish<ESTRIN>(P, tab[P.k]);
}

__device__ __forceinline__ float ln_odd_g(uint32_t G, const LnLds* __restrict__ tab) {
  return (float)ln_odd_d(G, 23, tab);
}

// Laplace(0, 1) sample from one word: u = (2 floor(x / 2^9) + 1) 2^-24, v = u - 1/2,
// g = 1 - 2|v|, L = -sign(v) ln g.  Computed on integers: N = 2a + 1 - 2^23 is the odd
// numerator of v (in units of 2^-24), G = 2^23 - |N| the odd numerator of g.
__device__ __forceinline__ float laplace_from_word(uint32_t x, const LnLds* __restrict__ tab) {
  const int32_t a = (int32_t)(x >> 9);
  const int32_t N = 2 * a + 1 - (1 << 23);
  const uint32_t G = (uint32_t)((1 << 23) - (N < 0 ? -N : N));
  const float lg = ln_odd_g(G, tab);
  return (N < 0) ? lg : -lg;
}

// The Laplace samples of the four words of a Philox block, the same values as
// laplace_from_word on each: the integer steps of all four come first, then their four
// table reads (in flight together), then the four binary64 evaluations.
__device__ __forceinline__ void laplace4(const U4& rnd, const LnLds* __restrict__ tab, float (&L)[4]) {
  const uint32_t x[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
  LnPrep P[4];
  bool neg[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int32_t N = 2 * (int32_t)(x[e] >> 9) + 1 - (1 << 23);
    neg[e] = N < 0;
    P[e] = ln_prep((uint32_t)((1 << 23) - (N < 0 ? -N : N)), 23);
  }
  LnLds t[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) t[e] = tab[P[e].k];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lg = (float)ln_finish(P[e], t[e]);
    L[e] = neg[e] ? lg : -lg;
  }
}

// --------------------------------------------------------------------------------
// Other auxiliary-matrix distributions (the ablation that swaps Laplace for a Gaussian,
// a Cauchy or a Student-t sample).  Every one is built from the same uniform as the
// Laplace sampler, u = (2 floor(x / 2^9) + 1) 2^-24, and every transcendental step is
// rounded once from a binary64 value accurate to a few units of 2^-53; exhaustive
// device checks over each input domain show that each rounding is the correct one.
// --------------------------------------------------------------------------------
enum { kAuxLaplace = 0, kAuxGauss = 1, kAuxCauchy = 2, kAuxStudentT2 = 3 };

// sin(pi x) and cos(pi x) for 0 <= x <= 1/4: Taylor polynomials in y = pi x (the
// first omitted terms are below 2^-53 of the result on this interval).
__device__ __forceinline__ double sinpi_q(double x) {
  const double y = x * 3.141592653589793, y2 = y * y;
  double p = -1.0 / 1307674368000.0;  // -1/15!
  p = fma(p, y2, 1.0 / 6227020800.0);
  p = fma(p, y2, -1.0 / 39916800.0);
  p = fma(p, y2, 1.0 / 362880.0);
  p = fma(p, y2, -1.0 / 5040.0);
  p = fma(p, y2, 1.0 / 120.0);
  p = fma(p, y2, -1.0 / 6.0);
  return fma(y * y2, p, y);
}
__device__ __forceinline__ double cospi_q(double x) {
  const double y = x * 3.141592653589793, y2 = y * y;
  double p = 1.0 / 20922789888000.0;  // 1/16!
  p = fma(p, y2, -1.0 / 87178291200.0);
  p = fma(p, y2, 1.0 / 479001600.0);
  p = fma(p, y2, -1.0 / 3628800.0);
  p = fma(p, y2, 1.0 / 40320.0);
  p = fma(p, y2, -1.0 / 720.0);
  p = fma(p, y2, 1.0 / 24.0);
  p = fma(p, y2, -0.5);
  return fma(y2, p, 1.0);
}
// cos(pi v) and sin(pi v) for 0 < v < 2 with at most 24 significant bits: the
// reductions (2 - v, 1 - a, 1/2 - a) are exact.
__device__ __forceinline__ double cospi_v(double v) {
  double a = v > 1.0 ? 2.0 - v : v;
  const bool neg = a > 0.5;
  if (neg) a = 1.0 - a;
  const double r = a <= 0.25 ? cospi_q(a) : sinpi_q(0.5 - a);
  return neg ? -r : r;
}
__device__ __forceinline__ double sinpi_v(double v) {
  const bool neg = v > 1.0;
  double a = neg ? v - 1.0 : v;
  if (a > 0.5) a = 1.0 - a;
  const double r = a <= 0.25 ? sinpi_q(a) : cospi_q(0.5 - a);
  return neg ? -r : r;
}
// tan(pi v) for |v| < 1/2 (exact reduction to [0, 1/4] through cot(pi (1/2 - a))).
__device__ __forceinline__ double tanpi_h(double v) {
  const double a = fabs(v);
  const double r = a <= 0.25 ? sinpi_q(a) / cospi_q(a) : cospi_q(0.5 - a) / sinpi_q(0.5 - a);
  return v < 0.0 ? -r : r;
}

// Element e (0..3) of a Philox block under distribution DIST.
//  Gaussian: Box-Muller over the word pairs (0, 1) and (2, 3); u1 from the first word
//    of the pair and u2 from the second; element 2p gets S cos(2 pi u2), element 2p + 1
//    S sin(2 pi u2), S = sqrt(-2 L), L = RN32(ln u1); each step rounded to binary32.
//  Cauchy: tan(pi (u - 1/2)).
//  Student-t with 2 degrees of freedom: its inverse distribution function,
//    (2u - 1) / sqrt(2u(1 - u)) = 2N / sqrt(2^47 - 2N^2) with u - 1/2 = N 2^-24.
template <int DIST>
__device__ __forceinline__ float aux_sample(const U4& rnd, unsigned e, const LnLds* __restrict__ tab) {
  if (DIST == kAuxLaplace) return laplace_from_word(pick_word(rnd, e), tab);
  if (DIST == kAuxGauss) {
    const uint32_t w1 = pick_word(rnd, e & 2u), w2 = pick_word(rnd, (e & 2u) | 1u);
    const float L = (float)ln_odd_d<false>(2u * (w1 >> 9) + 1u, 24, tab);
    const float S = sqrtf(-2.0f * L);
    const double v = (double)(2u * (w2 >> 9) + 1u) * 0x1p-23;  // 2 u2, exact
    const float C = (float)((e & 1u) ? sinpi_v(v) : cospi_v(v));
    return S * C;
  }
  const int32_t N = 2 * (int32_t)(pick_word(rnd, e) >> 9) + 1 - (1 << 23);  // u - 1/2 = N 2^-24
  if (DIST == kAuxCauchy) return (float)tanpi_h((double)N * 0x1p-24);
  const int64_t D = ((int64_t)1 << 47) - 2 * (int64_t)N * (int64_t)N;  // exact, 2^25 - 2 <= D < 2^47
  return (float)(2.0 * (double)N / sqrt((double)D));
}

__device__ __forceinline__ float aux_sample_rt(int dist, const U4& rnd, unsigned e, const LnLds* __restrict__ tab) {
  switch (dist) {
    case kAuxGauss: return aux_sample<kAuxGauss>(rnd, e, tab);
    case kAuxCauchy: return aux_sample<kAuxCauchy>(rnd, e, tab);
    case kAuxStudentT2: return aux_sample<kAuxStudentT2>(rnd, e, tab);
    default: return aux_sample<kAuxLaplace>(rnd, e, tab);
  }
}

// --------------------------------------------------------------------------------
// Wave reductions (64 lanes) with shuffles; exact for min / max / integer sums.
// --------------------------------------------------------------------------------
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Order key of a binary32: a signed integer whose order is the IEEE total order of
// the floats (-0 < +0), so that min / max reductions are exact integer operations.
__device__ __forceinline__ int f32_key(float v) {
  const int b = __float_as_int(v);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_f32(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }
// Minimum / maximum over the 64 lanes: DPP row shifts (1, 2, 4, 8) reduce each row of
// 16 lanes into its lane 15, two row broadcasts fold the rows into lane 63, whose
// value is returned to every lane.
__device__ __forceinline__ int wave_min_i32(int v) {
  constexpr int I = 0x7FFFFFFF;
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  constexpr int I = (int)0x80000000;
  v = max(v, __builtin_amdgcn_update_dpp(I, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(I, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(I, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(I, v, 0x118, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(I, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(I, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// binary32 -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t bf16_rne(float y) {
  uint32_t b = __float_as_uint(y);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// round(log2 |v|) for a nonzero binary32, exactly, from the bits: the unbiased
// exponent plus one when the significand is at or above sqrt(2) (field >= 0x3504F4;
// sqrt(2) is irrational, so there are no ties).  Subnormals are normalized first.
__device__ __forceinline__ int log2_round_bits(float v) {
  uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
  int ex = (int)(b >> 23);
  uint32_t frac = b & 0x7FFFFFu;
  if (ex == 0) {  // subnormal: shift the leading one up to bit 23
    const int lz = __clz(frac) - 8;  // frac != 0 here
    frac = (frac << lz) & 0x7FFFFFu;
    ex = 1 - lz;
  }
  return ex - 127 + (frac >= 0x3504F4u ? 1 : 0);
}

}  // namespace intlora
