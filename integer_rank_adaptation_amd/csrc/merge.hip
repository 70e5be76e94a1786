// IntLoRA merge kernels for gfx950: R* generation, per-channel statistics, the MLA
// adaptation term, and the MUL / SHIFT integer merges.
//
// Method ("IntLoRA: Integral Low-rank Adaptation of Quantized Diffusion Models",
// Paper-Notes ICML 2025):
//   AQS   W' = Q[W - sg(R)] + sg(R) + AB, R regenerated from a seed (no storage)
//   MLA   W' = [s I + (R + AB) / (W_round - z)] (.) (W_round - z)
//   VMC   R* = r^alpha R, r = sigma_W / sigma_R
//   MUL   W' = s_bar (U_round - z_bar) (.) (W_round - z)
//   SHIFT W' = sign(V) (.) [(W_round - z) >> shift]
// The merge runs as two kernels per layer:
//   adapt:     R* in registers (Philox -> Laplace -> x c_i), U = s + (R* + AB) / w
//              written to the workspace, per-tile row min / max over valid elements;
//   quantize:  row statistics from the tile partials, then the MUL or SHIFT code
//              and merged integer per element (HBM-bound: U + W_round in, m out).
#include "device_common.h"
#include "intlora_internal.h"

namespace intlora {

__device__ const LnEntry kLnTable[96] = {
#include "ln_table.inc"
};

__device__ __forceinline__ void load_ln_table(LnLds* dst) {
  for (int t = threadIdx.x; t < 96; t += blockDim.x) dst[t] = ln_lds_entry(kLnTable[t]);
}

// R*_ij for one element (general path).
__device__ __forceinline__ float rstar_element(uint64_t q, float ci, uint32_t layer_id, uint64_t seed,
                                               const LnLds* tab, int dist) {
  const U4 blk = philox_block(q >> 2, layer_id, seed);
  return ci * aux_sample_rt(dist, blk, (unsigned)(q & 3), tab);
}

// ---------------------------------------------------------------------------------
// K1: R*_ij = c_i * Laplace(Philox(seed, layer, i*n + j)) (or another distribution of
// the sampler ablation); one thread per counter block of four consecutive linear
// elements.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gen_r(int64_t d, int64_t n, uint64_t seed, uint32_t layer_id,
                                              const float* __restrict__ c, float* __restrict__ out, int dist) {
  __shared__ LnLds tab[96];
  load_ln_table(tab);
  __syncthreads();
  const uint64_t total = (uint64_t)d * (uint64_t)n;
  const uint64_t nblk = (total + 3) >> 2;
  for (uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
       b += (uint64_t)gridDim.x * blockDim.x) {
    const U4 v = philox_block(b, layer_id, seed);
    const uint64_t q0 = b << 2;
    uint64_t i = q0 / (uint64_t)n;
    uint64_t j = q0 - i * (uint64_t)n;
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (q0 + e < total) {
        r[e] = c[i] * aux_sample_rt(dist, v, (unsigned)e, tab);
      }
      if (++j == (uint64_t)n) {
        j = 0;
        ++i;
      }
    }
    if (q0 + 3 < total && ((reinterpret_cast<uintptr_t>(out) & 15) == 0)) {
      *reinterpret_cast<float4*>(out + q0) = make_float4(r[0], r[1], r[2], r[3]);
    } else {
      for (int e = 0; e < 4; ++e)
        if (q0 + e < total) out[q0 + e] = r[e];
    }
  }
}

// Debug: binary32 natural log on odd multiples of 2^-23 (input G, output ln(G 2^-23)).
__global__ __launch_bounds__(256) void k_ln_odd(int64_t count, const uint32_t* __restrict__ G,
                                               float* __restrict__ out) {
  __shared__ LnLds tab[96];
  load_ln_table(tab);
  __syncthreads();
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < count; t += (int64_t)gridDim.x * blockDim.x)
    out[t] = ln_odd_g(G[t], tab);
}

// ---------------------------------------------------------------------------------
// Block reductions for 256-thread blocks.
// ---------------------------------------------------------------------------------
template <typename T, typename Op>
__device__ __forceinline__ T block_reduce_256(T v, T* scratch /*[4]*/, Op op) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  T r = scratch[0];
  r = op(r, scratch[1]);
  r = op(r, scratch[2]);
  r = op(r, scratch[3]);
  return r;
}

// ---------------------------------------------------------------------------------
// sigma_W: population standard deviation of each row of W (binary64 accumulation,
// two passes: mean, then mean squared deviation), rounded to binary32.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sigma_w(int64_t n, const float* __restrict__ W,
                                                float* __restrict__ sigma) {
  __shared__ double red[4];
  const float* row = W + (int64_t)blockIdx.x * n;
  double acc = 0.0;
  for (int64_t j = threadIdx.x; j < n; j += 256) acc += (double)row[j];
  const double mean = block_reduce_256(acc, red, [](double a, double b) { return a + b; }) / (double)n;
  double ss = 0.0;
  for (int64_t j = threadIdx.x; j < n; j += 256) {
    const double e = (double)row[j] - mean;
    ss += e * e;
  }
  const double tot = block_reduce_256(ss, red, [](double a, double b) { return a + b; });
  if (threadIdx.x == 0) sigma[blockIdx.x] = (float)sqrt(tot / (double)n);
}

// VMC scale c_i = RN32((sigma_W,i / sqrt 2)^alpha) (sigma_R = sqrt 2 for unit Laplace).
// sigma_R = sqrt(2) for Laplace(0, 1); 1 (the standard deviation of the Gaussian, the
// scale of the Cauchy and Student-t samples) for the other distributions.
__global__ __launch_bounds__(256) void k_vmc_scale(int64_t d, const float* __restrict__ sigma, double alpha,
                                                  float* __restrict__ c, bool unit_sigma_r) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) c[i] = (float)pow(unit_sigma_r ? (double)sigma[i] : (double)sigma[i] / sqrt(2.0), alpha);
}

// ---------------------------------------------------------------------------------
// Base quantizer Q[W - R*] per output row (AQS set-up). One block per row; the row
// of x = W - R* is kept in LDS between the range pass and the code pass.
//   lo = min(0, min x), hi = max(0, max x), s = (hi - lo)/(2^b - 1) (1 if 0),
//   z = clamp(rint(-lo/s), 0, 2^b-1), W_round = clamp(rint(x/s) + z, 0, 2^b-1).
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_base_quant(int64_t n, int bits, uint64_t seed, uint32_t layer_id,
                                                   const float* __restrict__ W, const float* __restrict__ c,
                                                   uint8_t* __restrict__ wround, int32_t* __restrict__ z_out,
                                                   float* __restrict__ s_out, int dist) {
  extern __shared__ float xs[];  // n floats
  __shared__ LnLds tab[96];
  __shared__ float red[4];
  load_ln_table(tab);
  __syncthreads();
  const int64_t i = blockIdx.x;
  const float ci = c[i];
  float lo = 0.0f, hi = 0.0f;
  for (int64_t j = threadIdx.x; j < n; j += 256) {
    const float r = rstar_element((uint64_t)i * (uint64_t)n + (uint64_t)j, ci, layer_id, seed, tab, dist);
    const float x = W[i * n + j] - r;
    xs[j] = x;
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  }
  lo = block_reduce_256(lo, red, [](float a, float b) { return fminf(a, b); });
  hi = block_reduce_256(hi, red, [](float a, float b) { return fmaxf(a, b); });
  const int qmax = (1 << bits) - 1;
  float s = (hi - lo) / (float)qmax;
  if (!(s > 0.0f)) s = 1.0f;
  const float zf = rintf(-lo / s);
  const int z = zf < 0.0f ? 0 : (zf > (float)qmax ? qmax : (int)zf);
  if (threadIdx.x == 0) {
    s_out[i] = s;
    z_out[i] = z;
  }
  __syncthreads();
  auto code_of = [&](float x) -> int {
    float q = rintf(x / s);
    q = fminf(fmaxf(q, -1.0e6f), 1.0e6f);
    int v = (int)q + z;
    return v < 0 ? 0 : (v > qmax ? qmax : v);
  };
  if (bits == 8) {
    for (int64_t j = threadIdx.x; j < n; j += 256) wround[i * n + j] = (uint8_t)code_of(xs[j]);
  } else {  // 4-bit, two codes per byte, low nibble = even column
    const int64_t nb = n >> 1;
    for (int64_t jb = threadIdx.x; jb < nb; jb += 256) {
      const int a = code_of(xs[2 * jb]), b = code_of(xs[2 * jb + 1]);
      wround[i * nb + jb] = (uint8_t)(a | (b << 4));
    }
  }
}

// ---------------------------------------------------------------------------------
// Per-token symmetric int8 activation quantization: s_x = max|x| / 127 (1 if 0),
// X_q = clamp(rint(x / s_x), -127, 127), rowsum = sum X_q.  One block per token.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_act(int64_t n, const float* __restrict__ X, int8_t* __restrict__ xq,
                                                  float* __restrict__ sx_out, int32_t* __restrict__ rowsum) {
  __shared__ float redf[4];
  __shared__ int redi[4];
  const int64_t t = blockIdx.x;
  const float* row = X + t * n;
  float amax = 0.0f;
  for (int64_t j = threadIdx.x; j < n; j += 256) amax = fmaxf(amax, fabsf(row[j]));
  amax = block_reduce_256(amax, redf, [](float a, float b) { return fmaxf(a, b); });
  float sx = amax / 127.0f;
  if (!(sx > 0.0f)) sx = 1.0f;
  int sum = 0;
  for (int64_t j = threadIdx.x; j < n; j += 256) {
    float q = rintf(row[j] / sx);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    xq[t * n + j] = (int8_t)q;
    sum += (int)q;
  }
  sum = block_reduce_256(sum, redi, [](int a, int b) { return a + b; });
  if (threadIdx.x == 0) {
    sx_out[t] = sx;
    if (rowsum) rowsum[t] = sum;
  }
}

// ---------------------------------------------------------------------------------
// K2: adaptation term U and per-tile row range.  U is written for every element; the
// value at a w == 0 element is not specified (the quantize kernels never read it).
// ---------------------------------------------------------------------------------
constexpr int kAdaptCols = 1024;  // column-tile width of the general path

// Reciprocals RN32(1/w) of the signed pretrained integers w in [-255, 255] (0 for
// w = 0), for the division t / w below.
__device__ __forceinline__ void load_rcp_table(float* rcp) {
  for (int t = threadIdx.x; t < 511; t += blockDim.x) {
    const int w = t - 255;
    rcp[t] = w == 0 ? 0.0f : 1.0f / (float)w;
  }
}

// t / w, correctly rounded, for an integer 1 <= |w| <= 255 with y = RN32(1/w):
// q0 = RN(t y), r = t - q0 w (exact with a fused multiply-add), q = RN(q0 + r y).
// An exhaustive check over every binary32 significand of t and every such w shows
// q == RN(t / w); every step scales exactly with t's exponent, so this holds for all
// |t| in [2^-100, 2^100].  Outside that range (div_small_int_ok false) the caller
// uses the IEEE division.
__device__ __forceinline__ float div_small_int(float t, float wf, float y) {
  const float q0 = t * y;
  const float r = fmaf(-q0, wf, t);
  return fmaf(r, y, q0);
}
__device__ __forceinline__ bool div_small_int_ok(float t) {
  const float at = fabsf(t);
  return at >= 0x1p-100f && at <= 0x1p100f;
}
// Entry of w's reciprocal in the 511-entry table.  The index is clamped so that a zero
// point outside the code range (|w| > 255 is then possible) never reads past the table;
// rows with such a zero point (zero_point_ok false) take the IEEE division instead.
__device__ __forceinline__ int rcp_index(int w) { return min(max(w, -255), 255) + 255; }
__device__ __forceinline__ bool zero_point_ok(int z) { return (unsigned)z <= 255u; }

constexpr int kKeyPosInf = 0x7F800000;  // order key of +inf (identity of min)
constexpr int kKeyNegInf = (int)0x807FFFFF;  // order key of -inf (identity of max)

// ---------------------------------------------------------------------------------
// Adaptation with the rank-r product on the matrix cores.  v_mfma_f32_32x32x1f32
// adds one product per output per instruction as a fused multiply-add (one
// rounding), so a chain of r of them in k order reproduces the fmaf chain of the
// definition exactly.  The product is taken transposed (MFMA rows = columns j of U,
// MFMA columns = rows i), so each lane receives, per group of four accumulators,
// four consecutive columns of one row: one Philox block per group.  A wave covers
// 32 rows x 64 columns per row tile (two 32-column MFMA blocks over the same rows);
// a block of 4 waves covers 256 columns and `rtiles` row tiles, keeping its B
// columns in registers across them.
// ---------------------------------------------------------------------------------
typedef float v32f __attribute__((ext_vector_type(32)));
typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kMfmaCols = 256;
constexpr int kMfmaMaxRowTiles = 8;

// PTQ (the QLoRA-style comparison path): x = (s w + R*) + AB for every element instead
// of U, with no division and no excluded elements.
// Three waves per SIMD up to r = 32; at r = 64 the 64 B values per lane need the
// registers of two waves per SIMD (with three, every instantiation spilled, and the
// Laplace one ran 1-6 % slower on the Llama-shaped layers).
template <int R, bool W4, bool PTQ, int DIST>
__global__ __launch_bounds__(256, (R > 32 ? 2 : 3)) void k_adapt_mfma(int64_t d, int64_t n, uint64_t seed, uint32_t layer_id,
                                                    const uint8_t* __restrict__ wround, const int32_t* __restrict__ z,
                                                    const float* __restrict__ s, const float* __restrict__ c,
                                                    const float* __restrict__ A, const float* __restrict__ B,
                                                    float* __restrict__ U, int* __restrict__ pmin,
                                                    int* __restrict__ pmax, int ntiles, int rtiles, int64_t rb0,
                                                    unsigned long long* __restrict__ sat_zero, int64_t row0) {
  __shared__ LnLds tab[96];
  __shared__ float rcp[511];
  load_ln_table(tab);
  load_rcp_table(rcp);
  if (sat_zero && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *sat_zero = 0ull;
  __syncthreads();
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int64_t jw = (int64_t)blockIdx.x * kMfmaCols + wid * 64;  // the wave's first column
  // MFMA A operand: lane l holds B[k][jw + l] for every k
  float bcol[R];
  {
    const int64_t jl = jw + lane;
#pragma unroll
    for (int k = 0; k < R; ++k) bcol[k] = jl < n ? B[(int64_t)k * n + jl] : 0.0f;
  }
  for (int rt = 0; rt < rtiles; ++rt) {
    const int64_t i0 = ((rb0 + (int64_t)blockIdx.y) * rtiles + rt) * 32;
    if (i0 >= d) break;  // uniform over the block
    const int64_t i = i0 + li;
    const bool row_ok = i < d;
    // Every load of the tile is issued here, without branches (a row past d reads row
    // d - 1 and a group past n reads column 0; their results are never used), so the
    // loads are in flight together instead of each waiting behind a branch.
    const int64_t ic = row_ok ? i : d - 1;
    const int zi = z[ic];
    const bool zok = zero_point_ok(zi);
    const float ci = c[ic], si = s[ic];
    uint32_t wcode[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      int64_t jg = jw + 32 * (g >> 2) + 8 * (g & 3) + 4 * h;
      jg = jg < n ? jg : 0;
      if (W4)
        wcode[g] = *reinterpret_cast<const uint16_t*>(wround + ic * (n >> 1) + (jg >> 1));
      else
        wcode[g] = *reinterpret_cast<const uint32_t*>(wround + ic * n + jg);
    }
    // MFMA B operand: lane l holds A[i0 + l % 32][k], loaded 32 values at a time
    const float* Ai = A + ic * R;
    v32f acc;
#pragma unroll
    for (int r = 0; r < 32; ++r) acc[r] = 0.0f;
    constexpr int KC = R < 32 ? R : 32;
#pragma unroll
    for (int k0 = 0; k0 < R; k0 += KC) {
      float4 a4[KC / 4];
#pragma unroll
      for (int k = 0; k < KC / 4; ++k) a4[k] = *reinterpret_cast<const float4*>(Ai + k0 + 4 * k);
#pragma unroll
      for (int k = 0; k < KC / 4; ++k) {
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(bcol[k0 + 4 * k], a4[k].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(bcol[k0 + 4 * k + 1], a4[k].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(bcol[k0 + 4 * k + 2], a4[k].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(bcol[k0 + 4 * k + 3], a4[k].w, acc, 0, 0, 0);
      }
    }
    int kmin = kKeyPosInf, kmax = kKeyNegInf;
    if (row_ok) {
      const uint64_t qrow = (uint64_t)(i + row0) * (uint64_t)n;  // R's linear index of the row's column 0
      // reciprocal-table entry of w = code - zi is code + (255 - zc): exact when zi is in
      // [0, 255]; other rows take the IEEE division and only need an index in range
      const int rbase = 255 - min(max(zi, 0), 255);
      // The Gaussian and Cauchy samplers' longer chains do not fit the registers of
      // interleaved groups (they spilled): those laws keep one group at a time, with the
      // IEEE division behind a branch in each group.
      if constexpr (DIST == kAuxGauss || DIST == kAuxCauchy) {
        // accumulator group g = 4 blk + q: columns jw + 32 blk + 8 q + 4 h + 0..3
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const int64_t jg = jw + 32 * (g >> 2) + 8 * (g & 3) + 4 * h;
          if (jg >= n) continue;  // n % 4 == 0: a group is entirely inside or outside
          int code[4], w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            code[e] = W4 ? (int)((wcode[g] >> (4 * e)) & 15u) : (int)((wcode[g] >> (8 * e)) & 255u);
            w[e] = code[e] - zi;
          }
          float y[4];  // reciprocals of w, read first: the Philox rounds cover the LDS latency
          if (!PTQ) {
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = rcp[code[e] + rbase];
          }
          const U4 rnd = philox_block((qrow + (uint64_t)jg) >> 2, layer_id, seed);
          float rs[4];
          if (DIST == kAuxLaplace) {
            float L[4];
            laplace4(rnd, tab, L);
#pragma unroll
            for (int e = 0; e < 4; ++e) rs[e] = ci * L[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) rs[e] = ci * aux_sample<DIST>(rnd, (unsigned)e, tab);
          }
          float u[4], t[4], q[4];
          if (PTQ) {
#pragma unroll
            for (int e = 0; e < 4; ++e) q[e] = (si * (float)w[e] + rs[e]) + acc[4 * g + e];  // binary32, in this order
          } else {
            // the steps of div_small_int are exact for 2^-100 <= |t| < 2^100, i.e. biased
            // exponents 27 .. 226 (NaN and inf have 255); the group's extremes decide
            int emin = 255, emax = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              t[e] = rs[e] + acc[4 * g + e];
              q[e] = div_small_int(t[e], (float)w[e], y[e]);
              const int ex = (int)((__float_as_uint(t[e]) >> 23) & 0xFFu);
              emin = min(emin, ex);
              emax = max(emax, ex);
            }
            const bool slow = !zok || emin < 27 || emax > 226;
            // the IEEE division runs only in waves where some lane needs it
            if (__builtin_amdgcn_ballot_w64(slow) != 0) {
              __asm__ volatile("");  // keeps the branch: the division is not speculated
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (w[e] != 0 && (!zok || !div_small_int_ok(t[e]))) q[e] = t[e] / (float)w[e];
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool valid = PTQ || w[e] != 0;
            u[e] = PTQ ? q[e] : si + q[e];  // U of a w == 0 element is written but never read
            const int key = f32_key(u[e]);
            kmin = valid ? min(kmin, key) : kmin;
            kmax = valid ? max(kmax, key) : kmax;
          }
          *reinterpret_cast<float4*>(U + i * n + jg) = make_float4(u[0], u[1], u[2], u[3]);
        }
      } else {
        // The values u[e] of accumulator group g (g = 4 blk + q: columns jw + 32 blk + 8 q +
        // 4 h + 0..3, starting at jg) and whether each enters the row range.  The fast form
        // divides with div_small_int and returns true when the group is not certainly exact
        // (some t outside the window, or a zero point outside the code range): its values
        // are then excluded here and recomputed by the IEEE form after all groups.  With no
        // branch inside a group, the eight groups form one straight run that the compiler
        // interleaves (one group's Philox rounds and table reads beside another's ln).
        auto group = [&](int g, int64_t jg, auto ieee_tag, float (&u)[4], bool (&valid)[4]) -> bool {
          constexpr bool IEEE = decltype(ieee_tag)::value;
          int code[4], w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            code[e] = W4 ? (int)((wcode[g] >> (4 * e)) & 15u) : (int)((wcode[g] >> (8 * e)) & 255u);
            w[e] = code[e] - zi;
          }
          float y[4];  // reciprocals of w, read first: the Philox rounds cover the LDS latency
          if (!PTQ) {
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = rcp[code[e] + rbase];
          }
          const U4 rnd = philox_block((qrow + (uint64_t)jg) >> 2, layer_id, seed);
          float rs[4];
          if (DIST == kAuxLaplace) {
            float L[4];
            laplace4(rnd, tab, L);
#pragma unroll
            for (int e = 0; e < 4; ++e) rs[e] = ci * L[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) rs[e] = ci * aux_sample<DIST>(rnd, (unsigned)e, tab);
          }
          float q[4];
          bool slow = false;
          if (PTQ) {
#pragma unroll
            for (int e = 0; e < 4; ++e) q[e] = (si * (float)w[e] + rs[e]) + acc[4 * g + e];  // binary32, in this order
          } else {
            // the steps of div_small_int are exact for 2^-100 <= |t| < 2^100, i.e. biased
            // exponents 27 .. 226 (NaN and inf have 255); the group's extremes decide
            int emin = 255, emax = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float t = rs[e] + acc[4 * g + e];
              q[e] = div_small_int(t, (float)w[e], y[e]);
              if (IEEE && w[e] != 0 && (!zok || !div_small_int_ok(t))) q[e] = t / (float)w[e];
              const int ex = (int)((__float_as_uint(t) >> 23) & 0xFFu);
              emin = min(emin, ex);
              emax = max(emax, ex);
            }
            slow = !IEEE && (!zok || emin < 27 || emax > 226);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            valid[e] = PTQ || (w[e] != 0 && !slow);
            u[e] = PTQ ? q[e] : si + q[e];  // U of a w == 0 element is written but never read
          }
          return slow;
        };
        auto emit = [&](int64_t jg, const float (&u)[4], const bool (&valid)[4]) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = f32_key(u[e]);
            kmin = valid[e] ? min(kmin, key) : kmin;
            kmax = valid[e] ? max(kmax, key) : kmax;
          }
          *reinterpret_cast<float4*>(U + i * n + jg) = make_float4(u[0], u[1], u[2], u[3]);
        };
        uint32_t slow_groups = 0;
        auto fast = [&](auto whole_tag) {
          constexpr bool WHOLE = decltype(whole_tag)::value;  // the wave's 64 columns lie inside n
#pragma unroll
          for (int g = 0; g < 8; ++g) {
            const int64_t jg = jw + 32 * (g >> 2) + 8 * (g & 3) + 4 * h;
            if (!WHOLE && jg >= n) continue;  // n % 4 == 0: a group is entirely inside or outside
            float u[4];
            bool valid[4];
            const bool slow = group(g, jg, std::false_type{}, u, valid);
            slow_groups |= (uint32_t)slow << g;
            emit(jg, u, valid);
          }
        };
        if (jw + 64 <= n)
          fast(std::true_type{});
        else
          fast(std::false_type{});
        // the IEEE division runs only in waves where some lane needs it; its stores replace
        // the fast ones (same thread, later in program order)
        if (!PTQ && __builtin_amdgcn_ballot_w64(slow_groups != 0) != 0) {
          __asm__ volatile("");  // keeps the branch: the division is not speculated
#pragma unroll
          for (int g = 0; g < 8; ++g) {
            if (((slow_groups >> g) & 1u) == 0) continue;
            const int64_t jg = jw + 32 * (g >> 2) + 8 * (g & 3) + 4 * h;
            float u[4];
            bool valid[4];
            group(g, jg, std::true_type{}, u, valid);
            emit(jg, u, valid);
          }
        }
      }
    }
    // lanes l and l ^ 32 hold the same row; each wave writes the partial of its own 64
    // columns (partial column 4 blockIdx.x + wid), so the waves never wait for each other
    kmin = min(kmin, __shfl_xor(kmin, 32, kWave));
    kmax = max(kmax, __shfl_xor(kmax, 32, kWave));
    if (h == 0 && row_ok) {
      const int64_t col = (int64_t)blockIdx.x * 4 + wid;
      pmin[col * d + i] = kmin;
      pmax[col * d + i] = kmax;
    }
  }
}

// K2 (general path): any n, any r <= kMaxRank.  One thread per element; the same
// arithmetic as the fast path.  Tile partials over kAdaptCols columns.
__global__ __launch_bounds__(256) void k_adapt_generic(int64_t d, int64_t n, int r, int w_bits, uint64_t seed,
                                                      uint32_t layer_id, const uint8_t* __restrict__ wround,
                                                      const int32_t* __restrict__ z, const float* __restrict__ s,
                                                      const float* __restrict__ c, const float* __restrict__ A,
                                                      const float* __restrict__ B, float* __restrict__ U,
                                                      int* __restrict__ pmin, int* __restrict__ pmax, int ntiles,
                                                      unsigned long long* __restrict__ sat_zero, bool ptq, int dist,
                                                      int64_t row0) {
  __shared__ LnLds tab[96];
  __shared__ int smin[4], smax[4];
  load_ln_table(tab);
  if (sat_zero && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *sat_zero = 0ull;
  __syncthreads();
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int64_t i = blockIdx.y; i < d; i += gridDim.y) {
  int kmin = kKeyPosInf, kmax = kKeyNegInf;
  const int64_t jt = (int64_t)blockIdx.x * kAdaptCols;
  for (int64_t j = jt + threadIdx.x; j < jt + kAdaptCols && j < n; j += 256) {
    int code;
    if (w_bits == 4) {
      const uint8_t byte = wround[i * ((n + 1) >> 1) + (j >> 1)];
      code = (j & 1) ? (byte >> 4) : (byte & 15);
    } else {
      code = wround[i * n + j];
    }
    const int w = code - z[i];
    float acc = 0.0f;
    for (int k = 0; k < r; ++k) acc = fmaf(A[i * r + k], B[(int64_t)k * n + j], acc);
    const float rs = rstar_element((uint64_t)(i + row0) * (uint64_t)n + (uint64_t)j, c[i], layer_id, seed, tab, dist);
    const float t = rs + acc;
    const bool valid = ptq || w != 0;
    const float q = t / (float)(w != 0 ? w : 1);
    const float uu = ptq ? (s[i] * (float)w + rs) + acc : s[i] + q;
    U[i * n + j] = valid ? uu : 0.0f;
    if (valid) {
      kmin = min(kmin, f32_key(uu));
      kmax = max(kmax, f32_key(uu));
    }
  }
  kmin = wave_min_i32(kmin);
  kmax = wave_max_i32(kmax);
  if (lane == 0) {
    smin[wid] = kmin;
    smax[wid] = kmax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    pmin[(int64_t)blockIdx.x * d + i] = min(min(smin[0], smin[1]), min(smin[2], smin[3]));
    pmax[(int64_t)blockIdx.x * d + i] = max(max(smax[0], smax[1]), max(smax[2], smax[3]));
  }
  __syncthreads();  // smin / smax are reused by the next row
  }
}

// Row range from the wave partials (order keys): U_min / U_max are the least /
// greatest valid U of the row in the IEEE total order (+inf / -inf for a row without
// valid elements).  64 consecutive rows per block of kRangeWaves waves: lane l of every wave
// takes row i0 + l (coalesced reads of each partial column), wave w the partial columns
// w, w + kRangeWaves, ...; the waves' order keys are combined through LDS (min / max of
// integers: the same result in any order).  The result is valid in wave 0 only.
constexpr int kRangeWaves = 16;
__device__ __forceinline__ void row_range_block(const int* __restrict__ pmin, const int* __restrict__ pmax, int64_t d,
                                                int64_t i, int ntiles, float& umin, float& umax) {
  __shared__ int smin[kRangeWaves][64], smax[kRangeWaves][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int kmin = kKeyPosInf, kmax = kKeyNegInf;
  if (i < d) {
#pragma unroll 4
    for (int t = wid; t < ntiles; t += kRangeWaves) {
      kmin = min(kmin, pmin[(int64_t)t * d + i]);
      kmax = max(kmax, pmax[(int64_t)t * d + i]);
    }
  }
  smin[wid][lane] = kmin;
  smax[wid][lane] = kmax;
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int w = 1; w < kRangeWaves; ++w) {
      kmin = min(kmin, smin[w][lane]);
      kmax = max(kmax, smax[w][lane]);
    }
  }
  umin = key_f32(kmin);
  umax = key_f32(kmax);
}

// Exposes U_min / U_max (the statistics entry point).  `split` (nullable) is the
// per-row plane-split code of the MUL merge, cleared here and raised by the quantize
// kernel for rows holding some m >= 32640.  64 rows per block of kRangeWaves waves.
__global__ __launch_bounds__(64 * kRangeWaves) void k_row_range(int64_t d, int ntiles, const int* __restrict__ pmin,
                                                               const int* __restrict__ pmax, float* __restrict__ umin,
                                                               float* __restrict__ umax, uint8_t* __restrict__ split) {
  const int64_t i = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  float a, b;
  row_range_block(pmin, pmax, d, i, ntiles, a, b);
  if ((threadIdx.x >> 6) == 0 && i < d) {
    umin[i] = a;
    umax[i] = b;
    if (split) split[i] = 0;
  }
}

__device__ __forceinline__ void add_saturations(unsigned long long* sat, int local) {
  const unsigned long long tot = wave_sum_u64((unsigned long long)local);
  if (sat && (threadIdx.x & 63) == 0 && tot) atomicAdd(sat, tot);
}

// ---------------------------------------------------------------------------------
// Quantize kernels (MUL and SHIFT).  A block of 128 threads covers 1024 columns of
// kQRows rows; each thread owns 8 consecutive columns of every one of those rows, and
// all of its loads (U, W_round codes) are issued before any element is computed.
// Row groups are walked grid-stride, so any d fits the grid.
// ---------------------------------------------------------------------------------
typedef float vf4 __attribute__((ext_vector_type(4)));
typedef int vi4 __attribute__((ext_vector_type(4)));
typedef unsigned int vu2 __attribute__((ext_vector_type(2)));
// Plain (cached) vector loads and stores.  The U scratch the adaptation kernel has just
// written is read back largely from the Infinity Cache, and the merged integers stay
// there for the linear layer that reads them next; with non-temporal hints both round
// trips went to HBM (the FLUX block's step was 4 % slower).
__device__ __forceinline__ float4 load4f(const float* p) {
  const vf4 v = *reinterpret_cast<const vf4*>(p);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16(void* p, int4 v) { *reinterpret_cast<vi4*>(p) = vi4{v.x, v.y, v.z, v.w}; }
__device__ __forceinline__ void store8(void* p, uint2 v) { *reinterpret_cast<vu2*>(p) = vu2{v.x, v.y}; }
__device__ __forceinline__ void store4(void* p, uint32_t v) { *reinterpret_cast<uint32_t*>(p) = v; }

constexpr int kQThreads = 128;
constexpr int kQElems = 8;
constexpr int kQCols = kQThreads * kQElems;
constexpr int kQRows = 2;

// Smallest int16 whose row needs the bias byte split in the GEMM: the balanced split
// hi = (m + 128) >> 8 leaves the int8 range above 32639.
constexpr int kSplitBiasMin = 32640;

struct MulParams {
  float sbar;
  float rsbar;  // RN(1 / s_bar)
  int zbar;
};

// MUL: lo = min(U_min, 0), hi = max(U_max, 0), s_bar = (hi - lo)/(2^bU - 1) (1 unless
// > 0), z_bar = clamp(rint(-lo / s_bar)).
__device__ __forceinline__ MulParams mul_params(float umin, float umax, int qmax) {
  const float lo = fminf(umin, 0.0f), hi = fmaxf(umax, 0.0f);
  float sbar = (hi - lo) / (float)qmax;
  if (!(sbar > 0.0f)) sbar = 1.0f;
  const float zf = rintf(-lo / sbar);
  const int zbar = zf < 0.0f ? 0 : (zf > (float)qmax ? qmax : (int)zf);
  return MulParams{sbar, 1.0f / sbar, zbar};
}

// U_round = clamp(rint(U / s_bar) + z_bar, 0, 2^bU - 1)
__device__ __forceinline__ int mul_code(float u, float sbar, int zbar, int qmax) {
  float q = rintf(u / sbar);
  q = fminf(fmaxf(q, -65536.0f), 65536.0f);
  const int v = (int)q + zbar;
  return v < 0 ? 0 : (v > qmax ? qmax : v);
}

// U_round from q = U * RN(1/s_bar) instead of RN(U / s_bar).  With RN(1/s_bar) a
// normal number, q lies within (2^-23 + 2^-48) |U/s_bar| of U/s_bar and RN(U/s_bar)
// within 2^-24 |U/s_bar|, so for |q| < 512 the two are less than 2^-13 apart; when q
// is farther than 2^-11 from every half-integer (|q - rint(q)| < 1/2 - 2^-11; the
// difference is exact) they round to the same integer.  `exact` is false otherwise
// (also for a non-finite q or a subnormal RN(1/s_bar): rs_ok false), and the caller
// then recomputes the code with the IEEE division.
// (Every valid U lies in [lo, hi], so |U / s_bar| <= 2^bU - 1 < 512 whenever s_bar
// is the row's own scale.)
__device__ __forceinline__ int mul_code_fast(float u, const MulParams& P, bool rs_ok, int qmax, bool& exact) {
  const float qt = u * P.rsbar;
  const float r = rintf(qt);
  exact = rs_ok && fabsf(qt) < 512.0f && fabsf(qt - r) < 0.5f - 0x1p-11f;
  const float q = fminf(fmaxf(r, -65536.0f), 65536.0f);
  const int v = (int)q + P.zbar;
  return v < 0 ? 0 : (v > qmax ? qmax : v);
}

// m = (U_round - z_bar) w as int16, saturating (counted); w == 0 -> U_round = z_bar, m = 0.
__device__ __forceinline__ int mul_merge(int w, float u, const MulParams& P, int qmax, int& ur, int& nsat) {
  int mv = 0;
  ur = P.zbar;
  if (w != 0) {
    ur = mul_code(u, P.sbar, P.zbar, qmax);
    mv = (ur - P.zbar) * w;
  }
  if (mv > 32767) { mv = 32767; ++nsat; }
  if (mv < -32768) { mv = -32768; ++nsat; }
  return mv;
}

// Byte k (0 or 1) of four 32-bit values, packed into one dword with value e in byte e.
// __builtin_amdgcn_perm(a, b, sel): selector bytes 0-3 take b's bytes, 4-7 a's, 0x0C a zero.
__device__ __forceinline__ uint32_t gather_byte(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3, uint32_t k) {
  const uint32_t lo = __builtin_amdgcn_perm(v1, v0, 0x0C0C0000u | ((4u + k) << 8) | k);
  const uint32_t hi = __builtin_amdgcn_perm(v3, v2, ((4u + k) << 24) | (k << 16) | 0x0C0Cu);
  return lo | hi;
}

// Eight W_round codes of row i starting at column j0 (j0 % 8 == 0, n % 8 == 0).
template <bool W4>
__device__ __forceinline__ uint2 load_codes8(const uint8_t* __restrict__ wround, int64_t i, int64_t n, int64_t j0) {
  if (W4) return make_uint2(*reinterpret_cast<const uint32_t*>(wround + i * (n >> 1) + (j0 >> 1)), 0u);
  return *reinterpret_cast<const uint2*>(wround + i * n + j0);
}
template <bool W4>
__device__ __forceinline__ int code_of(uint2 v, int e) {
  if (W4) return (int)((v.x >> (4 * e)) & 15u);
  return (int)(((e < 4 ? v.x : v.y) >> (8 * (e & 3))) & 255u);
}
template <bool W4>
__device__ __forceinline__ int code_at(const uint8_t* __restrict__ wround, int64_t i, int64_t n, int64_t j) {
  if (W4) {
    const uint8_t byte = wround[i * (n >> 1) + (j >> 1)];
    return (j & 1) ? (byte >> 4) : (byte & 15);
  }
  return wround[i * n + j];
}

// Per-row parameters of the MUL quantizer, once per row before the element pass: the
// row range (the reduction of the adaptation kernel's partials into umin_out / umax_out,
// or the caller's umin_in / umax_in), s_bar and z_bar (written to the outputs), RN(1 /
// s_bar), and whether every merged integer of the row is certainly small:
// max |U_round - z_bar| max |W_round - z| <= 32639 (codes W_round in [0, wmax]), so that
// no element saturates or needs the bias byte split.  split (nullable) is cleared; the
// quantize kernel raises it for rows holding some m >= 32640.  With `planes` it is
// the row's byte-plane code instead: 0 for a small row (balanced split; the quantize
// kernel raises bit 0 when some high byte is not zero), 3 otherwise (bias split).
// 64 rows per block of kRangeWaves waves (the row range as in k_row_range); wave 0 then
// derives each row's parameters.
__global__ __launch_bounds__(64 * kRangeWaves) void k_mul_params(int64_t d, int ntiles, const int* __restrict__ pmin,
                                                                const int* __restrict__ pmax,
                                                                const float* __restrict__ umin_in,
                                                                const float* __restrict__ umax_in,
                                                                float* __restrict__ umin_out,
                                                                float* __restrict__ umax_out, int qmax, int wmax,
                                                                const int32_t* __restrict__ z, float* __restrict__ sbar,
                                                                int32_t* __restrict__ zbar, float* __restrict__ rs,
                                                                int* __restrict__ small, uint8_t* __restrict__ split,
                                                                bool planes) {
  const int64_t i = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  float a = 0.0f, b = 0.0f;
  if (!umin_in) row_range_block(pmin, pmax, d, i, ntiles, a, b);  // uniform: every wave reaches the barrier
  if ((threadIdx.x >> 6) != 0 || i >= d) return;
  {
    if (umin_in) {
      a = umin_in[i];
      b = umax_in[i];
    } else {
      umin_out[i] = a;
      umax_out[i] = b;
    }
    const MulParams P = mul_params(a, b, qmax);
    sbar[i] = P.sbar;
    zbar[i] = P.zbar;
    rs[i] = P.rsbar;
    const int64_t zi = z[i];
    const int64_t mw = max(zi < 0 ? -zi : zi, (int64_t)wmax - zi < 0 ? zi - wmax : (int64_t)wmax - zi);
    const int64_t mu = max(P.zbar, qmax - P.zbar);
    const bool sm = mw * mu <= (int64_t)(kSplitBiasMin - 1);
    small[i] = sm;
    if (split) split[i] = planes ? (sm ? 0 : 3) : 0;
  }
}

// Output forms of the MUL quantizer.
//  kOutInt16:  m as int16 d x n (and the split codes);
//  kOutCodes:  U_round itself as packed nibbles (u_bits <= 4, n even; low nibble = even
//              column), for a linear layer that forms m on load;
//  kOutPlanes: m already split into its two int8 planes, the layout the linear layer
//              reads without conversion: per row, the n high bytes, then the n low
//              bytes (d x 2n bytes; n % 16 == 0).  A small
//              row (plane code 0 on entry) takes the balanced split hi = (m + 128) >> 8,
//              lo = m - 256 hi, and its code becomes 1 when some hi is not zero; any other
//              row (code 3) takes the bias split hi = m >> 8, lo = (m & 0xFF) - 128.
// Per-row s_bar, z_bar, RN(1 / s_bar) and the small-row flag come from k_mul_params.
enum { kOutInt16 = 0, kOutCodes = 1, kOutPlanes = 2 };

template <bool W4, int OUT>
__global__ __launch_bounds__(kQThreads) void k_quant_mul(int64_t d, int64_t n, int u_bits,
                                                        const uint8_t* __restrict__ wround,
                                                        const int32_t* __restrict__ z, const float* __restrict__ U,
                                                        const float* __restrict__ sbar_r,
                                                        const int32_t* __restrict__ zbar_r,
                                                        const float* __restrict__ rs_r,
                                                        const int* __restrict__ small_r, int16_t* __restrict__ m,
                                                        uint8_t* __restrict__ split, uint8_t* __restrict__ uround_dbg,
                                                        unsigned long long* __restrict__ sat,
                                                        uint8_t* __restrict__ ucode) {
  const int qmax = (1 << u_bits) - 1;
  const int64_t j0 = (int64_t)blockIdx.x * kQCols + (int64_t)threadIdx.x * kQElems;
  const int64_t ngroups = (d + kQRows - 1) / kQRows;
  int nsat = 0;
  for (int64_t g = blockIdx.y; g < ngroups; g += gridDim.y) {
    const int64_t i0 = g * kQRows;
    if ((n & 7) == 0) {
      float4 ua[kQRows], ub[kQRows];
      uint2 cw[kQRows];
#pragma unroll
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i < d && j0 < n) {
          cw[rr] = load_codes8<W4>(wround, i, n, j0);
          ua[rr] = load4f(U + i * n + j0);
          ub[rr] = load4f(U + i * n + j0 + 4);
        }
      }
#pragma unroll
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i >= d || j0 >= n) break;
        const MulParams P{sbar_r[i], rs_r[i], zbar_r[i]};
        const bool rs_ok = P.rsbar >= 0x1p-126f;  // a normal reciprocal
        const bool small = small_r[i] != 0;
        const int zi = z[i];
        const float uu[8] = {ua[rr].x, ua[rr].y, ua[rr].z, ua[rr].w, ub[rr].x, ub[rr].y, ub[rr].z, ub[rr].w};
        int mm[8], ur[8], w[8];
        bool redo[8], any = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          w[e] = code_of<W4>(cw[rr], e) - zi;
          bool exact = true;
          ur[e] = w[e] != 0 ? mul_code_fast(uu[e], P, rs_ok, qmax, exact) : P.zbar;
          redo[e] = !exact;
          any = any || redo[e];
        }
        // the IEEE division runs only in waves where some lane needs it
        if (__builtin_amdgcn_ballot_w64(any) != 0) {
          __asm__ volatile("");  // keeps the branch: the division is not speculated
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (redo[e]) ur[e] = mul_code(uu[e], P.sbar, P.zbar, qmax);
        }
        if (OUT == kOutCodes) {
          uint32_t pk = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) pk |= (uint32_t)ur[e] << (4 * e);
          store4(ucode + ((i * n + j0) >> 1), pk);
          continue;
        }
        if (small) {  // |m| <= 32639 for the whole row: no saturation, no bias split
#pragma unroll
          for (int e = 0; e < 8; ++e) mm[e] = (ur[e] - P.zbar) * w[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            int mv = w[e] != 0 ? (ur[e] - P.zbar) * w[e] : 0;
            if (mv > 32767) { mv = 32767; ++nsat; }
            if (mv < -32768) { mv = -32768; ++nsat; }
            mm[e] = mv;
          }
          if (OUT == kOutInt16 && split) {  // the balanced byte split of the int16 GEMM needs m <= 32639
            int mx = mm[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mx = max(mx, mm[e]);
            if (mx >= kSplitBiasMin) split[i] = 1;
          }
        }
        if (OUT == kOutPlanes) {
          // In both splits the low plane is the low byte of m (m - 256 hi keeps it; the bias
          // split then flips bit 7), and the high plane is byte 1 of m + 128 (balanced) or of
          // m (bias).  The bytes of four values at a time are gathered with v_perm.
          uint32_t t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = (uint32_t)(small ? mm[e] + 128 : mm[e]);
          const uint32_t flip = small ? 0u : 0x80808080u;
          const uint2 hi = make_uint2(gather_byte(t[0], t[1], t[2], t[3], 1), gather_byte(t[4], t[5], t[6], t[7], 1));
          const uint2 lo = make_uint2(gather_byte((uint32_t)mm[0], (uint32_t)mm[1], (uint32_t)mm[2], (uint32_t)mm[3], 0) ^ flip,
                                      gather_byte((uint32_t)mm[4], (uint32_t)mm[5], (uint32_t)mm[6], (uint32_t)mm[7], 0) ^ flip);
          // Lanes 2k and 2k + 1 hold columns 0-7 and 8-15 of one group of 16 (n % 16 == 0,
          // so both are active for every row): they swap halves so that the even lane
          // stores the group's 16 high bytes (in the row's high plane) and the odd lane its
          // 16 low bytes (in the low plane, n bytes further on), one 16-byte store each.
          const bool odd = (threadIdx.x & 1) != 0;
          const uint2 give = odd ? hi : lo;
          const uint2 got = make_uint2((uint32_t)__shfl_xor((int)give.x, 1, kWave), (uint32_t)__shfl_xor((int)give.y, 1, kWave));
          uint8_t* grp = reinterpret_cast<uint8_t*>(m) + i * 2 * n + (j0 & ~(int64_t)15);
          if (odd)
            store16(grp + n, make_int4((int)got.x, (int)got.y, (int)lo.x, (int)lo.y));
          else
            store16(grp, make_int4((int)hi.x, (int)hi.y, (int)got.x, (int)got.y));
          if (small && (hi.x | hi.y) != 0u) split[i] = 1;
        } else {
        int4 pk;
        pk.x = (int)__builtin_amdgcn_perm((uint32_t)mm[1], (uint32_t)mm[0], 0x05040100u);
        pk.y = (int)__builtin_amdgcn_perm((uint32_t)mm[3], (uint32_t)mm[2], 0x05040100u);
        pk.z = (int)__builtin_amdgcn_perm((uint32_t)mm[5], (uint32_t)mm[4], 0x05040100u);
        pk.w = (int)__builtin_amdgcn_perm((uint32_t)mm[7], (uint32_t)mm[6], 0x05040100u);
        store16(m + i * n + j0, pk);
        }
        if (uround_dbg) {
          uint2 pu;
          pu.x = (uint32_t)ur[0] | ((uint32_t)ur[1] << 8) | ((uint32_t)ur[2] << 16) | ((uint32_t)ur[3] << 24);
          pu.y = (uint32_t)ur[4] | ((uint32_t)ur[5] << 8) | ((uint32_t)ur[6] << 16) | ((uint32_t)ur[7] << 24);
          *reinterpret_cast<uint2*>(uround_dbg + i * n + j0) = pu;
        }
      }
    } else {
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i >= d) break;
        const MulParams P{sbar_r[i], rs_r[i], zbar_r[i]};
        const int zi = z[i];
        int lo_code = 0;
        for (int e = 0; e < kQElems; ++e) {
          const int64_t j = j0 + e;
          if (j >= n) break;
          int uv;
          const int mv = mul_merge(code_at<W4>(wround, i, n, j) - zi, U[i * n + j], P, qmax, uv, nsat);
          if (OUT == kOutCodes) {  // n is even: the odd column of every pair exists
            if ((j & 1) == 0)
              lo_code = uv;
            else
              ucode[(i * n + j) >> 1] = (uint8_t)(lo_code | (uv << 4));
            continue;
          }
          m[i * n + j] = (int16_t)mv;
          if (split && mv >= kSplitBiasMin) split[i] = 1;
          if (uround_dbg) uround_dbg[i * n + j] = (uint8_t)uv;
        }
      }
    }
  }
  add_saturations(sat, nsat);
}

// QLoRA-style requant of x (the comparison path): the base quantizer of "1. AQS" per
// row at `bits`, over every element.  Its parameters follow the same formulas as the
// MUL quantizer (lo = min(x_min, 0), hi = max(x_max, 0), s' = (hi - lo)/(2^b - 1),
// z' = clamp(rint(-lo/s')), code = clamp(rint(x/s') + z')), so the same helpers serve.
// Output: uint8 codes (8 bits) or packed nibbles, low nibble = even column (4 bits).
template <bool OUT4>
__global__ __launch_bounds__(kQThreads) void k_quant_ptq(int64_t d, int64_t n, int bits, const float* __restrict__ X,
                                                        const float* __restrict__ xmin_r,
                                                        const float* __restrict__ xmax_r, uint8_t* __restrict__ code,
                                                        float* __restrict__ s_out, int32_t* __restrict__ z_out) {
  const int qmax = (1 << bits) - 1;
  const int64_t j0 = (int64_t)blockIdx.x * kQCols + (int64_t)threadIdx.x * kQElems;
  const int64_t ngroups = (d + kQRows - 1) / kQRows;
  for (int64_t g = blockIdx.y; g < ngroups; g += gridDim.y) {
    const int64_t i0 = g * kQRows;
    if ((n & 7) == 0) {
      float4 xa[kQRows], xb[kQRows];
#pragma unroll
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i < d && j0 < n) {
          xa[rr] = load4f(X + i * n + j0);
          xb[rr] = load4f(X + i * n + j0 + 4);
        }
      }
#pragma unroll
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i >= d) break;
        const MulParams P = mul_params(xmin_r[i], xmax_r[i], qmax);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
          s_out[i] = P.sbar;
          z_out[i] = P.zbar;
        }
        if (j0 >= n) continue;
        const float xx[8] = {xa[rr].x, xa[rr].y, xa[rr].z, xa[rr].w, xb[rr].x, xb[rr].y, xb[rr].z, xb[rr].w};
        int cd[8];
        bool redo[8], any = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bool exact = true;
          cd[e] = mul_code_fast(xx[e], P, P.rsbar >= 0x1p-126f, qmax, exact);
          redo[e] = !exact;
          any = any || redo[e];
        }
        if (__builtin_amdgcn_ballot_w64(any) != 0) {
          __asm__ volatile("");  // keeps the branch: the division is not speculated
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (redo[e]) cd[e] = mul_code(xx[e], P.sbar, P.zbar, qmax);
        }
        if (OUT4) {
          uint32_t pk = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) pk |= (uint32_t)cd[e] << (4 * e);
          store4(code + i * (n >> 1) + (j0 >> 1), pk);
        } else {
          uint2 pk;
          pk.x = (uint32_t)cd[0] | ((uint32_t)cd[1] << 8) | ((uint32_t)cd[2] << 16) | ((uint32_t)cd[3] << 24);
          pk.y = (uint32_t)cd[4] | ((uint32_t)cd[5] << 8) | ((uint32_t)cd[6] << 16) | ((uint32_t)cd[7] << 24);
          store8(code + i * n + j0, pk);
        }
      }
    } else {
      // general n (4-bit output needs even n, validated): pairs, so a packed byte is whole
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i >= d) break;
        const MulParams P = mul_params(xmin_r[i], xmax_r[i], qmax);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
          s_out[i] = P.sbar;
          z_out[i] = P.zbar;
        }
        for (int e = 0; e < kQElems; e += 2) {
          const int64_t j = j0 + e;
          if (j >= n) break;
          int c2[2] = {0, 0};
          for (int h = 0; h < 2; ++h)
            if (j + h < n) c2[h] = mul_code(X[i * n + j + h], P.sbar, P.zbar, qmax);
          if (OUT4) {
            code[i * (n >> 1) + (j >> 1)] = (uint8_t)(c2[0] | (c2[1] << 4));
          } else {
            code[i * n + j] = (uint8_t)c2[0];
            if (j + 1 < n) code[i * n + j + 1] = (uint8_t)c2[1];
          }
        }
      }
    }
  }
}

// SHIFT: s_bar = max(|U_min|, |U_max|) (1 for an empty / zero row), V = U / s_bar,
// shift = clamp(-round(log2|V|), 0, 2^bV - 1) (V == 0: largest code, m = 0),
// m = sign(V) (w >> shift) (arithmetic), saturated to bW signed bits.  Output int8
// (bW = 8) or packed int4 nibbles (bW = 4, low nibble = even column).
__device__ __forceinline__ float shift_scale(float umin, float umax) {
  float sb = fmaxf(fabsf(umin), fabsf(umax));
  if (!(sb > 0.0f) || isinf(sb)) sb = 1.0f;
  return sb;
}

__device__ __forceinline__ int shift_merge(int w, float u, float sbar, int smax, int mlo, int mhi, int& sh,
                                           int& nsat) {
  if (w == 0) {
    sh = 255;
    return 0;
  }
  const float v = u / sbar;
  int mv;
  if (v == 0.0f) {
    sh = smax;
    mv = 0;
  } else {
    int k = -log2_round_bits(v);
    sh = k < 0 ? 0 : (k > smax ? smax : k);
    const int fl = w >> (sh > 31 ? 31 : sh);
    mv = v > 0.0f ? fl : -fl;
  }
  if (mv > mhi) { mv = mhi; ++nsat; }
  if (mv < mlo) { mv = mlo; ++nsat; }
  return mv;
}

template <bool W4>
__global__ __launch_bounds__(kQThreads) void k_quant_shift(int64_t d, int64_t n, int v_bits,
                                                          const uint8_t* __restrict__ wround,
                                                          const int32_t* __restrict__ z, const float* __restrict__ U,
                                                          const float* __restrict__ umin_r,
                                                          const float* __restrict__ umax_r, uint8_t* __restrict__ m,
                                                          float* __restrict__ sbar_out,
                                                          uint8_t* __restrict__ shift_dbg,
                                                          unsigned long long* __restrict__ sat) {
  const int smax = (1 << v_bits) - 1;
  const int mhi = W4 ? 7 : 127, mlo = W4 ? -8 : -128;
  const int64_t j0 = (int64_t)blockIdx.x * kQCols + (int64_t)threadIdx.x * kQElems;
  const int64_t ngroups = (d + kQRows - 1) / kQRows;
  int nsat = 0;
  for (int64_t g = blockIdx.y; g < ngroups; g += gridDim.y) {
    const int64_t i0 = g * kQRows;
    if ((n & 7) == 0) {
      float4 ua[kQRows], ub[kQRows];
      uint2 cw[kQRows];
#pragma unroll
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i < d && j0 < n) {
          cw[rr] = load_codes8<W4>(wround, i, n, j0);
          ua[rr] = load4f(U + i * n + j0);
          ub[rr] = load4f(U + i * n + j0 + 4);
        }
      }
#pragma unroll
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i >= d) break;
        const float umin = umin_r[i], umax = umax_r[i];
        const float sbar = shift_scale(umin, umax);
        if (blockIdx.x == 0 && threadIdx.x == 0) sbar_out[i] = sbar;
        if (j0 >= n) continue;
        const int zi = z[i];
        const float uu[8] = {ua[rr].x, ua[rr].y, ua[rr].z, ua[rr].w, ub[rr].x, ub[rr].y, ub[rr].z, ub[rr].w};
        int mm[8], sh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          mm[e] = shift_merge(code_of<W4>(cw[rr], e) - zi, uu[e], sbar, smax, mlo, mhi, sh[e], nsat);
        if (W4) {
          uint32_t pk = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) pk |= ((uint32_t)mm[e] & 15u) << (4 * e);
          store4(m + i * (n >> 1) + (j0 >> 1), pk);
        } else {
          uint2 pk;
          pk.x = ((uint32_t)mm[0] & 255u) | (((uint32_t)mm[1] & 255u) << 8) | (((uint32_t)mm[2] & 255u) << 16) |
                 ((uint32_t)mm[3] << 24);
          pk.y = ((uint32_t)mm[4] & 255u) | (((uint32_t)mm[5] & 255u) << 8) | (((uint32_t)mm[6] & 255u) << 16) |
                 ((uint32_t)mm[7] << 24);
          store8(m + i * n + j0, pk);
        }
        if (shift_dbg) {
          uint2 ps;
          ps.x = (uint32_t)sh[0] | ((uint32_t)sh[1] << 8) | ((uint32_t)sh[2] << 16) | ((uint32_t)sh[3] << 24);
          ps.y = (uint32_t)sh[4] | ((uint32_t)sh[5] << 8) | ((uint32_t)sh[6] << 16) | ((uint32_t)sh[7] << 24);
          *reinterpret_cast<uint2*>(shift_dbg + i * n + j0) = ps;
        }
      }
    } else {
      // general n (W4 needs even n, validated): pairs, so that a packed byte is written whole
      for (int rr = 0; rr < kQRows; ++rr) {
        const int64_t i = i0 + rr;
        if (i >= d) break;
        const float umin = umin_r[i], umax = umax_r[i];
        const float sbar = shift_scale(umin, umax);
        if (blockIdx.x == 0 && threadIdx.x == 0) sbar_out[i] = sbar;
        const int zi = z[i];
        for (int e = 0; e < kQElems; e += 2) {
          const int64_t j = j0 + e;
          if (j >= n) break;
          int mm2[2] = {0, 0}, sh2[2] = {255, 255};
          for (int h = 0; h < 2; ++h) {
            const int64_t jj = j + h;
            if (jj < n)
              mm2[h] = shift_merge(code_at<W4>(wround, i, n, jj) - zi, U[i * n + jj], sbar, smax, mlo, mhi, sh2[h],
                                   nsat);
          }
          if (W4) {
            m[i * (n >> 1) + (j >> 1)] = (uint8_t)(((uint32_t)mm2[0] & 15u) | (((uint32_t)mm2[1] & 15u) << 4));
          } else {
            m[i * n + j] = (uint8_t)mm2[0];
            if (j + 1 < n) m[i * n + j + 1] = (uint8_t)mm2[1];
          }
          if (shift_dbg) {
            shift_dbg[i * n + j] = (uint8_t)sh2[0];
            if (j + 1 < n) shift_dbg[i * n + j + 1] = (uint8_t)sh2[1];
          }
        }
      }
    }
  }
  add_saturations(sat, nsat);
}

// =================================================================================
// Host launchers (called by the C ABI layer after validation).
// =================================================================================
// Blocks of the row-range kernels: one per 64 rows, every row covered (d < 2^31).
static inline unsigned range_blocks(int64_t d) { return (unsigned)(d > 0 ? (d + 63) / 64 : 1); }

static inline unsigned grid1(uint64_t work, unsigned block) {
  uint64_t g = (work + block - 1) / block;
  if (g > (1u << 20)) g = 1u << 20;
  return (unsigned)(g ? g : 1);
}

hipError_t launch_gen_r(int64_t d, int64_t n, uint64_t seed, uint32_t layer_id, const float* c, float* out, int dist,
                        hipStream_t st) {
  const uint64_t blocks4 = ((uint64_t)d * (uint64_t)n + 3) / 4;
  hipLaunchKernelGGL(k_gen_r, dim3(grid1(blocks4, 256)), dim3(256), 0, st, d, n, seed, layer_id, c, out, dist);
  return hipGetLastError();
}

// Debug: the auxiliary sample of each element of `blocks` given Philox blocks (4 words
// each) under distribution `dist`.
__global__ __launch_bounds__(256) void k_aux_debug(int64_t blocks, const uint32_t* __restrict__ words, int dist,
                                                  float* __restrict__ out) {
  __shared__ LnLds tab[96];
  load_ln_table(tab);
  __syncthreads();
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < blocks; t += (int64_t)gridDim.x * blockDim.x) {
    const U4 v{words[4 * t], words[4 * t + 1], words[4 * t + 2], words[4 * t + 3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * t + e] = aux_sample_rt(dist, v, (unsigned)e, tab);
  }
}

hipError_t launch_aux_debug(int64_t blocks, const uint32_t* words, int dist, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_aux_debug, dim3(grid1((uint64_t)blocks, 256)), dim3(256), 0, st, blocks, words, dist, out);
  return hipGetLastError();
}

// Diagnostic: the rank-r product acc[i][j] = sum_k A[i][k] B[k][j] formed on the
// matrix cores as the merge kernels form it, one instruction per k in increasing k,
// starting from +0 (d x r and r x n fp32 inputs; d x n output).  One wave per tile of
// 32 (FORM 0) or 4 (FORM 1) rows x 64 columns; d and n are multiples of the tile.
//  FORM 0, v_mfma_f32_32x32x1f32 taken transposed as in the adaptation kernel: lane l
//   supplies B[k][j0 + l] (A operand) and A[i0 + l % 32][k] (B operand); register
//   4 g + e of lane l ends with row i0 + l % 32, column j0 + 32 (g >> 2) + 8 (g & 3) +
//   4 (l >> 5) + e.
//  FORM 1, v_mfma_f32_4x4x1f32 as in the fused merge: lane l supplies B[k][j0 + l] and
//   A[i0 + l % 4][k]; register e of lane 4 b + q ends with row i0 + q, column j0 + 4 b + e.
template <int FORM>
__global__ __launch_bounds__(64) void k_debug_mfma_chain(int64_t d, int64_t n, int r, const float* __restrict__ A,
                                                        const float* __restrict__ B, float* __restrict__ out) {
  const int lane = threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.x * 64, i0 = (int64_t)blockIdx.y * (FORM == 0 ? 32 : 4);
  if (FORM == 0) {
    v32f acc;
#pragma unroll
    for (int x = 0; x < 32; ++x) acc[x] = 0.0f;
    for (int k = 0; k < r; ++k)
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(B[(int64_t)k * n + j0 + lane], A[(i0 + (lane & 31)) * r + k], acc,
                                                 0, 0, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[(i0 + (lane & 31)) * n + j0 + 32 * (g >> 2) + 8 * (g & 3) + 4 * (lane >> 5) + e] = acc[4 * g + e];
  } else {
    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < r; ++k)
      acc = __builtin_amdgcn_mfma_f32_4x4x1f32(B[(int64_t)k * n + j0 + lane], A[(i0 + (lane & 3)) * r + k], acc, 0, 0,
                                               0);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(i0 + (lane & 3)) * n + j0 + 4 * (lane >> 2) + e] = acc[e];
  }
}

hipError_t launch_debug_mfma_chain(int form, int64_t d, int64_t n, int r, const float* A, const float* B, float* out,
                                   hipStream_t st) {
  const dim3 grid((unsigned)(n / 64), (unsigned)(d / (form == 0 ? 32 : 4)));
  if (form == 0)
    hipLaunchKernelGGL(k_debug_mfma_chain<0>, grid, dim3(64), 0, st, d, n, r, A, B, out);
  else
    hipLaunchKernelGGL(k_debug_mfma_chain<1>, grid, dim3(64), 0, st, d, n, r, A, B, out);
  return hipGetLastError();
}

hipError_t launch_ln_odd(int64_t count, const uint32_t* G, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_ln_odd, dim3(grid1((uint64_t)count, 256)), dim3(256), 0, st, count, G, out);
  return hipGetLastError();
}

hipError_t launch_sigma_w(int64_t d, int64_t n, const float* W, float* sigma, hipStream_t st) {
  hipLaunchKernelGGL(k_sigma_w, dim3((unsigned)d), dim3(256), 0, st, n, W, sigma);
  return hipGetLastError();
}

hipError_t launch_vmc_scale(int64_t d, const float* sigma, double alpha, float* c, int dist, hipStream_t st) {
  hipLaunchKernelGGL(k_vmc_scale, dim3(grid1((uint64_t)d, 256)), dim3(256), 0, st, d, sigma, alpha, c,
                     dist != kAuxLaplace);
  return hipGetLastError();
}

hipError_t launch_base_quant(int64_t d, int64_t n, int bits, uint64_t seed, uint32_t layer_id, const float* W,
                             const float* c, uint8_t* wround, int32_t* z, float* s, int dist, hipStream_t st) {
  const size_t lds = (size_t)n * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_base_quant),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 32768 * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_base_quant, dim3((unsigned)d), dim3(256), lds, st, n, bits, seed, layer_id, W, c, wround, z, s,
                     dist);
  return hipGetLastError();
}

hipError_t launch_quant_act(int64_t M, int64_t n, const float* X, int8_t* xq, float* sx, int32_t* rowsum,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_quant_act, dim3((unsigned)M), dim3(256), 0, st, n, X, xq, sx, rowsum);
  return hipGetLastError();
}

// Row partials per row: one per wave (4 per 256-column block) on the matrix-core path,
// one per 1024-column tile on the general path.
int adapt_max_ntiles(int64_t n) { return 4 * (int)((n + kMfmaCols - 1) / kMfmaCols); }

template <int R, bool W4, bool PTQ, int DIST>
static int64_t mfma_slots() {
  static int64_t slots = 0;
  if (slots == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&k_adapt_mfma<R, W4, PTQ, DIST>), 256,
                                                     0) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
      return 1024;
    slots = (int64_t)cus * per_cu;
  }
  return slots;
}

template <int R, bool W4, bool PTQ, int DIST>
static hipError_t launch_adapt_mfma(const AdaptArgs& a, int* ntiles_out, hipStream_t st) {
  const int ntiles = (int)((a.n + kMfmaCols - 1) / kMfmaCols);
  *ntiles_out = 4 * ntiles;  // a partial per wave
  const int64_t row_tiles = (a.d + 31) / 32;
  const int64_t slots = mfma_slots<R, W4, PTQ, DIST>();
  // row tiles per block (1..8): the count whose grid best fills the resident slots
  int rtiles = 1;
  double best = -1.0;
  for (int rt = 1; rt <= kMfmaMaxRowTiles; ++rt) {
    const int64_t blocks = ((row_tiles + rt - 1) / rt) * (int64_t)ntiles;
    const int64_t rounds = (blocks + slots - 1) / slots;
    const double eff = (double)blocks / (double)(rounds * slots);
    if (eff >= best - 1e-9) {
      best = eff;
      rtiles = rt;
    }
  }
  const int64_t nrb = (row_tiles + rtiles - 1) / rtiles;
  for (int64_t rb0 = 0; rb0 < nrb; rb0 += 65535) {
    const int64_t cnt = nrb - rb0 < 65535 ? nrb - rb0 : 65535;
    const dim3 grid((unsigned)ntiles, (unsigned)cnt);
    unsigned long long* sz = rb0 == 0 ? a.sat_zero : nullptr;
    hipLaunchKernelGGL((k_adapt_mfma<R, W4, PTQ, DIST>), grid, dim3(256), 0, st, a.d, a.n, a.seed, a.layer_id, a.wround, a.z,
                       a.s, a.c, a.A, a.B, a.U, a.pmin, a.pmax, ntiles, rtiles, rb0, sz, a.row0);
  }
  return hipGetLastError();
}

template <int R, int DIST>
static hipError_t launch_adapt_md(const AdaptArgs& a, int* ntiles_out, hipStream_t st) {
  if (a.ptq)
    return a.w_bits == 4 ? launch_adapt_mfma<R, true, true, DIST>(a, ntiles_out, st)
                         : launch_adapt_mfma<R, false, true, DIST>(a, ntiles_out, st);
  return a.w_bits == 4 ? launch_adapt_mfma<R, true, false, DIST>(a, ntiles_out, st)
                       : launch_adapt_mfma<R, false, false, DIST>(a, ntiles_out, st);
}

template <int R>
static hipError_t launch_adapt_m(const AdaptArgs& a, int* ntiles_out, hipStream_t st) {
  switch (a.dist) {
    case kAuxGauss: return launch_adapt_md<R, kAuxGauss>(a, ntiles_out, st);
    case kAuxCauchy: return launch_adapt_md<R, kAuxCauchy>(a, ntiles_out, st);
    case kAuxStudentT2: return launch_adapt_md<R, kAuxStudentT2>(a, ntiles_out, st);
    default: return launch_adapt_md<R, kAuxLaplace>(a, ntiles_out, st);
  }
}

hipError_t launch_adapt(const AdaptArgs& a, int* ntiles_out, hipStream_t st) {
  const bool fast_ok = (a.n % 4) == 0 && ((reinterpret_cast<uintptr_t>(a.B) | reinterpret_cast<uintptr_t>(a.U)) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.wround) & 3) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.A) & 15) == 0;
  if (fast_ok && !a.force_generic) {
    switch (a.r) {
      case 4: return launch_adapt_m<4>(a, ntiles_out, st);
      case 8: return launch_adapt_m<8>(a, ntiles_out, st);
      case 16: return launch_adapt_m<16>(a, ntiles_out, st);
      case 32: return launch_adapt_m<32>(a, ntiles_out, st);
      case 64: return launch_adapt_m<64>(a, ntiles_out, st);
      default: break;
    }
  }
  const int ntiles = (int)((a.n + kAdaptCols - 1) / kAdaptCols);
  *ntiles_out = ntiles;
  dim3 grid((unsigned)ntiles, (unsigned)(a.d < 65535 ? (a.d ? a.d : 1) : 65535));
  hipLaunchKernelGGL(k_adapt_generic, grid, dim3(256), 0, st, a.d, a.n, a.r, a.w_bits, a.seed, a.layer_id, a.wround,
                     a.z, a.s, a.c, a.A, a.B, a.U, a.pmin, a.pmax, ntiles, a.sat_zero, a.ptq, a.dist, a.row0);
  return hipGetLastError();
}

hipError_t launch_row_range(int64_t d, int ntiles, const int* pmin, const int* pmax, float* umin, float* umax,
                            uint8_t* split, hipStream_t st) {
  hipLaunchKernelGGL(k_row_range, dim3(range_blocks(d)), dim3(64 * kRangeWaves), 0, st, d, ntiles, pmin, pmax, umin, umax,
                     split);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Fused single-pass MUL merge with no scratch memory.  A block owns RB = 16 / NG whole
// rows (8 for NG = 1; n <= 1024 NG) and keeps their U in LDS (RB rows at a pitch of n
// rounded up to 4 floats, at most 64 KB, sized to n so that three blocks share a
// compute unit where they fit; A's rows follow), so each
// row's range is complete (block reduction) before any of its elements is quantized
// and U never leaves the chip.  Thread t computes columns 4 (t + 256 g) .. + 3 of
// every row of the block (and quantizes the same ones).  The rank-r term is the fmaf
// chain of the definition on the vector ALU: B[k][4 columns] is read once (from L2)
// per column group and k and serves all RB rows.  Every other step is the one of the
// adaptation and quantize kernels, in the same order, so the outputs are the same bits.
// ---------------------------------------------------------------------------------
template <int NG>
struct FusedLds {
  static constexpr int RB = NG == 1 ? 8 : 16 / NG;  // rows per block
  static constexpr int COLS = 1024 * NG;
  // U rows + A rows (+ 8 floats: the last row's vector reads may run up to 7 past r)
  static constexpr int MAX_BYTES = RB * COLS * 4 + (RB * 128 + 8) * 4;
  static int64_t bytes(int64_t n, int r) {
    return (int64_t)RB * ((n + 3) & ~(int64_t)3) * 4 + ((int64_t)RB * ((r + 3) & ~3) + 8) * 4;
  }
};

template <int NG, bool W4, int DIST>
__global__ __launch_bounds__(256) void k_merge_fused(int64_t d, int64_t n, int r, int u_bits, uint64_t seed,
                                                    uint32_t layer_id, const uint8_t* __restrict__ wround,
                                                    const int32_t* __restrict__ z, const float* __restrict__ s,
                                                    const float* __restrict__ c, const float* __restrict__ A,
                                                    const float* __restrict__ B, int16_t* __restrict__ m,
                                                    float* __restrict__ sbar_out, int32_t* __restrict__ zbar_out,
                                                    uint8_t* __restrict__ split, uint8_t* __restrict__ uround_dbg,
                                                    unsigned long long* __restrict__ sat) {
  constexpr int RB = FusedLds<NG>::RB;
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  const int64_t pitch = (n + 3) & ~(int64_t)3;  // U's row pitch in LDS
  const int RP = (r + 3) & ~3;                  // A's row pitch in LDS: rows start 16-byte aligned
  float* __restrict__ sU = dyn;                 // RB x pitch
  float* __restrict__ sA = dyn + RB * pitch;    // RB x RP
  __shared__ LnLds tab[96];
  __shared__ float rcp[511];
  __shared__ int smin[4][RB], smax[4][RB];
  __shared__ int sflag[RB];
  load_ln_table(tab);
  load_rcp_table(rcp);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int qmax = (1 << u_bits) - 1;
  const bool quad = (n & 3) == 0;
  int nsat = 0;
  for (int64_t i0 = (int64_t)blockIdx.x * RB; i0 < d; i0 += (int64_t)gridDim.x * RB) {
    __syncthreads();  // tables in place; the previous rows' LDS reads are done
    for (int x = tid; x < RB * RP; x += 256) {
      const int rr = x / RP, k = x - rr * RP;
      sA[x] = i0 + rr < d && k < r ? A[(i0 + rr) * r + k] : 0.0f;
    }
    if (tid < RB) sflag[tid] = 0;
    __syncthreads();
    bool done = false;
    if constexpr (RB == 8) {  // measured: at RB = 4 the vector-ALU chain below is faster
      if (quad) {
        // Rank-r term on the matrix cores: v_mfma_f32_4x4x1f32 forms 16 blocks of 4 x 4
        // outer products with one rounding per k, so a chain of r of them in k order is
        // the fmaf chain of the definition.  Taken transposed (MFMA rows = columns j,
        // MFMA columns = rows i), lane 4b + q ends with row q of its row group and the 4
        // consecutive columns of block b: one Philox block per lane and chunk.  A wave
        // covers 4 chunks of 64 columns per column group.
        constexpr int RG = RB / 4;  // row groups of 4
        const int jr = lane & 3, bq = lane >> 2;
        int kmn[RG], kmx[RG], zr[RG];
        float cr[RG], sr[RG];
        int64_t ir[RG];
        bool okr[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          okr[rg] = i0 + 4 * rg + jr < d;
          ir[rg] = okr[rg] ? i0 + 4 * rg + jr : d - 1;  // a row past d is computed, never stored
          zr[rg] = z[ir[rg]];
          cr[rg] = c[ir[rg]];
          sr[rg] = s[ir[rg]];
          kmn[rg] = kKeyPosInf;
          kmx[rg] = kKeyNegInf;
        }
        for (int g = 0; g < NG; ++g) {
          const int64_t cw = 1024 * (int64_t)g + 256 * wid;  // the wave's first column
          if (cw >= n) break;                                // uniform over the wave
          int64_t colc[4];  // MFMA A operand: lane l holds B[k][cw + 64 ch + l] (clamped)
#pragma unroll
          for (int ch = 0; ch < 4; ++ch) colc[ch] = cw + 64 * ch + lane < n ? cw + 64 * ch + lane : n - 1;
          v4f acc[4][RG];
#pragma unroll
          for (int ch = 0; ch < 4; ++ch)
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) acc[ch][rg] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          constexpr int KU = 4;
          float bc[KU][4], bn[KU][4];
#pragma unroll
          for (int kk = 0; kk < KU; ++kk)
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) bc[kk][ch] = B[(int64_t)(kk < r ? kk : r - 1) * n + colc[ch]];
          for (int k0 = 0; k0 < r; k0 += KU) {
#pragma unroll
            for (int kk = 0; kk < KU; ++kk) {
              const int k = k0 + KU + kk;
#pragma unroll
              for (int ch = 0; ch < 4; ++ch) bn[kk][ch] = B[(int64_t)(k < r ? k : r - 1) * n + colc[ch]];
            }
            float4 av[RG];  // MFMA B operand: lane 4b + q holds A[row 4 rg + q][k]
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) av[rg] = *reinterpret_cast<const float4*>(sA + (4 * rg + jr) * RP + k0);
#pragma unroll
            for (int kk = 0; kk < KU; ++kk) {
              if (k0 + kk < r) {  // uniform over the block
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
                  const float a = kk == 0 ? av[rg].x : kk == 1 ? av[rg].y : kk == 2 ? av[rg].z : av[rg].w;
#pragma unroll
                  for (int ch = 0; ch < 4; ++ch)
                    acc[ch][rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(bc[kk][ch], a, acc[ch][rg], 0, 0, 0);
                }
              }
            }
#pragma unroll
            for (int kk = 0; kk < KU; ++kk)
#pragma unroll
              for (int ch = 0; ch < 4; ++ch) bc[kk][ch] = bn[kk][ch];
          }
#pragma unroll
          for (int ch = 0; ch < 4; ++ch) {
            const int64_t j0 = cw + 64 * ch + 4 * bq;
            if (j0 >= n) continue;  // n % 4 == 0: the 4 columns are all inside or all outside
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              const int64_t i = ir[rg];
              const uint32_t cv = W4 ? (uint32_t)*reinterpret_cast<const uint16_t*>(wround + ((i * n + j0) >> 1))
                                     : *reinterpret_cast<const uint32_t*>(wround + i * n + j0);
              const U4 rnd = philox_block(((uint64_t)i * (uint64_t)n + (uint64_t)j0) >> 2, layer_id, seed);
              int w[4];
              float t[4], q[4];
              bool slow = false;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                w[e] = (W4 ? (int)((cv >> (4 * e)) & 15u) : (int)((cv >> (8 * e)) & 255u)) - zr[rg];
                const float rs = cr[rg] * aux_sample<DIST>(rnd, (unsigned)e, tab);
                t[e] = rs + acc[ch][rg][e];
                q[e] = div_small_int(t[e], (float)w[e], rcp[rcp_index(w[e])]);
                slow = slow || (w[e] != 0 && !div_small_int_ok(t[e]));
              }
              if (__builtin_amdgcn_ballot_w64(slow || !zero_point_ok(zr[rg])) != 0) {
                __asm__ volatile("");  // keeps the branch: the division is not speculated
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (w[e] != 0 && (!zero_point_ok(zr[rg]) || !div_small_int_ok(t[e]))) q[e] = t[e] / (float)w[e];
              }
              float uu[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                uu[e] = sr[rg] + q[e];
                if (okr[rg] && w[e] != 0) {
                  const int key = f32_key(uu[e]);
                  kmn[rg] = min(kmn[rg], key);
                  kmx[rg] = max(kmx[rg], key);
                }
              }
              *reinterpret_cast<float4*>(sU + (4 * rg + jr) * pitch + j0) = make_float4(uu[0], uu[1], uu[2], uu[3]);
            }
          }
        }
        // each row's range over the wave: lanes with the same q hold the same row
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          int a = kmn[rg], b = kmx[rg];
#pragma unroll
          for (int o = 4; o < 64; o <<= 1) {
            a = min(a, __shfl_xor(a, o, kWave));
            b = max(b, __shfl_xor(b, o, kWave));
          }
          if (lane < 4) {
            smin[wid][4 * rg + lane] = a;
            smax[wid][4 * rg + lane] = b;
          }
        }
        done = true;
      }
    }
    if (!done) {
      int kmin[RB], kmax[RB];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        kmin[rr] = kKeyPosInf;
        kmax[rr] = kKeyNegInf;
      }
      for (int g = 0; g < NG; ++g) {
        const int64_t j0 = 4 * ((int64_t)tid + 256 * g);
        if (j0 >= n) break;
        float acc[RB][4];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rr][e] = 0.0f;
        if (quad) {
          // B is read in chunks of KU rows, all loads of a chunk issued together and the
          // next chunk's issued before the current one's products, so the L2 latency is
          // paid once per chunk instead of once per k.  k is clamped to r - 1 so the
          // loads need no branch; a clamped k is never used.
          constexpr int KU = RB >= 8 ? 2 : RB >= 4 ? 4 : 8;  // shorter chunks where more rows share a load
          float4 bc[KU], bn[KU];
#pragma unroll
          for (int kk = 0; kk < KU; ++kk)
            bc[kk] = *reinterpret_cast<const float4*>(B + (int64_t)(kk < r ? kk : r - 1) * n + j0);
          for (int k0 = 0; k0 < r; k0 += KU) {
#pragma unroll
            for (int kk = 0; kk < KU; ++kk) {
              const int k = k0 + KU + kk;
              bn[kk] = *reinterpret_cast<const float4*>(B + (int64_t)(k < r ? k : r - 1) * n + j0);
            }
            // A[rows][k0 .. k0 + KU) with vector LDS reads (k0 is a multiple of KU, the
            // pitch a multiple of 4; entries past r are read but never used)
            float av[RB][KU];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
#pragma unroll
              for (int c = 0; c < KU; c += (KU >= 4 ? 4 : 2)) {
                if (KU >= 4) {
                  const float4 v = *reinterpret_cast<const float4*>(sA + rr * RP + k0 + c);
                  av[rr][c] = v.x;
                  av[rr][c + 1] = v.y;
                  av[rr][c + 2] = v.z;
                  av[rr][c + 3] = v.w;
                } else {
                  const float2 v = *reinterpret_cast<const float2*>(sA + rr * RP + k0 + c);
                  av[rr][c] = v.x;
                  av[rr][c + 1] = v.y;
                }
              }
            }
#pragma unroll
            for (int kk = 0; kk < KU; ++kk) {
              if (k0 + kk < r) {  // uniform over the block
                const float b[4] = {bc[kk].x, bc[kk].y, bc[kk].z, bc[kk].w};
#pragma unroll
                for (int rr = 0; rr < RB; ++rr)
#pragma unroll
                  for (int e = 0; e < 4; ++e) acc[rr][e] = fmaf(av[rr][kk], b[e], acc[rr][e]);
              }
            }
#pragma unroll
            for (int kk = 0; kk < KU; ++kk) bc[kk] = bn[kk];
          }
        } else {
          for (int k = 0; k < r; ++k) {
            float b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = j0 + e < n ? B[(int64_t)k * n + j0 + e] : 0.0f;
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
              const float a = sA[rr * RP + k];
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[rr][e] = fmaf(a, b[e], acc[rr][e]);
            }
          }
        }
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          const bool row_ok = i0 + rr < d;
          const int64_t i = row_ok ? i0 + rr : d - 1;  // a row past d is computed, never stored
          const int zi = z[i];
          const float ci = c[i], si = s[i];
          int w[4];
          float rs[4];
          if (quad) {
            const uint32_t cv = W4 ? (uint32_t)*reinterpret_cast<const uint16_t*>(wround + ((i * n + j0) >> 1))
                                   : *reinterpret_cast<const uint32_t*>(wround + i * n + j0);
            const U4 rnd = philox_block(((uint64_t)i * (uint64_t)n + (uint64_t)j0) >> 2, layer_id, seed);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] = (W4 ? (int)((cv >> (4 * e)) & 15u) : (int)((cv >> (8 * e)) & 255u)) - zi;
              rs[e] = ci * aux_sample<DIST>(rnd, (unsigned)e, tab);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int64_t j = j0 + e < n ? j0 + e : n - 1;
              w[e] = code_at<W4>(wround, i, n, j) - zi;
              rs[e] = rstar_element((uint64_t)i * (uint64_t)n + (uint64_t)j, ci, layer_id, seed, tab, DIST);
            }
          }
          float t[4], q[4];
          const bool zok = zero_point_ok(zi);
          bool slow = !zok;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            t[e] = rs[e] + acc[rr][e];
            q[e] = div_small_int(t[e], (float)w[e], rcp[rcp_index(w[e])]);
            slow = slow || (w[e] != 0 && !div_small_int_ok(t[e]));
          }
          if (__builtin_amdgcn_ballot_w64(slow) != 0) {
            __asm__ volatile("");  // keeps the branch: the division is not speculated
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (w[e] != 0 && (!zok || !div_small_int_ok(t[e]))) q[e] = t[e] / (float)w[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float uu = si + q[e];
            sU[rr * pitch + j0 + e] = uu;
            if (row_ok && w[e] != 0 && j0 + e < n) {
              const int key = f32_key(uu);
              kmin[rr] = min(kmin[rr], key);
              kmax[rr] = max(kmax[rr], key);
            }
          }
        }
      }
      // each row's range over the block (order keys)
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int a = wave_min_i32(kmin[rr]), b = wave_max_i32(kmax[rr]);
        if (lane == 0) {
          smin[wid][rr] = a;
          smax[wid][rr] = b;
        }
      }
    }
    __syncthreads();
    for (int rr = 0; rr < RB; ++rr) {
      if (i0 + rr >= d) break;
      const int64_t i = i0 + rr;
      const int a = min(min(smin[0][rr], smin[1][rr]), min(smin[2][rr], smin[3][rr]));
      const int b = max(max(smax[0][rr], smax[1][rr]), max(smax[2][rr], smax[3][rr]));
      const MulParams P = mul_params(key_f32(a), key_f32(b), qmax);
      const bool rs_ok = P.rsbar >= 0x1p-126f;
      if (tid == 0) {
        sbar_out[i] = P.sbar;
        zbar_out[i] = P.zbar;
      }
      const int zi = z[i];
      for (int g = 0; g < NG; ++g) {
        const int64_t j0 = 4 * ((int64_t)tid + 256 * g);
        if (j0 >= n) break;
        int w[4], ur[4], mm[4];
        float uu[4];
        bool redo[4], any = false;
        if (quad) {
          const uint32_t cv = W4 ? (uint32_t)*reinterpret_cast<const uint16_t*>(wround + ((i * n + j0) >> 1))
                                 : *reinterpret_cast<const uint32_t*>(wround + i * n + j0);
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (W4 ? (int)((cv >> (4 * e)) & 15u) : (int)((cv >> (8 * e)) & 255u)) - zi;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (j0 + e < n ? code_at<W4>(wround, i, n, j0 + e) : zi) - zi;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uu[e] = sU[rr * pitch + j0 + e];
          bool exact = true;
          ur[e] = w[e] != 0 ? mul_code_fast(uu[e], P, rs_ok, qmax, exact) : P.zbar;
          redo[e] = !exact;
          any = any || redo[e];
        }
        if (__builtin_amdgcn_ballot_w64(any) != 0) {
          __asm__ volatile("");
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (redo[e]) ur[e] = mul_code(uu[e], P.sbar, P.zbar, qmax);
        }
        int mx = -32768;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int mv = w[e] != 0 ? (ur[e] - P.zbar) * w[e] : 0;
          if (j0 + e < n) {
            if (mv > 32767) { mv = 32767; ++nsat; }
            if (mv < -32768) { mv = -32768; ++nsat; }
            mx = max(mx, mv);
          }
          mm[e] = mv;
        }
        if (quad) {
          store8(m + i * n + j0, make_uint2((uint32_t)(mm[0] & 0xFFFF) | ((uint32_t)mm[1] << 16),
                                                 (uint32_t)(mm[2] & 0xFFFF) | ((uint32_t)mm[3] << 16)));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j0 + e < n) m[i * n + j0 + e] = (int16_t)mm[e];
        }
        if (mx >= kSplitBiasMin) sflag[rr] = 1;
        if (uround_dbg) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j0 + e < n) uround_dbg[i * n + j0 + e] = (uint8_t)ur[e];
        }
      }
    }
    __syncthreads();
    if (split && tid < RB && i0 + tid < d) split[i0 + tid] = (uint8_t)sflag[tid];
  }
  add_saturations(sat, nsat);
}

__global__ void k_zero_u64(unsigned long long* p) { *p = 0ull; }

static dim3 quant_grid(int64_t d, int64_t n) {
  const int64_t groups = (d + kQRows - 1) / kQRows;
  return dim3((unsigned)((n + kQCols - 1) / kQCols), (unsigned)(groups < 65535 ? (groups ? groups : 1) : 65535));
}

hipError_t launch_mul_params(int64_t d, int ntiles, const int* pmin, const int* pmax, const float* umin_in,
                             const float* umax_in, float* umin_out, float* umax_out, int u_bits, int w_bits,
                             const int32_t* z, float* sbar, int32_t* zbar, float* rs, int* small, uint8_t* split,
                             bool planes, hipStream_t st) {
  hipLaunchKernelGGL(k_mul_params, dim3(range_blocks(d)), dim3(64 * kRangeWaves), 0, st, d, ntiles, pmin, pmax, umin_in,
                     umax_in, umin_out, umax_out, (1 << u_bits) - 1, (1 << w_bits) - 1, z, sbar, zbar, rs, small,
                     split, planes);
  return hipGetLastError();
}

hipError_t launch_quant_mul(int64_t d, int64_t n, int w_bits, int u_bits, const uint8_t* wround, const int32_t* z,
                            const float* U, const float* sbar, const int32_t* zbar, const float* rs,
                            const int* small, void* m, uint8_t* split, uint8_t* uround_dbg,
                            unsigned long long* sat, uint8_t* ucode, bool planes, hipStream_t st) {
  const dim3 grid = quant_grid(d, n);
  int16_t* m16 = static_cast<int16_t*>(m);
#define INTLORA_QMUL(W4, OUT)                                                                                   \
  hipLaunchKernelGGL((k_quant_mul<W4, OUT>), grid, dim3(kQThreads), 0, st, d, n, u_bits, wround, z, U, sbar, \
                     zbar, rs, small, m16, split, uround_dbg, sat, ucode)
  if (ucode) {
    if (w_bits == 4)
      INTLORA_QMUL(true, kOutCodes);
    else
      INTLORA_QMUL(false, kOutCodes);
  } else if (planes) {
    if (w_bits == 4)
      INTLORA_QMUL(true, kOutPlanes);
    else
      INTLORA_QMUL(false, kOutPlanes);
  } else {
    if (w_bits == 4)
      INTLORA_QMUL(true, kOutInt16);
    else
      INTLORA_QMUL(false, kOutInt16);
  }
#undef INTLORA_QMUL
  return hipGetLastError();
}

hipError_t launch_quant_ptq(int64_t d, int64_t n, int bits, const float* X, const float* xmin, const float* xmax,
                            uint8_t* code, float* s_out, int32_t* z_out, hipStream_t st) {
  const dim3 grid = quant_grid(d, n);
  if (bits == 4)
    hipLaunchKernelGGL(k_quant_ptq<true>, grid, dim3(kQThreads), 0, st, d, n, bits, X, xmin, xmax, code, s_out, z_out);
  else
    hipLaunchKernelGGL(k_quant_ptq<false>, grid, dim3(kQThreads), 0, st, d, n, bits, X, xmin, xmax, code, s_out,
                       z_out);
  return hipGetLastError();
}

hipError_t launch_quant_shift(int64_t d, int64_t n, int w_bits, int v_bits, const uint8_t* wround, const int32_t* z,
                              const float* U, const float* umin, const float* umax, uint8_t* m, float* sbar,
                              uint8_t* shift_dbg, unsigned long long* sat, hipStream_t st) {
  const dim3 grid = quant_grid(d, n);
  if (w_bits == 4)
    hipLaunchKernelGGL(k_quant_shift<true>, grid, dim3(kQThreads), 0, st, d, n, v_bits, wround, z, U, umin, umax, m,
                       sbar, shift_dbg, sat);
  else
    hipLaunchKernelGGL(k_quant_shift<false>, grid, dim3(kQThreads), 0, st, d, n, v_bits, wround, z, U, umin, umax, m,
                       sbar, shift_dbg, sat);
  return hipGetLastError();
}

template <int NG, bool W4, int DIST>
static hipError_t launch_fused_t(const AdaptArgs& a, dim3 grid, int u_bits, int16_t* m, float* sbar, int32_t* zbar,
                                 uint8_t* split, uint8_t* uround_dbg, unsigned long long* sat, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_merge_fused<NG, W4, DIST>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, FusedLds<NG>::MAX_BYTES);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_merge_fused<NG, W4, DIST>), grid, dim3(256), (unsigned)FusedLds<NG>::bytes(a.n, a.r), st, a.d,
                     a.n, a.r, u_bits, a.seed, a.layer_id, a.wround, a.z, a.s, a.c, a.A, a.B, m, sbar, zbar, split,
                     uround_dbg, sat);
  return hipSuccess;
}

template <int DIST>
static hipError_t launch_fused_d(const AdaptArgs& a, int ng, dim3 grid, int u_bits, int16_t* m, float* sbar,
                                 int32_t* zbar, uint8_t* split, uint8_t* uround_dbg, unsigned long long* sat,
                                 hipStream_t st) {
#define INTLORA_FUSED(NG)                                                                                      \
  return a.w_bits == 4 ? launch_fused_t<NG, true, DIST>(a, grid, u_bits, m, sbar, zbar, split, uround_dbg, sat, st) \
                       : launch_fused_t<NG, false, DIST>(a, grid, u_bits, m, sbar, zbar, split, uround_dbg, sat, st)
  switch (ng) {
    case 1: INTLORA_FUSED(1);
    case 2: INTLORA_FUSED(2);
    case 4: INTLORA_FUSED(4);
    case 8: INTLORA_FUSED(8);
    default: INTLORA_FUSED(16);
  }
#undef INTLORA_FUSED
}

// Fused MUL merge: NG = columns / 1024 rounded up to a power of two (n <= 16384).
hipError_t launch_merge_fused(const AdaptArgs& a, int u_bits, int16_t* m, float* sbar, int32_t* zbar,
                              uint8_t* split, uint8_t* uround_dbg, unsigned long long* sat, hipStream_t st) {
  int ng = 1;
  while (ng < 16 && (int64_t)ng * 1024 < a.n) ng *= 2;
  if ((int64_t)ng * 1024 < a.n) return hipErrorInvalidValue;
  const int rb = ng == 1 ? 8 : 16 / ng;
  const int64_t groups = (a.d + rb - 1) / rb;
  const dim3 grid((unsigned)(groups < 8192 ? (groups > 0 ? groups : 1) : 8192));
  if (sat) hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(1), 0, st, sat);
  hipError_t e;
  switch (a.dist) {
    case kAuxGauss: e = launch_fused_d<kAuxGauss>(a, ng, grid, u_bits, m, sbar, zbar, split, uround_dbg, sat, st); break;
    case kAuxCauchy: e = launch_fused_d<kAuxCauchy>(a, ng, grid, u_bits, m, sbar, zbar, split, uround_dbg, sat, st); break;
    case kAuxStudentT2:
      e = launch_fused_d<kAuxStudentT2>(a, ng, grid, u_bits, m, sbar, zbar, split, uround_dbg, sat, st);
      break;
    default: e = launch_fused_d<kAuxLaplace>(a, ng, grid, u_bits, m, sbar, zbar, split, uround_dbg, sat, st); break;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace intlora
