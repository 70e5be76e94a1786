// Straight-through backward of the IntLoRA fake-quant merge to the LoRA factors, for
// gfx950 ([IntLoRA notes] "two implementation variants": training back-propagates
// through the quantizers with the STE; "1. AQS": R takes no gradient).
//
// With G = dL/dW' and the mask M = [W_round - z != 0] (the merged weight is the
// constant 0 where w = 0), the gradient reaching AB is D = G (.) M, and
//   dA = D B^T  (d x r, a reduction over the n columns),
//   dB = A^T D  (r x n, a reduction over the d rows).
// Both products run on the matrix cores (v_mfma_f32_32x32x2_f32, fp32 accumulation).
// A lane feeds one element per instruction, so the two K values of an instruction are
// taken four columns (dA) or four rows (dB) apart, and a lane loads four consecutive
// elements at once; the reduction order is fixed by the launch geometry, which
// depends only on (d, n), so results are deterministic.
//
// dA: a block covers 32 rows over one of S column ranges; its 4 waves interleave
//     8-column steps and are summed through LDS in wave order.  dB: a block covers 128
//     columns (32 per wave) over one of S' row ranges.  With S (S') > 1 the partial
//     sums go to the workspace and k_ste_reduce adds them in range order.
#include "device_common.h"
#include "intlora_internal.h"

namespace intlora {

typedef float v16f __attribute__((ext_vector_type(16)));

namespace ste {
constexpr int kThreads = 256;
constexpr int kDaRows = 32;    // rows per dA block
constexpr int kDbCols = 128;   // columns per dB block (32 per wave)
constexpr int kTargetBlocks = 512;
}  // namespace ste

// code of element (i, j): uint8 codes or packed nibbles (low nibble = even column)
template <bool W4>
__device__ __forceinline__ int ste_code(const uint8_t* __restrict__ wround, int64_t i, int64_t n, int64_t j) {
  if (W4) {
    const uint8_t b = wround[(i * n + j) >> 1];
    return (j & 1) ? (b >> 4) : (b & 15);
  }
  return wround[i * n + j];
}

// dA partial sums.  Lane l of a wave holds row i0 + (l & 31); per 8-column step at
// jb it feeds columns jb + 4 (l >> 5) + t to MFMA t (t = 0..3), the B operand being
// B[k0 + (l & 31)][same column].  RT = 32-wide k tiles (r <= 32 RT).
template <int RT, bool W4>
__global__ __launch_bounds__(ste::kThreads) void k_ste_da(int64_t d, int64_t n, int r,
                                                         const uint8_t* __restrict__ wround,
                                                         const int32_t* __restrict__ z,
                                                         const float* __restrict__ B,
                                                         const float* __restrict__ G, float* __restrict__ out,
                                                         int64_t cols_per_split) {
  __shared__ float red[4][RT][16][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int li = lane & 31, hk = lane >> 5;
  const int64_t i0 = (int64_t)blockIdx.x * ste::kDaRows;
  const int64_t i = i0 + li;
  const bool row_ok = i < d;
  const int zi = row_ok ? z[i] : 0;
  const int64_t c_lo = (int64_t)blockIdx.y * cols_per_split;
  const int64_t c_hi = c_lo + cols_per_split < n ? c_lo + cols_per_split : n;
  const bool vec = (n & 7) == 0;  // rows 16-byte aligned; steps never straddle n
  v16f acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;
  for (int64_t jb = c_lo + 8 * wid; jb < c_hi; jb += 32) {
    const int64_t c = jb + 4 * hk;  // this lane's four columns c .. c + 3
    float dv[4] = {0.f, 0.f, 0.f, 0.f};
    if (row_ok) {
      if (vec && c + 3 < c_hi) {
        const float4 g4 = *reinterpret_cast<const float4*>(G + i * n + c);
        uint32_t codes;
        if (W4) {
          codes = *reinterpret_cast<const uint16_t*>(wround + ((i * n + c) >> 1));
        } else {
          codes = *reinterpret_cast<const uint32_t*>(wround + i * n + c);
        }
        const float g[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int code = W4 ? (int)((codes >> (4 * e)) & 15u) : (int)((codes >> (8 * e)) & 255u);
          dv[e] = code != zi ? g[e] : 0.0f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < c_hi && ste_code<W4>(wround, i, n, c + e) != zi) dv[e] = G[i * n + c + e];
      }
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int k = 32 * t + li;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (k < r) {
        if (vec && c + 3 < c_hi) {
          const float4 b4 = *reinterpret_cast<const float4*>(B + (int64_t)k * n + c);
          bv[0] = b4.x;
          bv[1] = b4.y;
          bv[2] = b4.z;
          bv[3] = b4.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < c_hi) bv[e] = B[(int64_t)k * n + c + e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(dv[e], bv[e], acc[t], 0, 0, 0);
    }
  }
  // sum the four waves in wave order
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wid][t][v][lane] = acc[t][v];
  __syncthreads();
  float* part = out + (int64_t)blockIdx.y * d * r;
  for (int p = threadIdx.x; p < RT * 32 * 32; p += ste::kThreads) {
    const int t = p / 1024, rem = p % 1024;
    const int Mr = rem / 32, N = rem % 32;  // output row in the tile, k in the tile
    const int v = 4 * (Mr / 8) + (Mr % 4), l = N + 32 * ((Mr / 4) % 2);
    const int64_t row = i0 + Mr;
    const int k = 32 * t + N;
    if (row < d && k < r) part[row * r + k] = ((red[0][t][v][l] + red[1][t][v][l]) + red[2][t][v][l]) + red[3][t][v][l];
  }
}

// dB partial sums.  Wave w covers columns j0 = 128 bx + 32 w + (l & 31); per 8-row
// step at ib lane l feeds rows ib + 4 (l >> 5) + t to MFMA t, the A operand being
// A[that row][k0 + (l & 31)].
template <int RT, bool W4>
__global__ __launch_bounds__(ste::kThreads) void k_ste_db(int64_t d, int64_t n, int r,
                                                         const uint8_t* __restrict__ wround,
                                                         const int32_t* __restrict__ z,
                                                         const float* __restrict__ A,
                                                         const float* __restrict__ G, float* __restrict__ out,
                                                         int64_t rows_per_split) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int li = lane & 31, hk = lane >> 5;
  const int64_t jw = (int64_t)blockIdx.x * ste::kDbCols + 32 * wid;
  const int64_t j = jw + li;
  const bool col_ok = j < n;
  const int64_t r_lo = (int64_t)blockIdx.y * rows_per_split;
  const int64_t r_hi = r_lo + rows_per_split < d ? r_lo + rows_per_split : d;
  v16f acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;
  for (int64_t ib = r_lo; ib < r_hi; ib += 8) {
    const int64_t rb = ib + 4 * hk;  // this lane's four rows rb .. rb + 3
    float dv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = rb + e;
      dv[e] = (col_ok && i < r_hi && ste_code<W4>(wround, i, n, j) != z[i]) ? G[i * n + j] : 0.0f;
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int k = 32 * t + li;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = rb + e;
        const float av = (k < r && i < r_hi) ? A[i * r + k] : 0.0f;
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, dv[e], acc[t], 0, 0, 0);
      }
    }
  }
  // lane l, register v: k = 32 t + 8 (v / 4) + 4 (l / 32) + v % 4, column jw + l % 32
  float* part = out + (int64_t)blockIdx.y * r * n;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = 32 * t + 8 * (v / 4) + 4 * hk + (v % 4);
      if (k < r && col_ok) part[(int64_t)k * n + j] = acc[t][v];
    }
}

// out[x] = sum over s = 0 .. S-1 of part[s][x], in that order.
__global__ __launch_bounds__(256) void k_ste_reduce(int64_t count, int S, const float* __restrict__ part,
                                                   float* __restrict__ out) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < count; x += (int64_t)gridDim.x * blockDim.x) {
    float s = part[x];
    for (int q = 1; q < S; ++q) s += part[(int64_t)q * count + x];
    out[x] = s;
  }
}

// Launch geometry (a pure function of d and n, so results do not depend on the device).
SteSplits ste_splits(int64_t d, int64_t n) {
  SteSplits sp;
  const int64_t row_tiles = (d + ste::kDaRows - 1) / ste::kDaRows;
  int64_t s = (ste::kTargetBlocks + row_tiles - 1) / row_tiles;
  int64_t smax = n / 256 > 1 ? n / 256 : 1;
  sp.S = (int)(s < 1 ? 1 : (s > smax ? smax : s));
  sp.cols_per_split = (((n + sp.S - 1) / sp.S) + 31) / 32 * 32;  // a multiple of the 32-column round
  sp.S = (int)((n + sp.cols_per_split - 1) / sp.cols_per_split);
  const int64_t col_groups = (n + ste::kDbCols - 1) / ste::kDbCols;
  int64_t s2 = (ste::kTargetBlocks + col_groups - 1) / col_groups;
  int64_t s2max = d / 64 > 1 ? d / 64 : 1;
  sp.S2 = (int)(s2 < 1 ? 1 : (s2 > s2max ? s2max : s2));
  sp.rows_per_split = (((d + sp.S2 - 1) / sp.S2) + 7) / 8 * 8;
  sp.S2 = (int)((d + sp.rows_per_split - 1) / sp.rows_per_split);
  return sp;
}

size_t ste_ws_bytes(int64_t d, int64_t n, int r) {
  const SteSplits sp = ste_splits(d, n);
  size_t b = 0;
  if (sp.S > 1) b += ((size_t)sp.S * d * r * 4 + 255) & ~size_t(255);
  if (sp.S2 > 1) b += ((size_t)sp.S2 * r * n * 4 + 255) & ~size_t(255);
  return b;
}

template <int RT, bool W4>
static void launch_ste_rt(int64_t d, int64_t n, int r, const uint8_t* wround, const int32_t* z, const float* A,
                          const float* B, const float* G, float* pa, float* pb, const SteSplits& sp, hipStream_t st) {
  hipLaunchKernelGGL((k_ste_da<RT, W4>), dim3((unsigned)((d + ste::kDaRows - 1) / ste::kDaRows), (unsigned)sp.S),
                     dim3(ste::kThreads), 0, st, d, n, r, wround, z, B, G, pa, sp.cols_per_split);
  hipLaunchKernelGGL((k_ste_db<RT, W4>), dim3((unsigned)((n + ste::kDbCols - 1) / ste::kDbCols), (unsigned)sp.S2),
                     dim3(ste::kThreads), 0, st, d, n, r, wround, z, A, G, pb, sp.rows_per_split);
}

hipError_t launch_ste_backward(int64_t d, int64_t n, int r, int w_bits, const uint8_t* wround, const int32_t* z,
                               const float* A, const float* B, const float* G, float* dA, float* dB, void* ws,
                               hipStream_t st) {
  const SteSplits sp = ste_splits(d, n);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* pa = dA;
  float* pb = dB;
  if (sp.S > 1) {
    pa = reinterpret_cast<float*>(p);
    p += ((size_t)sp.S * d * r * 4 + 255) & ~size_t(255);
  }
  if (sp.S2 > 1) pb = reinterpret_cast<float*>(p);
  const int rt = (r + 31) / 32;
#define INTLORA_STE(RT)                                                                  \
  do {                                                                                   \
    if (w_bits == 4)                                                                     \
      launch_ste_rt<RT, true>(d, n, r, wround, z, A, B, G, pa, pb, sp, st);             \
    else                                                                                 \
      launch_ste_rt<RT, false>(d, n, r, wround, z, A, B, G, pa, pb, sp, st);            \
  } while (0)
  switch (rt) {
    case 1: INTLORA_STE(1); break;
    case 2: INTLORA_STE(2); break;
    case 3: INTLORA_STE(3); break;
    default: INTLORA_STE(4); break;
  }
#undef INTLORA_STE
  if (sp.S > 1) {
    const int64_t cnt = d * (int64_t)r;
    hipLaunchKernelGGL(k_ste_reduce, dim3((unsigned)((cnt + 255) / 256 < 4096 ? (cnt + 255) / 256 : 4096)), dim3(256),
                       0, st, cnt, sp.S, pa, dA);
  }
  if (sp.S2 > 1) {
    const int64_t cnt = (int64_t)r * n;
    hipLaunchKernelGGL(k_ste_reduce, dim3((unsigned)((cnt + 255) / 256 < 4096 ? (cnt + 255) / 256 : 4096)), dim3(256),
                       0, st, cnt, sp.S2, pb, dB);
  }
  return hipGetLastError();
}

}  // namespace intlora
