// Straight-through backward of the IntLoRA fake-quant merge to the LoRA factors, for
// gfx950 ([IntLoRA notes] "two implementation variants": training back-propagates
// through the quantizers with the STE; "1. AQS": R takes no gradient).
//
// With G = dL/dW' and the mask M = [W_round - z != 0] (the merged weight is the
// constant 0 where w = 0), the gradient reaching AB is D = G (.) M, and
//   dA = D B^T  (d x r, a reduction over the n columns),
//   dB = A^T D  (r x n, a reduction over the d rows).
//
// One fused kernel reads G and the codes once.  A block owns a chunk of 256 columns
// and a range of rows, walked in tiles of 32 rows: each tile of D is loaded with
// coalesced 16-byte row reads, masked and staged in LDS, and feeds both products on
// the matrix cores (v_mfma_f32_32x32x2_f32, fp32 accumulation):
//   - dA: each wave takes 64 of the 256 columns (its slice of B held in registers for
//     the whole walk); the four waves' 32 x r sums are added in wave order and written
//     per (column chunk, row tile);
//   - dB: each wave accumulates r x 64 (its columns) over all of the block's row
//     tiles, written per (row range, column chunk).
// k_ste_reduce then adds the column chunks (dA) and the row ranges (dB) in order.
// The launch geometry depends only on (d, n, r), so results are deterministic.
#include "device_common.h"
#include "intlora_internal.h"

namespace intlora {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace ste {
constexpr int kThreads = 256;
constexpr int kRows = 32;          // rows per tile
constexpr int kCols = 256;         // columns per block (64 per wave)
constexpr int kPitch = kCols + 4;  // LDS row pitch of the D tile (floats)
// Blocks resident at once on 256 compute units: two per unit for one k tile (about
// 200 registers a lane), one for more.  The grid is sized to fill them in one round.
constexpr int kSlots1 = 512;
constexpr int kSlotsN = 256;
}  // namespace ste

// LDS of a block with RT 32-wide k tiles (r <= 32 RT): the D tile, A's rows of the
// tile, and the dA cross-wave buffer (one tile behind: written after a tile's
// products, added and stored while the next tile's run).
template <int RT>
struct SteLds {
  static constexpr int D = ste::kRows * ste::kPitch;  // floats
  static constexpr int A = ste::kRows * 32 * RT;      // floats, [row][k]
  static constexpr int RED = 4 * RT * 16 * 64;        // floats
  static constexpr int BYTES = 4 * (D + A + RED);
};

// FAST: every column of the block's chunk is inside the matrix and rows are made of
// 16-byte aligned quads (n % 4 == 0): loads need no per-element test.  The blocks of
// one launch take column chunks chunk0 + blockIdx.x.
template <int RT, bool W4, bool FAST>
__global__ __launch_bounds__(ste::kThreads) void k_ste(int64_t d, int64_t n, int r,
                                                      const uint8_t* __restrict__ wround,
                                                      const int32_t* __restrict__ z, const float* __restrict__ A,
                                                      const float* __restrict__ B, const float* __restrict__ G,
                                                      float* __restrict__ pa, float* __restrict__ pb,
                                                      int64_t rows_per_split, int64_t chunk0) {
  using namespace ste;
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* sD = sm;
  float* sA = sD + SteLds<RT>::D;
  float* sR = sA + SteLds<RT>::A;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hk = lane >> 5;
  const int64_t chunk = chunk0 + blockIdx.x;
  const int64_t c0 = chunk * kCols;
  const int64_t r_lo = (int64_t)blockIdx.y * rows_per_split;
  const int64_t r_hi = r_lo + rows_per_split < d ? r_lo + rows_per_split : d;

  v16f accB[RT][2];  // dB: k tile t, column tile q (32 columns) of this wave
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int v = 0; v < 16; ++v) accB[t][q][v] = 0.0f;

  // A tile's loads, all issued before any is used (no branch between them): wave wid
  // takes rows wid + 4 yy of the tile, lane the columns c0 + 4 lane .. + 3 (G, their
  // codes, the row's zero point), and 4 RT values of A's rows.  Row indices are clamped
  // into the block's range; rows past it, and A's entries past r, are zeroed when the
  // tile is staged in LDS.  The element path (not FAST) masks columns past n on load
  // and sets the zero point to -1, which no code equals.  (Holding the next tile in
  // registers during the products was measured slower: the other block on the compute
  // unit covers the load latency.)
  constexpr int AQ = 4 * RT;
  float4 pg[8];
  uint32_t pc[8];
  int pz[8];
  float pa_[AQ];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int yy = 0; yy < 8; ++yy) {
      int64_t i = t0 + wid + 4 * yy;
      i = i < r_hi ? i : r_hi - 1;
      const int64_t c = c0 + 4 * lane;
      if (FAST) {
        pz[yy] = z[i];
        const v4f g4 = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(G + i * n + c));
        pg[yy] = make_float4(g4.x, g4.y, g4.z, g4.w);
        if (W4)
          pc[yy] = *reinterpret_cast<const uint16_t*>(wround + ((i * n + c) >> 1));
        else
          pc[yy] = *reinterpret_cast<const uint32_t*>(wround + i * n + c);
      } else {
        const int zi = z[i];
        float dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t j = c + e;
          const int64_t jc = j < n ? j : n - 1;
          const int code = W4 ? ((wround[(i * n + jc) >> 1] >> (4 * (jc & 1))) & 15) : wround[i * n + jc];
          const float g = G[i * n + jc];
          dv[e] = (j < n && code != zi) ? g : 0.0f;
        }
        pg[yy] = make_float4(dv[0], dv[1], dv[2], dv[3]);
        pc[yy] = 0;
        pz[yy] = -1;
      }
    }
#pragma unroll
    for (int u = 0; u < AQ; ++u) {
      const int x = tid + kThreads * u;
      const int y = x / (32 * RT), k = x % (32 * RT);
      int64_t i = t0 + y;
      i = i < r_hi ? i : r_hi - 1;
      pa_[u] = A[i * r + (k < r ? k : r - 1)];
    }
  };

  // dA of the tile at t0: the four waves' sums in the dA buffer, added in wave order,
  // written as the partial of (column chunk, rows).  Lane l, register v of a wave's
  // 32 x 32 block hold row 8 (v / 4) + 4 (l / 32) + v % 4 and k l % 32.
  auto flush_dA = [&](int64_t t0) {
    float* part = pa + chunk * d * r;
#pragma unroll
    for (int u = 0; u < 4 * RT; ++u) {
      const int p = tid + kThreads * u;
      const int t = p / 1024, rem = p % 1024;
      const int Mr = rem / 32, N = rem % 32;  // row in the tile, k in the tile
      const int v = 4 * (Mr / 8) + (Mr % 4), l = N + 32 * ((Mr / 4) % 2);
      const int64_t row = t0 + Mr;
      const int k = 32 * t + N;
      if (row < r_hi && k < r) {
        const float s0 = sR[((0 * RT + t) * 16 + v) * 64 + l], s1 = sR[((1 * RT + t) * 16 + v) * 64 + l];
        const float s2 = sR[((2 * RT + t) * 16 + v) * 64 + l], s3 = sR[((3 * RT + t) * 16 + v) * 64 + l];
        part[row * r + k] = ((s0 + s1) + s2) + s3;
      }
    }
  };


  // dA's B operand for every MFMA of the walk (loaded after the first tile's fetch is
  // in flight): step s8 (8 columns), MFMA e, k tile t -> B[32 t + li][c0 + 64 wid +
  // 8 s8 + 4 hk + e], zero past r and past n; a FAST block reads each step's four
  // columns as one 16-byte load.
  float bv[RT][8][4];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int k = 32 * t + li;
    const int64_t kc = k < r ? k : r - 1;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const int64_t j0 = c0 + 64 * wid + 8 * s8 + 4 * hk;
      if (FAST) {
        const v4f b4 = *reinterpret_cast<const v4f*>(B + kc * n + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[t][s8][e] = k < r ? b4[e] : 0.0f;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t j = j0 + e;
          const float v = B[kc * n + (j < n ? j : n - 1)];
          bv[t][s8][e] = (k < r && j < n) ? v : 0.0f;
        }
      }
    }
  }
  for (int64_t i0 = r_lo; i0 < r_hi; i0 += kRows) {
    __syncthreads();  // the previous tile's D and A reads and dA buffer writes are done
    fetch(i0);
#pragma unroll
    for (int yy = 0; yy < 8; ++yy) {
      const float g[4] = {pg[yy].x, pg[yy].y, pg[yy].z, pg[yy].w};
      float dv[4];
      const bool row_ok = i0 + wid + 4 * yy < r_hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int code = W4 ? (int)((pc[yy] >> (4 * e)) & 15u) : (int)((pc[yy] >> (8 * e)) & 255u);
        dv[e] = (row_ok && code != pz[yy]) ? g[e] : 0.0f;
      }
      *reinterpret_cast<float4*>(sD + (wid + 4 * yy) * kPitch + 4 * lane) = make_float4(dv[0], dv[1], dv[2], dv[3]);
    }
#pragma unroll
    for (int u = 0; u < AQ; ++u) {
      const int x = tid + kThreads * u;
      const int y = x / (32 * RT), k = x % (32 * RT);
      sA[x] = (i0 + y < r_hi && k < r) ? pa_[u] : 0.0f;
    }
    __syncthreads();
    if (i0 > r_lo) flush_dA(i0 - kRows);

    // dA over this wave's 64 columns: MFMA e of step s8 takes columns 8 s8 + 4 hk + e
    // (A operand D[li][column], B operand B[32 t + li][column])
    v16f accA[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) accA[t][v] = 0.0f;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const float4 d4 = *reinterpret_cast<const float4*>(sD + li * kPitch + 64 * wid + 8 * s8 + 4 * hk);
      const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          accA[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(dvv[e], bv[t][s8][e], accA[t], 0, 0, 0);
    }
    // dB: column tile q (columns 64 wid + 32 q + li); MFMA e of an 8-row step takes row
    // rs + 4 hk + e (A operand A[row][32 t + li], B operand D[row][column])
#pragma unroll
    for (int rs = 0; rs < kRows; rs += 8) {
      const int rb = rs + 4 * hk;
      float av[RT][4];
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) av[t][e] = sA[(rb + e) * 32 * RT + 32 * t + li];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float dq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dq[e] = sD[(rb + e) * kPitch + 64 * wid + 32 * q + li];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            accB[t][q] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[t][e], dq[e], accB[t][q], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave has read the dA buffer (the flush above)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) sR[((wid * RT + t) * 16 + v) * 64 + lane] = accA[t][v];
  }
  __syncthreads();
  flush_dA(r_lo + ((r_hi - r_lo - 1) / kRows) * kRows);
  // dB partial of (row range, column chunk): lane l, register v -> k = 32 t + 8 (v / 4) +
  // 4 (l / 32) + v % 4, column c0 + 64 wid + 32 q + l % 32
  float* part = pb + (int64_t)blockIdx.y * r * n;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t j = c0 + 64 * wid + 32 * q + li;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int k = 32 * t + 8 * (v / 4) + 4 * hk + (v % 4);
        if (k < r && j < n) part[(int64_t)k * n + j] = accB[t][q][v];
      }
    }
}

// out[x] = sum over s = 0 .. S-1 of part[s][x], in that order (loads issued eight at
// a time, the additions in sequence).
__global__ __launch_bounds__(256) void k_ste_reduce(int64_t count, int S, const float* __restrict__ part,
                                                   float* __restrict__ out) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < count; x += (int64_t)gridDim.x * blockDim.x) {
    float s = part[x];
    int q = 1;
    for (; q + 8 <= S; q += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(q + u) * count + x];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; q < S; ++q) s += part[(int64_t)q * count + x];
    out[x] = s;
  }
}

// Launch geometry, a pure function of (d, n, r): column chunks of 256, and row ranges
// (whole 32-row tiles) so that the chunks times the ranges fit the resident blocks in
// one round.
SteSplits ste_splits(int64_t d, int64_t n, int r) {
  SteSplits sp;
  sp.S = (int)((n + ste::kCols - 1) / ste::kCols);
  sp.cols_per_split = ste::kCols;
  const int64_t slots = r <= 32 ? ste::kSlots1 : ste::kSlotsN;
  int64_t s2 = slots / sp.S;
  const int64_t tiles = (d + ste::kRows - 1) / ste::kRows;
  if (s2 > tiles) s2 = tiles;
  if (s2 < 1) s2 = 1;
  sp.rows_per_split = ((tiles + s2 - 1) / s2) * ste::kRows;
  sp.S2 = (int)((d + sp.rows_per_split - 1) / sp.rows_per_split);
  if (sp.S2 < 1) sp.S2 = 1;
  return sp;
}

size_t ste_ws_bytes(int64_t d, int64_t n, int r) {
  const SteSplits sp = ste_splits(d, n, r);
  size_t b = 0;
  if (sp.S > 1) b += ((size_t)sp.S * d * r * 4 + 255) & ~size_t(255);
  if (sp.S2 > 1) b += ((size_t)sp.S2 * r * n * 4 + 255) & ~size_t(255);
  return b;
}

template <int RT, bool W4, bool FAST>
static hipError_t launch_ste_part(int64_t d, int64_t n, int r, const uint8_t* wround, const int32_t* z,
                                  const float* A, const float* B, const float* G, float* pa, float* pb,
                                  const SteSplits& sp, int64_t chunk0, int64_t chunks, hipStream_t st) {
  if (chunks <= 0) return hipSuccess;
  if (SteLds<RT>::BYTES > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ste<RT, W4, FAST>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, SteLds<RT>::BYTES);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_ste<RT, W4, FAST>), dim3((unsigned)chunks, (unsigned)sp.S2), dim3(ste::kThreads),
                     SteLds<RT>::BYTES, st, d, n, r, wround, z, A, B, G, pa, pb, sp.rows_per_split, chunk0);
  return hipGetLastError();
}

// Column chunks whose 256 columns are all inside rows of aligned quads take the FAST
// kernel; the rest (the ragged last chunk, or every chunk when n % 4 != 0) the element
// path.
template <int RT, bool W4>
static hipError_t launch_ste_rt(int64_t d, int64_t n, int r, const uint8_t* wround, const int32_t* z,
                                const float* A, const float* B, const float* G, float* pa, float* pb,
                                const SteSplits& sp, hipStream_t st) {
  const int64_t fast = (n & 3) == 0 ? n / ste::kCols : 0;
  const hipError_t e = launch_ste_part<RT, W4, true>(d, n, r, wround, z, A, B, G, pa, pb, sp, 0, fast, st);
  if (e != hipSuccess) return e;
  return launch_ste_part<RT, W4, false>(d, n, r, wround, z, A, B, G, pa, pb, sp, fast, sp.S - fast, st);
}

hipError_t launch_ste_backward(int64_t d, int64_t n, int r, int w_bits, const uint8_t* wround, const int32_t* z,
                               const float* A, const float* B, const float* G, float* dA, float* dB, void* ws,
                               hipStream_t st) {
  const SteSplits sp = ste_splits(d, n, r);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* pa = dA;
  float* pb = dB;
  if (sp.S > 1) {
    pa = reinterpret_cast<float*>(p);
    p += ((size_t)sp.S * d * r * 4 + 255) & ~size_t(255);
  }
  if (sp.S2 > 1) pb = reinterpret_cast<float*>(p);
  const int rt = (r + 31) / 32;
  hipError_t e;
#define INTLORA_STE(RT) \
  e = w_bits == 4 ? launch_ste_rt<RT, true>(d, n, r, wround, z, A, B, G, pa, pb, sp, st) \
                  : launch_ste_rt<RT, false>(d, n, r, wround, z, A, B, G, pa, pb, sp, st)
  switch (rt) {
    case 1: INTLORA_STE(1); break;
    case 2: INTLORA_STE(2); break;
    case 3: INTLORA_STE(3); break;
    default: INTLORA_STE(4); break;
  }
#undef INTLORA_STE
  if (e != hipSuccess) return e;
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
