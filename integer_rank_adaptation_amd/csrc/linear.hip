// Integer linear layer on IntLoRA merged integers for gfx950 (int8 MFMA).
//
// Y[t, i] = bf16( RN32( RN32( float(exact) * s_x[t] ) * s_bar[i] ) ),
// exact = sum_j X_q[t, j] * m[i, j].  The merged integers are the deployed weights
// (IntLoRA Paper-Notes, "training and inference efficiency": no PTQ after merging);
// activations use per-token scales, weights per-channel scales (SVDQuant article,
// "implementation details", 8-bit setting).
//
// Formats of m:
//   INT8  (SHIFT, b_W = 8)   one int8 plane;
//   INT4  (SHIFT, b_W = 4)   packed nibbles, unpacked on the way into LDS as 16*w
//                            (nibble placed in the high half of each byte), so the
//                            accumulator is 16 * exact and is shifted back exactly;
//   INT16 (MUL)              bias byte split on the way into LDS:
//                            hi = m >> 8, lo = (m & 0xFF) - 128, two int8 planes,
//                            exact = 256 acc_hi + acc_lo + 128 rowsum(X_q) (int64).
//
// Tiling: a 256-thread block (4 waves, 2 x 2) computes 256 tokens x 256 MFMA columns
// (256 outputs, or 128 outputs x 2 planes); each wave owns 128 x 128 = 4 x 4 tiles of
// v_mfma_i32_32x32x32_i8.  K advances 64 bytes per stage through a double-buffered LDS
// tile with a padded 80-byte row stride (conflict-free 16-byte fragment reads); the
// next stage's global loads are issued before the current stage's MFMAs.
#include "device_common.h"
#include "intlora_internal.h"

namespace intlora {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

namespace lin {
constexpr int BM = 256;
constexpr int BNC = 256;
constexpr int BK = 64;
constexpr int STRIDE = BK + 16;
constexpr int TILE_A = BM * STRIDE;
constexpr int TILE_B = BNC * STRIDE;
constexpr int STAGE = TILE_A + TILE_B;
constexpr int LDS_BYTES = 2 * STAGE;
}  // namespace lin

enum { F_INT4 = 4, F_INT8 = 8, F_INT16 = 16 };

template <int F>
struct BStage {
  v4i r[4];
};

// Global -> registers for one K stage.
template <int F>
__device__ __forceinline__ void load_stage(int kt, int64_t M, int64_t d, int64_t n, int64_t t0, int64_t o0,
                                           const int8_t* __restrict__ xq, const uint8_t* __restrict__ m, v4i (&ra)[4],
                                           v4i (&rb)[4]) {
  using namespace lin;
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = (tid >> 2) + 64 * p;
    const int64_t kb = k0 + (tid & 3) * 16;
    v4i v = {0, 0, 0, 0};
    if (t0 + row < M && kb < n) v = *reinterpret_cast<const v4i*>(xq + (t0 + row) * n + kb);
    ra[p] = v;
  }
  if (F == F_INT8) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = (tid >> 2) + 64 * p;
      const int64_t kb = k0 + (tid & 3) * 16;
      v4i v = {0, 0, 0, 0};
      if (o0 + row < d && kb < n) v = *reinterpret_cast<const v4i*>(m + (o0 + row) * n + kb);
      rb[p] = v;
    }
  } else if (F == F_INT16) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = (tid >> 3) + 32 * p;        // output row 0..127
      const int64_t ke = k0 + (tid & 7) * 8;      // first K element of the chunk
      v4i v = {0, 0, 0, 0};
      if (o0 + row < d && ke < n) v = *reinterpret_cast<const v4i*>(m + ((o0 + row) * n + ke) * 2);
      rb[p] = v;
    }
  } else {  // F_INT4
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int row = (tid >> 1) + 128 * p;       // output row 0..255
      const int64_t ke = k0 + (tid & 1) * 32;     // first K element of the 32-element chunk
      v4i v = {0, 0, 0, 0};
      if (o0 + row < d && ke < n) v = *reinterpret_cast<const v4i*>(m + (o0 + row) * (n >> 1) + (ke >> 1));
      rb[p] = v;
    }
  }
}

// Registers -> LDS (with the INT4 unpack / INT16 byte split).
template <int F>
__device__ __forceinline__ void store_stage(uint8_t* __restrict__ st, const v4i (&ra)[4], const v4i (&rb)[4]) {
  using namespace lin;
  const int tid = threadIdx.x;
  uint8_t* As = st;
  uint8_t* Bs = st + TILE_A;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = (tid >> 2) + 64 * p;
    *reinterpret_cast<v4i*>(As + row * STRIDE + (tid & 3) * 16) = ra[p];
  }
  if (F == F_INT8) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = (tid >> 2) + 64 * p;
      *reinterpret_cast<v4i*>(Bs + row * STRIDE + (tid & 3) * 16) = rb[p];
    }
  } else if (F == F_INT16) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = (tid >> 3) + 32 * p;
      const int hrow = 64 * (row >> 5) + (row & 31);  // hi plane block 2q, lo plane block 2q+1
      const int kb = (tid & 7) * 8;
      const uint32_t x0 = (uint32_t)rb[p].x, x1 = (uint32_t)rb[p].y, x2 = (uint32_t)rb[p].z, x3 = (uint32_t)rb[p].w;
      // little-endian int16 pairs: high bytes are bytes 1, 3 of each dword
      uint2 hi, lo;
      hi.x = __builtin_amdgcn_perm(x1, x0, 0x07050301u);
      hi.y = __builtin_amdgcn_perm(x3, x2, 0x07050301u);
      lo.x = __builtin_amdgcn_perm(x1, x0, 0x06040200u) ^ 0x80808080u;
      lo.y = __builtin_amdgcn_perm(x3, x2, 0x06040200u) ^ 0x80808080u;
      *reinterpret_cast<uint2*>(Bs + hrow * STRIDE + kb) = hi;
      *reinterpret_cast<uint2*>(Bs + (hrow + 32) * STRIDE + kb) = lo;
    }
  } else {  // F_INT4: 16 packed bytes -> 32 int8 holding 16 * w
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int row = (tid >> 1) + 128 * p;
      const int kb = (tid & 1) * 32;
      const uint32_t xs[4] = {(uint32_t)rb[p].x, (uint32_t)rb[p].y, (uint32_t)rb[p].z, (uint32_t)rb[p].w};
      uint32_t o[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t H = xs[q] & 0xF0F0F0F0u;          // odd columns, already x16
        const uint32_t L = (xs[q] << 4) & 0xF0F0F0F0u;   // even columns, x16
        o[2 * q] = __builtin_amdgcn_perm(H, L, 0x05010400u);
        o[2 * q + 1] = __builtin_amdgcn_perm(H, L, 0x07030602u);
      }
      v4i w0 = {(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
      v4i w1 = {(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
      *reinterpret_cast<v4i*>(Bs + row * STRIDE + kb) = w0;
      *reinterpret_cast<v4i*>(Bs + row * STRIDE + kb + 16) = w1;
    }
  }
}

template <int F>
__global__ __launch_bounds__(256, 1) void k_linear(int64_t M, int64_t d, int64_t n, const int8_t* __restrict__ xq,
                                                  const float* __restrict__ sx, const int32_t* __restrict__ rowsum,
                                                  const uint8_t* __restrict__ m, const float* __restrict__ sbar,
                                                  uint16_t* __restrict__ Y, int32_t* __restrict__ acc_dbg,
                                                  int tiles_m, int tiles_n) {
  using namespace lin;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  constexpr int OUT_PER_BLOCK = (F == F_INT16) ? 128 : 256;

  // Blocks are dealt round-robin to the 8 XCDs; renumber so that each XCD receives a
  // contiguous range of tiles, walked M-fastest (consecutive tiles share the weight
  // tile, and the token tiles they cycle through stay in that XCD's L2).
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  {
    const int per = nblk / 8, rem = nblk % 8;
    const int x = bid % 8, loc = bid / 8;
    const int base = x * per + (x < rem ? x : rem);
    if (loc < per + (x < rem ? 1 : 0)) bid = base + loc;
  }
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int64_t t0 = (int64_t)tm * BM;
  const int64_t o0 = (int64_t)tn * OUT_PER_BLOCK;

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int KT = (int)((n + BK - 1) / BK);
  v4i ra[4], rb[4];
  load_stage<F>(0, M, d, n, t0, o0, xq, m, ra, rb);
  store_stage<F>(lds, ra, rb);
  __syncthreads();

  const int frag_row = lane & 31, frag_k = (lane >> 5) * 16;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage<F>(kt + 1, M, d, n, t0, o0, xq, m, ra, rb);
    const uint8_t* As = lds + cur * STAGE;
    const uint8_t* Bs = As + TILE_A;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const v4i*>(As + (wm * 128 + i * 32 + frag_row) * STRIDE + ks * 32 + frag_k);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const v4i*>(Bs + (wn * 128 + j * 32 + frag_row) * STRIDE + ks * 32 + frag_k);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_stage<F>(lds + (cur ^ 1) * STAGE, ra, rb);
    __syncthreads();
  }

  // Epilogue through LDS, one 32-row slab (i) at a time: each wave parks its 32 x 128
  // int32 accumulators in its own 16 KB region, then reads them back row-wise so
  // that every lane owns whole outputs and the bf16 stores are contiguous.
  // Lane l, register r of a 32x32 tile hold token row 8(r/4) + 4(l/32) + r%4 and
  // column l%32 of that tile.
  __syncthreads();
  int32_t* R = reinterpret_cast<int32_t*>(lds) + wid * (32 * 128);
  const int col_in = lane & 31;
  const int row_hi = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) R[(8 * (r >> 2) + row_hi + (r & 3)) * 128 + j * 32 + col_in] = acc[i][j][r];
    __syncthreads();
    const int64_t tok_base = t0 + wm * 128 + i * 32;
    if (F == F_INT16) {
      // region columns: [hi 0..31 | lo 0..31 | hi 32..63 | lo 32..63] of the wave's 64 outputs
      const int half = lane >> 5;
      for (int rr = 0; rr < 32; rr += 2) {
        const int row = rr + half;
        const int64_t tok = tok_base + row;
        if (tok < M) {
          const int64_t rs128 = 128 * (int64_t)rowsum[tok];
          const float sxt = sx[tok];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int64_t col = o0 + wn * 64 + q * 32 + col_in;
            if (col < d) {
              const int ahi = R[row * 128 + q * 64 + col_in];
              const int alo = R[row * 128 + q * 64 + 32 + col_in];
              const int64_t exact = 256 * (int64_t)ahi + (int64_t)alo + rs128;
              float y = (float)(double)exact;
              y = y * sxt;
              y = y * sbar[col];
              Y[tok * d + col] = bf16_rne(y);
              if (acc_dbg) {
                acc_dbg[tok * d + col] = ahi;
                acc_dbg[M * d + tok * d + col] = alo;
              }
            }
          }
        }
      }
    } else {
      for (int rr = 0; rr < 32; ++rr) {
        const int64_t tok = tok_base + rr;
        if (tok < M) {
          const float sxt = sx[tok];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int c = 2 * lane + q;
            const int64_t col = o0 + wn * 128 + c;
            if (col < d) {
              const int a = R[rr * 128 + c];
              const int exact = (F == F_INT4) ? (a >> 4) : a;
              float y = (float)exact;
              y = y * sxt;
              y = y * sbar[col];
              Y[tok * d + col] = bf16_rne(y);
              if (acc_dbg) acc_dbg[tok * d + col] = exact;
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_linear(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx, const int32_t* rowsum,
                         int wfmt, const void* m, const float* sbar, uint16_t* Y, int32_t* acc_dbg, hipStream_t st) {
  using namespace lin;
  const int out_per_block = (wfmt == F_INT16) ? 128 : 256;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((d + out_per_block - 1) / out_per_block);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const uint8_t* mb = static_cast<const uint8_t*>(m);
  static bool attr_set = false;
  if (!attr_set) {
    const void* fns[3] = {reinterpret_cast<const void*>(&k_linear<F_INT8>), reinterpret_cast<const void*>(&k_linear<F_INT4>),
                          reinterpret_cast<const void*>(&k_linear<F_INT16>)};
    for (const void* f : fns) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  switch (wfmt) {
    case F_INT8:
      hipLaunchKernelGGL(k_linear<F_INT8>, grid, dim3(256), LDS_BYTES, st, M, d, n, xq, sx, rowsum, mb, sbar, Y,
                         acc_dbg, tiles_m, tiles_n);
      break;
    case F_INT4:
      hipLaunchKernelGGL(k_linear<F_INT4>, grid, dim3(256), LDS_BYTES, st, M, d, n, xq, sx, rowsum, mb, sbar, Y,
                         acc_dbg, tiles_m, tiles_n);
      break;
    default:
      hipLaunchKernelGGL(k_linear<F_INT16>, grid, dim3(256), LDS_BYTES, st, M, d, n, xq, sx, rowsum, mb, sbar, Y,
                         acc_dbg, tiles_m, tiles_n);
      break;
  }
  return hipGetLastError();
}

}  // namespace intlora
