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
//   INT4  (SHIFT, b_W = 4)   packed nibbles, unpacked after the LDS read as 16*w
//                            (nibble in the high half of each byte), so the
//                            accumulator is 16 * exact and is shifted back exactly;
//   INT16 (MUL)              bias byte split after the LDS read:
//                            hi = m >> 8, lo = (m & 0xFF) - 128, two int8 planes,
//                            exact = 256 acc_hi + acc_lo + 128 rowsum(X_q) (int64).
//
// Data path: every operand goes from HBM straight into LDS with buffer_load ... lds
// (16 bytes per lane, no VGPR staging) through a 3-stage ring, so the loads of stage
// k+2 are in flight while stage k computes.  Out-of-range rows and K chunks read as
// zero through the buffer descriptor.  LDS rows are XOR-swizzled in 16-byte chunks
// (conflict-free fragment reads); the swizzle is realized by the global address each
// lane fetches, since a direct load writes lane l's 16 bytes at base + 16 l.
//
// Tiling: a 256-thread block (4 waves, 2 x 2) computes 256 tokens x 128 MFMA columns
// (128 outputs, or 64 outputs x 2 planes); each wave owns 128 x 64 = 4 x 2 tiles of
// v_mfma_i32_32x32x32_i8 with the weight fragment as the A operand, so a lane's four
// consecutive accumulators are four consecutive outputs of one token.  Two blocks
// share a CU; one block's barrier overlaps the other's MFMAs.
#include "device_common.h"
#include "intlora_internal.h"

namespace intlora {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

enum { F_INT4 = 4, F_INT8 = 8, F_INT16 = 16 };

namespace lin {
constexpr int kThreads = 256;
constexpr int BM = 256;        // tokens per block
constexpr int BK = 64;         // K elements per stage
constexpr int kStages = 3;
constexpr int kGroupM = 8;     // token tiles per group of the tile order (L2 reuse)
constexpr int A_BYTES = BM * BK;                // 16 KB
constexpr int B_BYTES_8 = 128 * BK;             // 8 KB: 128 output rows x 64 int8
constexpr int B_BYTES_16 = 64 * BK * 2;         // 8 KB: 64 output rows x 64 int16
constexpr int B_BYTES_4 = 128 * BK / 2;         // 4 KB: 128 output rows x 64 nibbles
template <int F>
struct Cfg {
  static constexpr int B_BYTES = F == F_INT16 ? B_BYTES_16 : (F == F_INT8 ? B_BYTES_8 : B_BYTES_4);
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = kStages * STAGE;
  static constexpr int OUT = F == F_INT16 ? 64 : 128;          // outputs per block
  static constexpr int A_LOADS = A_BYTES / 1024 / 4;           // direct loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / 4;
  static constexpr int LOADS = A_LOADS + B_LOADS;
};
}  // namespace lin

// XOR swizzles of the 16-byte chunks of an LDS row (chosen so that the 16 or 8 lanes
// served together by a ds_read_b128 hit distinct banks, for 64- or 32-bank LDS).
__device__ __forceinline__ int swz64(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }   // 64-byte rows
__device__ __forceinline__ int swz128(int row) { return (row ^ (row >> 3)) & 7; }        // 128-byte rows
__device__ __forceinline__ int swz32(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }   // 32-byte rows

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;  // offsets stay below 2^31; larger tensors get a per-tile base
  const int nrec = (int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every record: the lane reads zeros

// Issue the direct loads of one K stage into one LDS stage buffer.
template <int F>
__device__ __forceinline__ void issue_stage(int kt, int64_t n, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                            uint8_t* stage) {
  using namespace lin;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t k0 = (int64_t)kt * BK;
  // A (tokens): 16 rows of 64 bytes per direct load
#pragma unroll
  for (int q = 0; q < Cfg<F>::A_LOADS; ++q) {
    const int g = wid * Cfg<F>::A_LOADS + q;
    const int row = 16 * g + (lane >> 2);
    const int c = (lane & 3) ^ swz64(row);
    const int64_t kb = k0 + 16 * c;
    const uint32_t off = kb < n ? (uint32_t)(row * n + kb) : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + g * 1024), 16, off, 0, 0, 0);
  }
  uint8_t* Bs = stage + A_BYTES;
  if (F == F_INT8) {
#pragma unroll
    for (int q = 0; q < Cfg<F>::B_LOADS; ++q) {
      const int g = wid * Cfg<F>::B_LOADS + q;
      const int row = 16 * g + (lane >> 2);
      const int c = (lane & 3) ^ swz64(row);
      const int64_t kb = k0 + 16 * c;
      const uint32_t off = kb < n ? (uint32_t)(row * n + kb) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + g * 1024), 16, off, 0, 0, 0);
    }
  } else if (F == F_INT16) {
#pragma unroll
    for (int q = 0; q < Cfg<F>::B_LOADS; ++q) {
      const int g = wid * Cfg<F>::B_LOADS + q;
      const int row = 8 * g + (lane >> 3);          // 128-byte rows (64 int16)
      const int c = (lane & 7) ^ swz128(row);
      const int64_t ke = k0 + 8 * c;                // first K element of the chunk
      const uint32_t off = ke < n ? (uint32_t)(2 * (row * n + ke)) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + g * 1024), 16, off, 0, 0, 0);
    }
  } else {  // F_INT4: 32-byte rows (64 nibbles)
#pragma unroll
    for (int q = 0; q < Cfg<F>::B_LOADS; ++q) {
      const int g = wid * Cfg<F>::B_LOADS + q;
      const int row = 32 * g + (lane >> 1);
      const int c = (lane & 1) ^ swz32(row);
      const int64_t ke = k0 + 32 * c;
      const uint32_t off = ke < n ? (uint32_t)(row * (n >> 1) + (ke >> 1)) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + g * 1024), 16, off, 0, 0, 0);
    }
  }
}

// vmcnt-only wait (expcnt / lgkmcnt left unconstrained), N <= 15.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8));
}

// INT4 fragment: 8 packed bytes (16 nibbles, K order) -> 16 int8 holding 16 * w.
__device__ __forceinline__ void unpack4(uint32_t x, uint32_t& o0, uint32_t& o1) {
  const uint32_t H = x & 0xF0F0F0F0u;         // odd K, already x16
  const uint32_t L = (x << 4) & 0xF0F0F0F0u;  // even K, x16
  o0 = __builtin_amdgcn_perm(H, L, 0x05010400u);
  o1 = __builtin_amdgcn_perm(H, L, 0x07030602u);
}

template <int F>
__global__ __launch_bounds__(lin::kThreads, 2) void k_linear(int64_t M, int64_t d, int64_t n,
                                                            const int8_t* __restrict__ xq,
                                                            const float* __restrict__ sx,
                                                            const int32_t* __restrict__ rowsum,
                                                            const uint8_t* __restrict__ m,
                                                            const float* __restrict__ sbar, uint16_t* __restrict__ Y,
                                                            int32_t* __restrict__ acc_dbg, int tiles_m, int tiles_n) {
  using namespace lin;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  constexpr int OUT = Cfg<F>::OUT;
  constexpr int STAGE = Cfg<F>::STAGE;

  // Blocks are dealt round-robin to the 8 XCDs; renumber so that each XCD receives a
  // contiguous range of tile ids, then walk tile ids in groups of kGroupM token tiles
  // (weight-tile index fastest inside a group), so that the blocks resident on one XCD
  // at a time cover a near-square patch of tiles and share operands in its L2.
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  {
    const int per = nblk / 8, rem = nblk % 8;
    const int x = bid % 8, loc = bid / 8;
    const int base = x * per + (x < rem ? x : rem);
    if (loc < per + (x < rem ? 1 : 0)) bid = base + loc;
  }
  const int group = bid / (kGroupM * tiles_n);
  const int tm_first = group * kGroupM;
  const int gsize = (tiles_m - tm_first) < kGroupM ? (tiles_m - tm_first) : kGroupM;
  const int in_group = bid - group * kGroupM * tiles_n;
  const int tm = tm_first + in_group % gsize, tn = in_group / gsize;
  const int64_t t0 = (int64_t)tm * BM;
  const int64_t o0 = (int64_t)tn * OUT;

  // Buffer descriptors based at this block's first token row / first output row.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(xq + t0 * n, (M - t0) * n);
  const int64_t wrow = F == F_INT16 ? 2 * n : (F == F_INT8 ? n : n / 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(m + o0 * wrow, (d - o0) * wrow);

  v16i acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int KT = (int)((n + BK - 1) / BK);
  issue_stage<F>(0, n, ra, rb, lds);
  if (KT > 1) issue_stage<F>(1, n, ra, rb, lds + STAGE);

  const int fr = lane & 31, h = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt has landed once at most the next stage's loads are outstanding
    if (kt + 1 < KT)
      wait_vmcnt<Cfg<F>::LOADS>();
    else
      wait_vmcnt<0>();
    // Every wave has its own loads of stage kt in LDS (vmcnt above); after the barrier
    // all waves' are, and no wave still reads the buffer the next issue overwrites.
    // A bare s_barrier: a fence here would also wait for the loads of stage kt+1.
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < KT) issue_stage<F>(kt + 2, n, ra, rb, lds + ((kt + 2) % kStages) * STAGE);
    const uint8_t* As = lds + (kt % kStages) * STAGE;
    const uint8_t* Bs = As + A_BYTES;

    // B fragments for both K sub-steps (sub-step ks of lane half h covers K 32h + 16ks ...)
    v4i bf[2][2];  // [ks][j]
    if (F == F_INT8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + fr;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          bf[ks][j] = *reinterpret_cast<const v4i*>(Bs + row * 64 + (((2 * h + ks) ^ swz64(row)) << 4));
      }
    } else if (F == F_INT16) {
      const int row = wn * 32 + fr;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c0 = 4 * h + 2 * ks;
        const v4i r0 = *reinterpret_cast<const v4i*>(Bs + row * 128 + ((c0 ^ swz128(row)) << 4));
        const v4i r1 = *reinterpret_cast<const v4i*>(Bs + row * 128 + (((c0 + 1) ^ swz128(row)) << 4));
        const uint32_t x[8] = {(uint32_t)r0.x, (uint32_t)r0.y, (uint32_t)r0.z, (uint32_t)r0.w,
                               (uint32_t)r1.x, (uint32_t)r1.y, (uint32_t)r1.z, (uint32_t)r1.w};
        // little-endian int16: the high byte of each value is byte 1 or 3 of its dword
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf[ks][0][q] = (int)__builtin_amdgcn_perm(x[2 * q + 1], x[2 * q], 0x07050301u);
          bf[ks][1][q] = (int)(__builtin_amdgcn_perm(x[2 * q + 1], x[2 * q], 0x06040200u) ^ 0x80808080u);
        }
      }
    } else {  // F_INT4: one 16-byte chunk per lane holds both sub-steps
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + fr;
        const v4i r = *reinterpret_cast<const v4i*>(Bs + row * 32 + ((h ^ swz32(row)) << 4));
        uint32_t o0_, o1_, o2_, o3_;
        unpack4((uint32_t)r.x, o0_, o1_);
        unpack4((uint32_t)r.y, o2_, o3_);
        bf[0][j] = v4i{(int)o0_, (int)o1_, (int)o2_, (int)o3_};
        unpack4((uint32_t)r.z, o0_, o1_);
        unpack4((uint32_t)r.w, o2_, o3_);
        bf[1][j] = v4i{(int)o0_, (int)o1_, (int)o2_, (int)o3_};
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + fr;
        af[i] = *reinterpret_cast<const v4i*>(As + row * 64 + (((2 * h + ks) ^ swz64(row)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[ks][j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue straight from the accumulators: lane l, register r of tile (i, j) holds
  // token t0 + wm*128 + 32 i + (l % 32) and MFMA column 8 (r / 4) + 4 (l / 32) + r % 4
  // of tile j; four consecutive registers are four consecutive outputs of one token.
  const int tok_in = lane & 31;
  const int colq = 4 * (lane >> 5);
  const bool vec_ok = (d & 3) == 0;
  float sxt[4];
  int64_t rs128[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t tok = t0 + wm * 128 + i * 32 + tok_in;
    sxt[i] = tok < M ? sx[tok] : 0.0f;
    rs128[i] = (F == F_INT16 && tok < M) ? 128 * (int64_t)rowsum[tok] : 0;
  }
  constexpr int NJ = (F == F_INT16) ? 1 : 2;  // column tiles (INT16: one output tile, two planes)
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t c0 = o0 + wn * ((F == F_INT16) ? 32 : 64) + j * 32 + 8 * a + colq;
      const bool full = vec_ok && c0 + 3 < d;
      float4 sb = make_float4(0.f, 0.f, 0.f, 0.f);
      if (full) {
        sb = *reinterpret_cast<const float4*>(sbar + c0);
      } else {
        if (c0 < d) sb.x = sbar[c0];
        if (c0 + 1 < d) sb.y = sbar[c0 + 1];
        if (c0 + 2 < d) sb.z = sbar[c0 + 2];
        if (c0 + 3 < d) sb.w = sbar[c0 + 3];
      }
      const float sbv[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tok = t0 + wm * 128 + i * 32 + tok_in;
        if (tok >= M) continue;
        int e0[4], e1[4];
        uint32_t hv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float y;
          if (F == F_INT16) {
            e0[b] = acc[i][0][4 * a + b];
            e1[b] = acc[i][1][4 * a + b];
            const int64_t exact = 256 * (int64_t)e0[b] + (int64_t)e1[b] + rs128[i];
            y = (float)(double)exact;
          } else {
            const int v = acc[i][j][4 * a + b];
            e0[b] = (F == F_INT4) ? (v >> 4) : v;
            y = (float)e0[b];
          }
          y = y * sxt[i];
          y = y * sbv[b];
          hv[b] = bf16_rne(y);
        }
        uint16_t* Yp = Y + tok * d + c0;
        int32_t* D0 = acc_dbg ? acc_dbg + tok * d + c0 : nullptr;
        int32_t* D1 = acc_dbg ? acc_dbg + M * d + tok * d + c0 : nullptr;
        if (full) {
          *reinterpret_cast<uint2*>(Yp) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
          if (D0) {
            *reinterpret_cast<int4*>(D0) = make_int4(e0[0], e0[1], e0[2], e0[3]);
            if (F == F_INT16) *reinterpret_cast<int4*>(D1) = make_int4(e1[0], e1[1], e1[2], e1[3]);
          }
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            if (c0 + b < d) {
              Yp[b] = (uint16_t)hv[b];
              if (D0) {
                D0[b] = e0[b];
                if (F == F_INT16) D1[b] = e1[b];
              }
            }
          }
        }
      }
    }
  }
}

hipError_t launch_linear(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx, const int32_t* rowsum,
                         int wfmt, const void* m, const float* sbar, uint16_t* Y, int32_t* acc_dbg, hipStream_t st) {
  using namespace lin;
  const int out_per_block = (wfmt == F_INT16) ? Cfg<F_INT16>::OUT : Cfg<F_INT8>::OUT;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((d + out_per_block - 1) / out_per_block);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const uint8_t* mb = static_cast<const uint8_t*>(m);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_linear<F_INT8>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Cfg<F_INT8>::LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_linear<F_INT4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, Cfg<F_INT4>::LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_linear<F_INT16>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, Cfg<F_INT16>::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  switch (wfmt) {
    case F_INT8:
      hipLaunchKernelGGL(k_linear<F_INT8>, grid, dim3(kThreads), Cfg<F_INT8>::LDS, st, M, d, n, xq, sx, rowsum, mb,
                         sbar, Y, acc_dbg, tiles_m, tiles_n);
      break;
    case F_INT4:
      hipLaunchKernelGGL(k_linear<F_INT4>, grid, dim3(kThreads), Cfg<F_INT4>::LDS, st, M, d, n, xq, sx, rowsum, mb,
                         sbar, Y, acc_dbg, tiles_m, tiles_n);
      break;
    default:
      hipLaunchKernelGGL(k_linear<F_INT16>, grid, dim3(kThreads), Cfg<F_INT16>::LDS, st, M, d, n, xq, sx, rowsum, mb,
                         sbar, Y, acc_dbg, tiles_m, tiles_n);
      break;
  }
  return hipGetLastError();
}

}  // namespace intlora
