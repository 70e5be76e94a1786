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
// (16 bytes per lane, no VGPR staging) through a 4-stage ring, so the loads of stages
// k+2 and k+3 are in flight while stage k computes.  Out-of-range rows and K chunks read as
// zero through the buffer descriptor.  LDS rows are XOR-swizzled in 16-byte chunks
// (conflict-free fragment reads); the swizzle is realized by the global address each
// lane fetches, since a direct load writes lane l's 16 bytes at base + 16 l.
//
// Tiling: a 256-thread block (4 waves, 2 x 2) computes 256 tokens x 256 MFMA columns
// (256 outputs, or 128 outputs x 2 planes); each wave owns 128 x 128 = 4 x 4 tiles of
// v_mfma_i32_32x32x32_i8 (256 accumulators, one wave per SIMD) with the weight
// fragment as the A operand, so a lane's four consecutive accumulators are four
// consecutive outputs of one token.  A 4-stage ring keeps two stages of loads in
// flight; the barrier of iteration k publishes stage k+1, so the first fragments of
// the next stage are read while the current stage's MFMAs run.
#include "device_common.h"
#include "intlora_internal.h"

namespace intlora {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

enum { F_INT4 = 4, F_INT8 = 8, F_INT16 = 16 };

namespace lin {
constexpr int kThreads = 256;  // 4 waves: 2 (tokens) x 2 (MFMA columns), 128 x 128 per wave
constexpr int BM = 256;        // tokens per block
constexpr int BK = 64;         // K elements per stage
constexpr int kStages = 4;
constexpr int kGroupM = 8;     // token tiles per group of the tile order (L2 reuse)
constexpr int A_BYTES = BM * BK;                // 16 KB
constexpr int B_BYTES_8 = 256 * BK;             // 16 KB: 256 output rows x 64 int8
constexpr int B_BYTES_16 = 128 * BK * 2;        // 16 KB: 128 output rows x 64 int16
constexpr int B_BYTES_4 = 256 * BK / 2;         // 8 KB: 256 output rows x 64 nibbles
template <int F>
struct Cfg {
  static constexpr int B_BYTES = F == F_INT16 ? B_BYTES_16 : (F == F_INT8 ? B_BYTES_8 : B_BYTES_4);
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = kStages * STAGE;
  static constexpr int OUT = F == F_INT16 ? 128 : 256;         // outputs per block
  static constexpr int A_LOADS = A_BYTES / 1024 / 4;           // direct loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / 4;
  static constexpr int LOADS = A_LOADS + B_LOADS;
};
}  // namespace lin

// XOR swizzles of the 16-byte chunks of an LDS row, chosen by timing the fragment
// read pattern on gfx950 (each is conflict-free there for its ds_read width).
__device__ __forceinline__ int swz64(int row) { return (row ^ (row >> 2)) & 3; }          // 64-byte rows
__device__ __forceinline__ int swz128(int row) { return (row ^ (row >> 2)) & 7; }         // 128-byte rows
__device__ __forceinline__ int swz32(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }   // 32-byte rows

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;  // offsets stay below 2^31; larger tensors get a per-tile base
  const int nrec = (int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every record: the lane reads zeros

// Offset `off` if the chunk starting at K element `k` lies inside the row, else an
// out-of-range offset (the lane reads zeros).  Branch-free 32-bit arithmetic.
__device__ __forceinline__ uint32_t in_row(uint32_t off, int k, int n) {
  const uint32_t keep = (uint32_t)((k - n) >> 31);  // all ones when k < n
  return (off & keep) | (kOOB & ~keep);
}

// Issue the direct loads of one K stage into one LDS stage buffer.  Row and column
// offsets fit in 32 bits (the descriptors are based at the block's first row).
template <int F>
__device__ __forceinline__ void issue_stage(int kt, int n, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                            uint8_t* stage) {
  using namespace lin;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k0 = kt * BK;
  // A (tokens): 16 rows of 64 bytes per direct load
#pragma unroll
  for (int q = 0; q < Cfg<F>::A_LOADS; ++q) {
    const int g = wid * Cfg<F>::A_LOADS + q;
    const int row = 16 * g + (lane >> 2);
    const int k = k0 + 16 * ((lane & 3) ^ swz64(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + g * 1024), 16,
                                             in_row((uint32_t)(row * n + k), k, n), 0, 0, 0);
  }
  uint8_t* Bs = stage + A_BYTES;
  if (F == F_INT8) {
#pragma unroll
    for (int q = 0; q < Cfg<F>::B_LOADS; ++q) {
      const int g = wid * Cfg<F>::B_LOADS + q;
      const int row = 16 * g + (lane >> 2);
      const int k = k0 + 16 * ((lane & 3) ^ swz64(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + g * 1024), 16,
                                               in_row((uint32_t)(row * n + k), k, n), 0, 0, 0);
    }
  } else if (F == F_INT16) {
#pragma unroll
    for (int q = 0; q < Cfg<F>::B_LOADS; ++q) {
      const int g = wid * Cfg<F>::B_LOADS + q;
      const int row = 8 * g + (lane >> 3);          // 128-byte rows (64 int16)
      const int k = k0 + 8 * ((lane & 7) ^ swz128(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + g * 1024), 16,
                                               in_row((uint32_t)(2 * (row * n + k)), k, n), 0, 0, 0);
    }
  } else {  // F_INT4: 32-byte rows (64 nibbles)
#pragma unroll
    for (int q = 0; q < Cfg<F>::B_LOADS; ++q) {
      const int g = wid * Cfg<F>::B_LOADS + q;
      const int row = 32 * g + (lane >> 1);
      const int k = k0 + 32 * ((lane & 1) ^ swz32(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + g * 1024), 16,
                                               in_row((uint32_t)(row * (n >> 1) + (k >> 1)), k, n), 0, 0, 0);
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

// Fragments of one K sub-step: A (tokens) for 4 tiles and B (weights) for 4 MFMA
// column tiles; sub-step ks of lane half h covers K 32 h + 16 ks .. + 16 of the stage.
template <int F>
__device__ __forceinline__ void read_frags(const uint8_t* __restrict__ As, int wm, int wn, int ks, int fr, int h,
                                           v4i (&af)[4], v4i (&bf)[4]) {
  using namespace lin;
  const uint8_t* Bs = As + A_BYTES;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + i * 32 + fr;
    af[i] = *reinterpret_cast<const v4i*>(As + row * 64 + (((2 * h + ks) ^ swz64(row)) << 4));
  }
  if (F == F_INT8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + j * 32 + fr;
      bf[j] = *reinterpret_cast<const v4i*>(Bs + row * 64 + (((2 * h + ks) ^ swz64(row)) << 4));
    }
  } else if (F == F_INT16) {
    // two output tiles of 32; tile q gives MFMA column tiles 2q (hi plane), 2q+1 (lo plane)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = wn * 64 + q * 32 + fr;
      const int c0 = 4 * h + 2 * ks;
      const v4i r0 = *reinterpret_cast<const v4i*>(Bs + row * 128 + ((c0 ^ swz128(row)) << 4));
      const v4i r1 = *reinterpret_cast<const v4i*>(Bs + row * 128 + (((c0 + 1) ^ swz128(row)) << 4));
      const uint32_t x[8] = {(uint32_t)r0.x, (uint32_t)r0.y, (uint32_t)r0.z, (uint32_t)r0.w,
                             (uint32_t)r1.x, (uint32_t)r1.y, (uint32_t)r1.z, (uint32_t)r1.w};
      // little-endian int16: the high byte of each value is byte 1 or 3 of its dword
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf[2 * q][e] = (int)__builtin_amdgcn_perm(x[2 * e + 1], x[2 * e], 0x07050301u);
        bf[2 * q + 1][e] = (int)(__builtin_amdgcn_perm(x[2 * e + 1], x[2 * e], 0x06040200u) ^ 0x80808080u);
      }
    }
  } else {  // F_INT4: 8 packed bytes per lane and sub-step (half of the lane's 16-byte chunk)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + j * 32 + fr;
      const uint2 r = *reinterpret_cast<const uint2*>(Bs + row * 32 + ((h ^ swz32(row)) << 4) + 8 * ks);
      uint32_t o0_, o1_, o2_, o3_;
      unpack4(r.x, o0_, o1_);
      unpack4(r.y, o2_, o3_);
      bf[j] = v4i{(int)o0_, (int)o1_, (int)o2_, (int)o3_};
    }
  }
}

template <int F>
__global__ __launch_bounds__(lin::kThreads, 1) void k_linear(int64_t M, int64_t d, int64_t n,
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

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int KT = (int)((n + BK - 1) / BK);
  const int fr = lane & 31, h = lane >> 5;
  // The loop body is one basic block so that the schedule below holds: stages past
  // the end are still issued, every lane of them reading zeros (out-of-range offset)
  // into a ring buffer that is never read again, and the fragment reads of stage k+1
  // at the last iteration fetch unused data.  vmcnt accounting is then uniform.
  issue_stage<F>(0, (int)n, ra, rb, lds);
  issue_stage<F>(1, (int)n, ra, rb, lds + STAGE);
  issue_stage<F>(2, (int)n, ra, rb, lds + 2 * STAGE);
  wait_vmcnt<2 * Cfg<F>::LOADS>();
  __builtin_amdgcn_s_barrier();
  v4i af0[4], bf0[4], af1[4], bf1[4];
  read_frags<F>(lds, wm, wn, 0, fr, h, af0, bf0);

  // Per iteration: the loads of stage k+3 and the reads of sub-step 1 are issued in
  // the shadow of the first eight MFMAs of sub-step 0; the reads of stage k+1 sub-step
  // 0 in the shadow of the first eight MFMAs of sub-step 1; VALU fragment conversion
  // (INT16 byte split, INT4 unpack) after them.
  constexpr int kValu = F == F_INT16 ? 3 : (F == F_INT4 ? 5 : 0);
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt+1 has landed (loads of kt+2 may still be in flight); after the barrier
    // it is visible to all waves and nobody reads stage kt-1, whose buffer kt+3 reuses
    wait_vmcnt<Cfg<F>::LOADS>();
    __builtin_amdgcn_s_barrier();
    issue_stage<F>(kt + 3, (int)n, ra, rb, lds + ((kt + 3) % kStages) * STAGE);
    const uint8_t* As = lds + (kt % kStages) * STAGE;
    read_frags<F>(As, wm, wn, 1, fr, h, af1, bf1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf0[j], af0[i], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (kValu) __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
    }
    read_frags<F>(lds + ((kt + 1) % kStages) * STAGE, wm, wn, 0, fr, h, af0, bf0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf1[j], af1[i], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (kValu) __builtin_amdgcn_sched_group_barrier(0x002, kValu, 1);
    }
  }
  wait_vmcnt<0>();  // the trailing zero-reading loads land before LDS is reused

  // Epilogue, one 32-token slab (i) at a time through LDS: each wave writes its 32 x 128
  // int32 accumulators as 16-byte groups (lane l, registers 4a..4a+3 of tile j are
  // token l % 32, MFMA columns 32 j + 8 a + 4 (l / 32) + 0..3) into a padded region of
  // its own, then reads them back row-contiguously; each lane finishes four outputs.
  __syncthreads();
  constexpr int RS = 132;  // padded row stride (ints): conflict-free 16-byte accesses
  int32_t* R = reinterpret_cast<int32_t*>(lds) + wid * (32 * RS);
  const bool vec_ok = (d & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<v4i*>(R + fr * RS + j * 32 + 8 * a + 4 * h) =
            v4i{acc[i][j][4 * a], acc[i][j][4 * a + 1], acc[i][j][4 * a + 2], acc[i][j][4 * a + 3]};
    // (a wave's LDS accesses complete in order: its own reads below see these writes)
    const int64_t tok_base = t0 + wm * 128 + i * 32;
    if (F == F_INT16) {
      // region row: [hi 0..31 | lo 0..31 | hi 32..63 | lo 32..63] of the wave's 64 outputs
      const int o = 4 * (lane & 15);                 // first of four outputs of this lane
      const int hcol = (o >> 5) * 64 + (o & 31);
      const int64_t c0 = o0 + wn * 64 + o;
      const bool full = vec_ok && c0 + 3 < d;
      for (int rr = 0; rr < 32; rr += 4) {
        const int row = rr + (lane >> 4);
        const int64_t tok = tok_base + row;
        if (tok >= M || c0 >= d) continue;
        const v4i hi = *reinterpret_cast<const v4i*>(R + row * RS + hcol);
        const v4i lo = *reinterpret_cast<const v4i*>(R + row * RS + hcol + 32);
        const int64_t rs128 = 128 * (int64_t)rowsum[tok];
        const float sxt = sx[tok];
        uint32_t hv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t exact = 256 * (int64_t)hi[b] + (int64_t)lo[b] + rs128;
          float y = (float)(double)exact;
          y = y * sxt;
          y = y * (c0 + b < d ? sbar[c0 + b] : 0.0f);
          hv[b] = bf16_rne(y);
        }
        uint16_t* Yp = Y + tok * d + c0;
        if (full) {
          *reinterpret_cast<uint2*>(Yp) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
          if (acc_dbg) {
            *reinterpret_cast<v4i*>(acc_dbg + tok * d + c0) = hi;
            *reinterpret_cast<v4i*>(acc_dbg + M * d + tok * d + c0) = lo;
          }
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (c0 + b < d) {
              Yp[b] = (uint16_t)hv[b];
              if (acc_dbg) {
                acc_dbg[tok * d + c0 + b] = hi[b];
                acc_dbg[M * d + tok * d + c0 + b] = lo[b];
              }
            }
        }
      }
    } else {
      const int cc = 4 * (lane & 31);                // first of four columns of this lane
      const int64_t c0 = o0 + wn * 128 + cc;
      const bool full = vec_ok && c0 + 3 < d;
      for (int rr = 0; rr < 32; rr += 2) {
        const int row = rr + (lane >> 5);
        const int64_t tok = tok_base + row;
        if (tok >= M || c0 >= d) continue;
        const v4i v = *reinterpret_cast<const v4i*>(R + row * RS + cc);
        const float sxt = sx[tok];
        int ex[4];
        uint32_t hv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          ex[b] = (F == F_INT4) ? (v[b] >> 4) : v[b];
          float y = (float)ex[b];
          y = y * sxt;
          y = y * (c0 + b < d ? sbar[c0 + b] : 0.0f);
          hv[b] = bf16_rne(y);
        }
        uint16_t* Yp = Y + tok * d + c0;
        if (full) {
          *reinterpret_cast<uint2*>(Yp) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
          if (acc_dbg) *reinterpret_cast<v4i*>(acc_dbg + tok * d + c0) = v4i{ex[0], ex[1], ex[2], ex[3]};
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (c0 + b < d) {
              Yp[b] = (uint16_t)hv[b];
              if (acc_dbg) acc_dbg[tok * d + c0 + b] = ex[b];
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
