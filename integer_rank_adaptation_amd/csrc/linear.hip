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
//   INT16 (MUL)              byte split into two int8 planes after the LDS read, one
//                            split per launch, chosen from the rows' split codes:
//                            bias (some code 1, any int16): hi = m >> 8,
//                              lo = (m & 0xFF) - 128, exact = 256 acc_hi + acc_lo +
//                              128 rowsum(X_q);
//                            balanced (all codes 0: every m <= 32639):
//                              hi = (m + 128) >> 8, lo = m - 256 hi,
//                              exact = 256 acc_hi + acc_lo;
//                            formed exactly in binary64 (|exact| < 2^53).  For merged
//                            integers of small magnitude the balanced high plane is all
//                            zeros, which lowers the matrix cores' switching power (the
//                            chip runs at a higher clock).  Each split has its own copy
//                            of the K loop.
//   UW4 (MUL, merge on load) U's 4-bit codes and the 4-bit base codes (packed nibbles),
//                            with the per-row zero points z_bar, z: m = (U_round -
//                            z_bar) (W_round - z) is formed after the LDS read in
//                            packed 16-bit lanes (|m| <= 225, exact) and split like
//                            INT16 with the balanced split (always valid here).  The
//                            merged integers never exist in memory; several adapters
//                            share one copy of the base codes.
//
// Data path: every operand goes from HBM straight into LDS with buffer_load ... lds
// (16 bytes per lane, no VGPR staging) through a 4-stage ring, so the loads of stages
// k+2 and k+3 are in flight while stage k computes.  Each stage gets buffer
// descriptors based at its first K element, so a lane's offsets are fixed for the
// whole loop; rows past the end and stages past n read zeros through the descriptor
// range.  LDS rows are XOR-swizzled in 16-byte chunks (conflict-free fragment reads);
// the swizzle is realized by the global address each lane fetches, since a direct
// load writes lane l's 16 bytes at base + 16 l.
//
// Tiling: a 256-thread block (4 waves, 2 x 2) computes 256 tokens x 256 MFMA columns
// (256 outputs, or 128 outputs x 2 planes); each wave owns 128 x 128 = 4 x 4 tiles of
// v_mfma_i32_32x32x32_i8 (256 accumulators, one wave per SIMD) with the weight
// fragment as the A operand, so a lane's four consecutive accumulators are four
// consecutive outputs of one token.  Two operand register sets alternate: while the
// 16 MFMAs of one 32-deep K sub-step run on one set, the other is read from LDS (one
// read per MFMA) and format-converted, and the stage's direct loads are issued, in an
// order pinned with sched_barrier.  The barrier of iteration k publishes stage k+1.
//
// Epilogue: per-token scales / row sums and per-output scales go to LDS once; the
// accumulators pass through a padded LDS region per wave so that each lane writes four
// consecutive bf16 outputs of one row (hardware round-to-nearest-even conversion).
#include <type_traits>

#include "device_common.h"
#include "intlora_internal.h"

namespace intlora {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// F_P16T / F_P16N: the int16 merged integers stored as their two byte planes (per row,
// the n high bytes, then the n low bytes); F_P16T multiplies both planes, F_P16N only
// the low plane (every high byte of the call is zero), whose rows it reads as whole
// contiguous runs.
enum { F_INT4 = 4, F_INT8 = 8, F_INT16 = 16, F_P16T = 17, F_P16N = 18, F_UW4 = 44 };
// B-tile layout families in LDS: 128-byte rows (64 int16, or 64 high + 64 low bytes)
// for 128 outputs; 64-byte rows (64 int8) for 256 outputs.
constexpr bool is_l16(int F) { return F == F_INT16 || F == F_P16T; }
constexpr bool is_l8(int F) { return F == F_INT8 || F == F_P16N; }
constexpr bool planar(int F) { return F == F_P16T || F == F_P16N; }

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
constexpr int B_BYTES_UW4 = 2 * 128 * BK / 2;   // 8 KB: U then W codes, 128 output rows x 64 nibbles each
constexpr int EPI_RS = 64 * 2 + 16;             // epilogue staging row: 64 bf16 outputs + 16 bytes pad
constexpr int EPI_WAVE = 32 * EPI_RS;           // one wave's 32 tokens x 64 outputs
constexpr int EPI_VEC = 4 * EPI_WAVE;           // offset of the per-tile vectors in the epilogue region
constexpr int EPI_BYTES = EPI_VEC + 4 * 4 * 256;
template <int F>
struct Cfg {
  static constexpr int B_BYTES =
      is_l16(F) ? B_BYTES_16 : (is_l8(F) ? B_BYTES_8 : (F == F_UW4 ? B_BYTES_UW4 : B_BYTES_4));
  static constexpr bool TWO = F == F_INT16 || F == F_UW4 || F == F_P16T;  // two byte planes of int16 values
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int RING = kStages * STAGE;
  static constexpr int LDS = RING + EPI_BYTES;
  static constexpr int OUT = TWO ? 128 : 256;                  // outputs per block
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

// Per-lane byte offsets of the lane's 16-byte chunks inside one K stage, relative to
// the stage's first K element: they do not change from stage to stage (each stage
// gets a buffer descriptor based at its first K element), so the main loop spends no
// vector instructions on addresses.  `akk` is the lane's first K element of each A
// chunk (for the zero fill of a partial last stage).
template <int F>
struct Plan {
  uint32_t a[lin::Cfg<F>::A_LOADS];
  uint32_t b[lin::Cfg<F>::B_LOADS];
  int akk[lin::Cfg<F>::A_LOADS];
};

template <int F>
__device__ __forceinline__ void make_plan(int n, Plan<F>& p) {
  using namespace lin;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < Cfg<F>::A_LOADS; ++q) {  // A (tokens): 16 rows of 64 bytes per load
    const int g = wid * Cfg<F>::A_LOADS + q;
    const int row = 16 * g + (lane >> 2);
    const int kk = 16 * ((lane & 3) ^ swz64(row));
    p.a[q] = (uint32_t)(row * n + kk);
    p.akk[q] = kk;
  }
#pragma unroll
  for (int q = 0; q < Cfg<F>::B_LOADS; ++q) {
    const int g = wid * Cfg<F>::B_LOADS + q;
    if (F == F_INT8) {           // 64-byte rows
      const int row = 16 * g + (lane >> 2);
      p.b[q] = (uint32_t)(row * n + 16 * ((lane & 3) ^ swz64(row)));
    } else if (F == F_P16N) {    // 64-byte rows of the low plane (n bytes into the row)
      const int row = 16 * g + (lane >> 2);
      p.b[q] = (uint32_t)(row * 2 * n + n + 16 * ((lane & 3) ^ swz64(row)));
    } else if (F == F_P16T) {    // 128-byte LDS rows: chunk c holds 16 high (c even) or low
      const int row = 8 * g + (lane >> 3);  // (c odd) bytes of columns 16 (c / 2) + 0..15
      const int c = (lane & 7) ^ swz128(row);
      p.b[q] = (uint32_t)(row * 2 * n + (c & 1) * n + 16 * (c >> 1));
    } else if (is_l16(F)) {      // 128-byte rows (64 int16)
      const int row = 8 * g + (lane >> 3);
      p.b[q] = (uint32_t)(2 * (row * n + 8 * ((lane & 7) ^ swz128(row))));
    } else if (F == F_UW4) {     // 32-byte rows: loads 0..3 U's 128 rows, 4..7 W's (same offsets)
      const int row = 32 * (g & 3) + (lane >> 1);
      p.b[q] = (uint32_t)(row * (n >> 1) + 16 * ((lane & 1) ^ swz32(row)));
    } else {                     // F_INT4: 32-byte rows (64 nibbles)
      const int row = 32 * g + (lane >> 1);
      p.b[q] = (uint32_t)(row * (n >> 1) + 16 * ((lane & 1) ^ swz32(row)));
    }
  }
}

// Descriptors of K stage kt: based at the stage's first K element, so that the
// per-lane offsets of the plan stay fixed.  Rows past the end of the operand and
// stages past n fall outside the record count and read zeros.
template <int F>
__device__ __forceinline__ void stage_rsrc(int kt, const int8_t* a_tile, int64_t a_bytes, const uint8_t* b_tile,
                                           int64_t b_bytes, __amdgpu_buffer_rsrc_t& ra, __amdgpu_buffer_rsrc_t& rb) {
  using namespace lin;
  const int k0 = kt * BK;
  // bytes of the stage's first K element from the row start: INT16 2 per element, the
  // planes and INT8 1 (a plane's offset within the row is in the plan), INT4 / UW4 1/2
  const int64_t kb = F == F_INT16 ? 2 * (int64_t)k0 : ((F == F_INT8 || planar(F)) ? (int64_t)k0 : (int64_t)(k0 >> 1));
  ra = make_rsrc(a_tile + k0, a_bytes - k0);
  rb = make_rsrc(b_tile + kb, b_bytes - kb);
}

// Direct load number q (A loads first, then B) of one stage into the stage buffer.
// With KTAIL (n not a multiple of BK) the A chunks past n in a partial stage read
// zeros, which zeroes their products whatever the B bytes there are.
// UW4: b_tile is the tile of U's codes; the base codes lie wdelta bytes after it (the
// same layout), so one extra descriptor reaches them.
template <int F, bool KTAIL>
__device__ __forceinline__ void issue_load(int q, int n, int kt, const int8_t* a_tile, int64_t a_bytes,
                                           const uint8_t* b_tile, int64_t b_bytes, const Plan<F>& p,
                                           uint8_t* stage, int64_t wdelta) {
  using namespace lin;
  const int k0 = kt * BK;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (q < Cfg<F>::A_LOADS) {
    __amdgpu_buffer_rsrc_t ra, rb;
    stage_rsrc<F>(kt, a_tile, a_bytes, b_tile, b_bytes, ra, rb);
    const int g = wid * Cfg<F>::A_LOADS + q;
    uint32_t off = p.a[q];
    if (KTAIL) off = p.akk[q] < n - k0 ? off : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + g * 1024), 16, off, 0, 0, 0);
  } else {
    const int qb = q - Cfg<F>::A_LOADS;
    const int g = wid * Cfg<F>::B_LOADS + qb;
    __amdgpu_buffer_rsrc_t ra, rb;
    const uint8_t* bsrc = (F == F_UW4 && g >= 4)
                              ? reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(b_tile) + (uintptr_t)wdelta)
                              : b_tile;
    stage_rsrc<F>(kt, a_tile, a_bytes, bsrc, b_bytes, ra, rb);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + A_BYTES + g * 1024), 16, p.b[qb], 0, 0, 0);
  }
}

template <int F, bool KTAIL>
__device__ __forceinline__ void issue_stage(int kt, int n, const int8_t* a_tile, int64_t a_bytes,
                                            const uint8_t* b_tile, int64_t b_bytes, const Plan<F>& p,
                                            uint8_t* stage, int64_t wdelta) {
#pragma unroll
  for (int q = 0; q < lin::Cfg<F>::LOADS; ++q)
    issue_load<F, KTAIL>(q, n, kt, a_tile, a_bytes, b_tile, b_bytes, p, stage, wdelta);
}

// vmcnt-only wait (expcnt / lgkmcnt left unconstrained), N <= 15.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// INT4 fragment: 8 packed bytes (16 nibbles, K order) -> 16 int8 holding 16 * w.
__device__ __forceinline__ void unpack4(uint32_t x, uint32_t& o0, uint32_t& o1) {
  const uint32_t H = x & 0xF0F0F0F0u;         // odd K, already x16
  const uint32_t L = (x << 4) & 0xF0F0F0F0u;  // even K, x16
  o0 = __builtin_amdgcn_perm(H, L, 0x05010400u);
  o1 = __builtin_amdgcn_perm(H, L, 0x07030602u);
}

// Raw B fragment bytes of one K sub-step (LDS read), before format conversion.
template <int F>
struct RawB {
  v4i v[4];
};

// Per-lane byte offsets of the fragment reads inside an LDS stage, for sub-steps ks = 0, 1
// (second index: the two 16-byte chunks of an INT16 row).  The swizzles depend only on
// row bits 0..4, i.e. on the lane's row within a 32-row tile, so the other fragments of
// a sub-step lie at constant distances (2048 bytes per A tile and per INT8 B tile, 4096
// per INT16 B tile, 1024 per INT4 B tile) and the reads fold them into their offsets.
struct LdsLane {
  uint32_t a[2];
  uint32_t b[2][2];
};

template <int F>
__device__ __forceinline__ LdsLane lds_lane(int wm, int wn, int fr, int h) {
  using namespace lin;
  LdsLane ll;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    ll.a[ks] = (uint32_t)((wm * 128 + fr) * 64 + (((2 * h + ks) ^ swz64(fr)) << 4));
    if (is_l8(F)) {
      ll.b[ks][0] = (uint32_t)(A_BYTES + (wn * 128 + fr) * 64 + (((2 * h + ks) ^ swz64(fr)) << 4));
      ll.b[ks][1] = 0;
    } else if (is_l16(F)) {  // INT16: the two chunks of 8 values; P16T: high then low bytes of 16
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        ll.b[ks][jj] = (uint32_t)(A_BYTES + (wn * 64 + fr) * 128 + (((4 * h + 2 * ks + jj) ^ swz128(fr)) << 4));
    } else if (F == F_UW4) {  // U's row of the lane's first output tile; W 4096 bytes on
      ll.b[ks][0] = (uint32_t)(A_BYTES + (wn * 64 + fr) * 32 + ((h ^ swz32(fr)) << 4) + 8 * ks);
      ll.b[ks][1] = 0;
    } else {
      ll.b[ks][0] = (uint32_t)(A_BYTES + (wn * 128 + fr) * 32 + ((h ^ swz32(fr)) << 4) + 8 * ks);
      ll.b[ks][1] = 0;
    }
  }
  return ll;
}

// A (tokens) fragments of one K sub-step: 4 tiles; sub-step ks of lane half h covers
// K 32 h + 16 ks .. + 16 of the stage.
__device__ __forceinline__ void read_a(const uint8_t* __restrict__ S, const LdsLane& ll, int ks, v4i (&af)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const v4i*>(S + ll.a[ks] + i * 2048);
}

// Raw B chunk j (0..3) of sub-step ks.  INT16: two output tiles of 32 rows, 32 int16
// (two 16-byte chunks) per lane and sub-step; INT4: 8 packed bytes per lane and
// sub-step (half of the lane's 16-byte chunk).
template <int F>
__device__ __forceinline__ v4i read_b_chunk(const uint8_t* __restrict__ S, const LdsLane& ll, int ks, int j) {
  if (is_l8(F)) return *reinterpret_cast<const v4i*>(S + ll.b[ks][0] + j * 2048);
  if (is_l16(F)) return *reinterpret_cast<const v4i*>(S + ll.b[ks][j & 1] + (j >> 1) * 4096);
  // INT4: tile j; UW4: chunk 2 q holds U's and 2 q + 1 W's 16 nibbles of output tile q
  const uint32_t off = F == F_UW4 ? (uint32_t)((j >> 1) * 1024 + (j & 1) * 4096) : (uint32_t)(j * 1024);
  const uint2 r = *reinterpret_cast<const uint2*>(S + ll.b[ks][0] + off);
  return v4i{(int)r.x, (int)r.y, 0, 0};
}

template <int F>
__device__ __forceinline__ void read_b(const uint8_t* __restrict__ S, const LdsLane& ll, int ks, RawB<F>& rw) {
#pragma unroll
  for (int j = 0; j < 4; ++j) rw.v[j] = read_b_chunk<F>(S, ll, ks, j);
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
// two int16 + add (per 16-bit half, no carry between them)
__device__ __forceinline__ uint32_t add16x2(uint32_t x, uint32_t a) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(us2, x) + __builtin_bit_cast(us2, a));
}

// The two int8 planes (x: high, y: low) of the four int16 in (x0, x1), little-endian:
// the high byte of each value is byte 1 or 3 of its dword.  Bias split: the high bytes,
// and the low bytes with bit 7 flipped; balanced split: the high bytes of m + 128 and
// the low bytes as they are.
template <bool BIAS>
__device__ __forceinline__ uint2 split16(uint32_t x0, uint32_t x1) {
  if (BIAS)
    return make_uint2(__builtin_amdgcn_perm(x1, x0, 0x07050301u),
                      __builtin_amdgcn_perm(x1, x0, 0x06040200u) ^ 0x80808080u);
  return make_uint2(__builtin_amdgcn_perm(add16x2(x1, 0x00800080u), add16x2(x0, 0x00800080u), 0x07050301u),
                    __builtin_amdgcn_perm(x1, x0, 0x06040200u));
}

typedef short s2v __attribute__((ext_vector_type(2)));

// UW4: the four merged integers of K 4 h' .. 4 h' + 3 of one output row (h' = 2 x +
// half within the 8-K dword pair), as two dwords of int16 pairs in K order, from the
// dwords u, w of 8 nibbles each (byte b holds K 2b in its low nibble, 2b + 1 in its
// high one) and the row's zero points broadcast to both 16-bit halves (zb2, zw2):
// m = (u - z_bar) (w - z) in packed 16-bit lanes, exact since |m| <= 225.
__device__ __forceinline__ uint2 uw4_m(uint32_t u, uint32_t w, uint32_t zb2, uint32_t zw2, int half) {
  const uint32_t ul = u & 0x0F0F0F0Fu, uh = (u >> 4) & 0x0F0F0F0Fu;
  const uint32_t wl = w & 0x0F0F0F0Fu, wh = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t b0 = 2u * (uint32_t)half, b1 = b0 + 1u;
  // output bytes: (low byte of K even, 0, low byte of K odd, 0); selector 12 gives 0
  const uint32_t s0 = 0x0C000C00u | b0 | ((4u + b0) << 16);
  const uint32_t s1 = 0x0C000C00u | b1 | ((4u + b1) << 16);
  const s2v zb = __builtin_bit_cast(s2v, zb2), zw = __builtin_bit_cast(s2v, zw2);
  const s2v u0 = __builtin_bit_cast(s2v, __builtin_amdgcn_perm(uh, ul, s0)) - zb;
  const s2v u1 = __builtin_bit_cast(s2v, __builtin_amdgcn_perm(uh, ul, s1)) - zb;
  const s2v w0 = __builtin_bit_cast(s2v, __builtin_amdgcn_perm(wh, wl, s0)) - zw;
  const s2v w1 = __builtin_bit_cast(s2v, __builtin_amdgcn_perm(wh, wl, s1)) - zw;
  return make_uint2(__builtin_bit_cast(uint32_t, u0 * w0), __builtin_bit_cast(uint32_t, u1 * w1));
}

// B (weight) MFMA operands for 4 column tiles from the raw bytes.  INT16 and UW4: tile
// q of outputs gives MFMA column tiles 2q (hi plane) and 2q+1 (lo plane).  zp (UW4
// only): z_bar and z of the lane's rows in output tiles 0 and 1, broadcast to both
// 16-bit halves.
template <int F, bool BIAS>
__device__ __forceinline__ void convert_piece(int p, const RawB<F>& rw, v4i (&bf)[4], const uint32_t (&zp)[4]);

template <int F, bool BIAS>
__device__ __forceinline__ void convert_b(const RawB<F>& rw, v4i (&bf)[4], const uint32_t (&zp)[4]) {
  if (F == F_UW4) {
#pragma unroll
    for (int p = 0; p < 8; ++p) convert_piece<F, BIAS>(p, rw, bf, zp);
    return;
  }
  if (is_l8(F) || F == F_P16T) {  // already int8 operands (P16T: chunk 2q high, 2q + 1 low of tile q)
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = rw.v[j];
  } else if (F == F_INT16) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const v4i r0 = rw.v[2 * q], r1 = rw.v[2 * q + 1];
      const uint32_t x[8] = {(uint32_t)r0.x, (uint32_t)r0.y, (uint32_t)r0.z, (uint32_t)r0.w,
                             (uint32_t)r1.x, (uint32_t)r1.y, (uint32_t)r1.z, (uint32_t)r1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 hl = split16<BIAS>(x[2 * e], x[2 * e + 1]);
        bf[2 * q][e] = (int)hl.x;
        bf[2 * q + 1][e] = (int)hl.y;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t o0_, o1_, o2_, o3_;
      unpack4((uint32_t)rw.v[j].x, o0_, o1_);
      unpack4((uint32_t)rw.v[j].y, o2_, o3_);
      bf[j] = v4i{(int)o0_, (int)o1_, (int)o2_, (int)o3_};
    }
  }
}

// One LDS read of a sub-step: reads 0..3 are the raw B chunks, 4..7 the A fragments.
template <int F>
__device__ __forceinline__ void read_piece(int q, const uint8_t* __restrict__ S, const LdsLane& ll, int ks,
                                           v4i (&af)[4], RawB<F>& rw) {
  if (q >= 4)
    af[q - 4] = *reinterpret_cast<const v4i*>(S + ll.a[ks] + (q - 4) * 2048);
  else
    rw.v[q] = read_b_chunk<F>(S, ll, ks, q);
}

// Conversion piece p (0..7) of the raw B bytes into MFMA operands.
template <int F, bool BIAS>
__device__ __forceinline__ void convert_piece(int p, const RawB<F>& rw, v4i (&bf)[4], const uint32_t (&zp)[4]) {
  if (is_l8(F)) {
    if (p < 4) bf[p] = rw.v[p];
  } else if (F == F_P16T) {
    const int q = p >> 2, e = p & 3;
    bf[2 * q][e] = rw.v[2 * q][e];
    bf[2 * q + 1][e] = rw.v[2 * q + 1][e];
  } else if (F == F_UW4) {
    const int q = p >> 2, e = p & 3;  // output tile q, K 4e .. 4e + 3 of the sub-step
    const uint2 mm = uw4_m((uint32_t)rw.v[2 * q][e >> 1], (uint32_t)rw.v[2 * q + 1][e >> 1], zp[2 * q],
                           zp[2 * q + 1], e & 1);
    const uint2 hl = split16<false>(mm.x, mm.y);
    bf[2 * q][e] = (int)hl.x;
    bf[2 * q + 1][e] = (int)hl.y;
  } else if (F == F_INT16) {
    const int q = p >> 2, e = p & 3;  // output tile q, dword pair e
    const v4i& lo16 = rw.v[2 * q + (e >> 1)];
    const uint32_t x0 = (uint32_t)lo16[2 * (e & 1)], x1 = (uint32_t)lo16[2 * (e & 1) + 1];
    const uint2 hl = split16<BIAS>(x0, x1);
    bf[2 * q][e] = (int)hl.x;
    bf[2 * q + 1][e] = (int)hl.y;
  } else {
    const int j = p >> 1, w = p & 1;
    uint32_t o0_, o1_;
    unpack4((uint32_t)rw.v[j][w], o0_, o1_);
    bf[j][2 * w] = (int)o0_;
    bf[j][2 * w + 1] = (int)o1_;
  }
}

__device__ __forceinline__ void mfma16(const v4i (&af)[4], const v4i (&bf)[4], v16i (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af[i], acc[i][j], 0, 0, 0);
}

// Reads an accumulator where it is used: without this the compiler copies all 256
// accumulators out of the AGPRs at once after the main loop (and spills them).
__device__ __forceinline__ int acc_read(int v) {
  int r;
  __asm__ volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
  return r;
}

// Tile id -> (token tile, weight tile): tile ids are walked in groups of kGroupM token
// tiles (token tile fastest inside a group), so consecutive ids form near-square
// patches that share operands in L2.
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, int& tm, int& tn) {
  using namespace lin;
  const int group = tile / (kGroupM * tiles_n);
  const int tm_first = group * kGroupM;
  const int gsize = (tiles_m - tm_first) < kGroupM ? (tiles_m - tm_first) : kGroupM;
  const int in_group = tile - group * kGroupM * tiles_n;
  tm = tm_first + in_group % gsize;
  tn = in_group / gsize;
}

// Whether any of the d codes (16-byte aligned) is not zero, for this thread's share:
// the block's threads together cover all d and the caller combines their flags.  A
// thread's loads carry no branch between them, so for d <= 64 blockDim.x the whole scan
// costs one memory round trip.
__device__ __forceinline__ int any_code(const uint8_t* __restrict__ code, int64_t d) {
  const int64_t d16 = d & ~(int64_t)15;
  const int64_t stride = 16 * (int64_t)blockDim.x;
  int fl = 0;
  for (int64_t x0 = 16 * (int64_t)threadIdx.x; x0 < d16; x0 += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t x = x0 + u * stride;
      v[u] = x < d16 ? *reinterpret_cast<const uint4*>(code + x) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) fl |= (int)((v[u].x | v[u].y | v[u].z | v[u].w) != 0u);
  }
  const int64_t k = d16 + threadIdx.x;
  if (k < d) fl |= (int)(code[k] != 0);
  return fl;
}

// Persistent kernel: each block owns the tiles r * G + slot (r = 0, 1, ...), where G is
// the grid size and slot renumbers the block so that each of the 8 XCDs (blocks are
// dealt to them round-robin) receives a contiguous range of slots, i.e. a compact
// patch of tiles in every round.  The K stages of a block's consecutive tiles form one
// continuous stream through the LDS ring: the loads of the next tile's first stages
// are issued during the current tile's last iterations, and the epilogue (which has
// an LDS region of its own) runs while they are in flight.
// The body of the kernel for format F, on the block's dynamic LDS `lds`.  split: the
// INT16 split codes, or (byte planes) the plane codes, whose bit 1 marks a row stored in
// the bias split.
template <int F, bool KTAIL>
__device__ __forceinline__ void linear_body(uint8_t* __restrict__ lds, int64_t M, int64_t d, int64_t n,
                                            const int8_t* __restrict__ xq, const float* __restrict__ sx,
                                            const int32_t* __restrict__ rowsum, const uint8_t* __restrict__ m,
                                            const uint8_t* __restrict__ split, const float* __restrict__ sbar,
                                            uint16_t* __restrict__ Y, int32_t* __restrict__ acc_dbg, int tiles_m,
                                            int tiles_n, int64_t wdelta, const int32_t* __restrict__ zbar_p,
                                            const int32_t* __restrict__ zw_p) {
  using namespace lin;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  constexpr int OUT = Cfg<F>::OUT;
  constexpr int STAGE = Cfg<F>::STAGE;
  const int ntile = tiles_m * tiles_n;
  const int G = gridDim.x;
  int slot = blockIdx.x;
  {
    const int per = G / 8, rem = G % 8;
    const int x = slot % 8, loc = slot / 8;
    const int base = x * per + (x < rem ? x : rem);
    if (loc < per + (x < rem ? 1 : 0)) slot = base + loc;
  }
  const int my_tiles = slot < ntile ? (ntile - slot + G - 1) / G : 0;
  const int64_t wrow = (F == F_INT16 || planar(F)) ? 2 * n : (F == F_INT8 ? n : n / 2);  // bytes per weight row
  const int KT = (int)((n + BK - 1) / BK);
  const int fr = lane & 31, h = lane >> 5;
  Plan<F> plan;
  make_plan<F>((int)n, plan);

  // operand tiles of local tile lt (null range past the block's last tile: zero loads)
  auto tile_ptrs = [&](int lt, const int8_t*& at, int64_t& ab, const uint8_t*& bt, int64_t& bb) {
    if (lt < my_tiles) {
      int tm, tn;
      tile_coords(lt * G + slot, tiles_m, tiles_n, tm, tn);
      at = xq + (int64_t)tm * BM * n;
      ab = (M - (int64_t)tm * BM) * n;
      bt = m + (int64_t)tn * OUT * wrow;
      bb = (d - (int64_t)tn * OUT) * wrow;
    } else {
      at = xq;
      ab = 0;
      bt = m;
      bb = 0;
    }
  };
  const int8_t* a_cur;
  const uint8_t* b_cur;
  int64_t ab_cur, bb_cur;
  const int8_t* a_nxt;
  const uint8_t* b_nxt;
  int64_t ab_nxt, bb_nxt;
  tile_ptrs(0, a_cur, ab_cur, b_cur, bb_cur);
  tile_ptrs(1, a_nxt, ab_nxt, b_nxt, bb_nxt);

  // UW4: the zero points of the lane's rows (output tiles q = 0, 1) of local tile lt,
  // each broadcast to both 16-bit halves: zp = {z_bar q0, z q0, z_bar q1, z q1}.  The
  // current tile's set converts its stages; the next tile's set converts that tile's
  // first sub-step, at the end of the current tile.  The next set is loaded right
  // after the first barrier of a tile, between two stages' direct loads, so the
  // in-order load counter covers it without extra waits.
  uint32_t zpc[4] = {0, 0, 0, 0}, zpn[4] = {0, 0, 0, 0};
  auto load_zp = [&](int lt, uint32_t (&zp)[4]) {
    if (lt < my_tiles) {
      int tm, tn;
      tile_coords(lt * G + slot, tiles_m, tiles_n, tm, tn);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t o = (int64_t)tn * OUT + wn * 64 + 32 * q + fr;
        const uint32_t zb = o < d ? (uint32_t)zbar_p[o] : 0u, zw = o < d ? (uint32_t)zw_p[o] : 0u;
        zp[2 * q] = zb | (zb << 16);
        zp[2 * q + 1] = zw | (zw << 16);
      }
    }
  };
  if (F == F_UW4) load_zp(0, zpc);

  // INT16 split of the launch: bias when some row's code is 1 (or there are no codes),
  // else balanced.  The codes are read before the first stages are issued and voted
  // on at the prologue's barrier.
  int fl = 0;
  if (F == F_INT16) fl = split == nullptr ? 1 : any_code(split, d);

  // stages 0..2 of the stream (KT >= 3 whenever a block owns more than one tile)
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    if (g < KT)
      issue_stage<F, KTAIL>(g, (int)n, a_cur, ab_cur, b_cur, bb_cur, plan, lds + g * STAGE, wdelta);
    else
      issue_stage<F, KTAIL>(g - KT, (int)n, a_nxt, ab_nxt, b_nxt, bb_nxt, plan, lds + g * STAGE, wdelta);
  }
  uint8_t* epi = lds + Cfg<F>::RING;
  int* vote = reinterpret_cast<int*>(epi + EPI_VEC);  // free until the first epilogue
  if (F == F_INT16 && lane == 0) vote[wid] = __builtin_amdgcn_ballot_w64(fl != 0) != 0 ? 1 : 0;
  wait_vmcnt<2 * Cfg<F>::LOADS>();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the vote is in LDS before the barrier
  __builtin_amdgcn_s_barrier();
  const bool bias = F == F_INT16 && (vote[0] | vote[1] | vote[2] | vote[3]) != 0;

  v4i a0[4], b0[4], a1[4], b1[4];
  RawB<F> rw;
  const LdsLane ll = lds_lane<F>(wm, wn, fr, h);
  read_a(lds, ll, 0, a0);
  read_b<F>(lds, ll, 0, rw);
  if (F == F_INT16 && bias)
    convert_b<F, true>(rw, b0, zpc);
  else
    convert_b<F, false>(rw, b0, zpc);

  int g = 0;  // global stage index of the stream
  for (int lt = 0; lt < my_tiles; ++lt) {
    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    // the K loop, one copy per split (uniform over the launch)
    auto k_loop = [&](auto bias_tag) {
      constexpr bool BIAS = decltype(bias_tag)::value;
      for (int kt = 0; kt < KT; ++kt, ++g) {
        // stage g+1 has landed (loads of g+2 may still be in flight); after the barrier it
        // is visible to all waves and nobody reads stage g-1, whose buffer g+3 reuses
        wait_vmcnt<Cfg<F>::LOADS>();
        __builtin_amdgcn_s_barrier();
        if (F == F_UW4 && kt == 0) load_zp(lt + 1, zpn);
        // stage g+3 is stage kt+3 of this tile or stage kt+3-KT of the next one
        const bool same = kt + 3 < KT;
        const int kl = same ? kt + 3 : kt + 3 - KT;
        const int8_t* al = same ? a_cur : a_nxt;
        const uint8_t* bl = same ? b_cur : b_nxt;
        const int64_t abl = same ? ab_cur : ab_nxt;
        const int64_t bbl = same ? bb_cur : bb_nxt;
        uint8_t* ldst = lds + ((g + 3) % kStages) * STAGE;
        const uint8_t* S0 = lds + (g % kStages) * STAGE;
        const uint8_t* S1 = lds + ((g + 1) % kStages) * STAGE;
        // Each half (one 32-deep K sub-step): 16 MFMAs on the current operand set,
        // interleaved one by one with the LDS reads of the next set (first eight MFMAs),
        // the stage's direct loads (spread over both halves) and the conversion of the
        // next set (last eight MFMAs).  sched_barrier fixes the order.
        // sub-step 0 of stage g on set 0; set 1 <- sub-step 1 of stage g
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b0[q & 3], a0[q >> 2], acc[q >> 2][q & 3], 0, 0, 0);
          if (q < 8) read_piece<F>(q, S0, ll, 1, a1, rw);
          if (q >= 8 && q - 8 < (Cfg<F>::LOADS + 1) / 2)
            issue_load<F, KTAIL>(q - 8, (int)n, kl, al, abl, bl, bbl, plan, ldst, wdelta);
          if (q >= 8) convert_piece<F, BIAS>(q - 8, rw, b1, zpc);
          __builtin_amdgcn_sched_barrier(0);
        }
        // sub-step 1 of stage g on set 1; set 0 <- sub-step 0 of stage g+1 (the next
        // tile's first stage after the last stage of this one)
        // (the next tile's set is read only in the last iteration, long after its loads
        // landed: a select in every iteration would wait for them in the first)
        uint32_t zs[4] = {zpc[0], zpc[1], zpc[2], zpc[3]};
        if (F == F_UW4 && kt + 1 == KT) {
          __asm__ volatile("");
#pragma unroll
          for (int u = 0; u < 4; ++u) zs[u] = zpn[u];
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1[q & 3], a1[q >> 2], acc[q >> 2][q & 3], 0, 0, 0);
          if (q < 8) read_piece<F>(q, S1, ll, 0, a0, rw);
          if (q >= 8 && q - 8 + (Cfg<F>::LOADS + 1) / 2 < Cfg<F>::LOADS)
            issue_load<F, KTAIL>(q - 8 + (Cfg<F>::LOADS + 1) / 2, (int)n, kl, al, abl, bl, bbl, plan, ldst, wdelta);
          if (q >= 8) convert_piece<F, BIAS>(q - 8, rw, b0, zs);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    if (F == F_INT16 && bias)
      k_loop(std::true_type{});
    else
      k_loop(std::false_type{});

    // ------------------------------------------------------------ epilogue of tile lt
    int tm, tn;
    tile_coords(lt * G + slot, tiles_m, tiles_n, tm, tn);
    const int64_t t0 = (int64_t)tm * BM;
    const int64_t o0 = (int64_t)tn * OUT;
    float* tok_sx = reinterpret_cast<float*>(epi + EPI_VEC);
    int32_t* tok_rs = reinterpret_cast<int32_t*>(epi + EPI_VEC + 4 * BM);
    float* col_sb = reinterpret_cast<float*>(epi + EPI_VEC + 8 * BM);
    int* col_bias = reinterpret_cast<int*>(epi + EPI_VEC + 12 * BM);  // P16T: rows in the bias split
    {
      const int64_t t = t0 + tid;
      tok_sx[tid] = t < M ? sx[t] : 0.0f;
      if (F == F_INT16 || F == F_P16T) tok_rs[tid] = t < M ? rowsum[t] : 0;
      if (tid < OUT) col_sb[tid] = o0 + tid < d ? sbar[o0 + tid] : 0.0f;
      if (F == F_P16T && tid < OUT) col_bias[tid] = o0 + tid < d ? (int)((split[o0 + tid] >> 1) & 1u) : 0;
    }
    __syncthreads();
    uint8_t* stg = epi + wid * EPI_WAVE;
    constexpr bool TWO = Cfg<F>::TWO;
    constexpr int PASSES = TWO ? 1 : 2;  // 64 outputs of the wave per pass
    const bool vec_ok = (d & 7) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_barrier(0);  // read one slab's accumulators at a time
      const int tl = wm * 128 + i * 32 + fr;  // this lane's token inside the block
      const float sxt = tok_sx[tl];
      const double rs128 = (F == F_INT16 && bias) || F == F_P16T ? 128.0 * (double)tok_rs[tl] : 0.0;  // bias split
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        // outputs of this pass, in MFMA layout: lane l, registers 4a..4a+3 of column tile
        // j are token l % 32 and MFMA columns 32 j + 8 a + 4 (l / 32) + 0..3
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            __builtin_amdgcn_sched_barrier(0);
            const int oc = 32 * jj + 8 * a + 4 * h;                       // output column in the pass
            const int ow = (TWO ? 0 : 64 * p) + oc;                       // output column in the wave
            const float4 sb = *reinterpret_cast<const float4*>(col_sb + (TWO ? wn * 64 : wn * 128) + ow);
            const float sbv[4] = {sb.x, sb.y, sb.z, sb.w};
            int cb[4] = {1, 1, 1, 1};  // INT16: the launch's split applies to every row
            if (F == F_P16T) {
              const int4 b4 = *reinterpret_cast<const int4*>(col_bias + wn * 64 + ow);
              cb[0] = b4.x;
              cb[1] = b4.y;
              cb[2] = b4.z;
              cb[3] = b4.w;
            }
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (TWO) {
                const int hi = acc_read(acc[i][2 * jj][4 * a + e]), lo = acc_read(acc[i][2 * jj + 1][4 * a + e]);
                // exact = 256 acc_hi + acc_lo (+ 128 rowsum for the bias split), exact in
                // binary64 (|exact| < 2^53)
                const double ex = fma(256.0, (double)hi, (double)lo) + (cb[e] ? rs128 : 0.0);
                y[e] = ((float)ex * sxt) * sbv[e];
              } else {
                const int v = acc_read(acc[i][2 * p + jj][4 * a + e]);
                y[e] = ((float)(F == F_INT4 ? (v >> 4) : v) * sxt) * sbv[e];
              }
            }
            const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){y[0], y[1]}, bf2));
            const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){y[2], y[3]}, bf2));
            *reinterpret_cast<uint2*>(stg + fr * EPI_RS + 2 * oc) = make_uint2(p01, p23);
            if (acc_dbg) {
              const int64_t tok = t0 + tl;
              const int64_t c = o0 + (TWO ? wn * 64 : wn * 128) + ow;
              if (tok < M) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  if (c + e >= d) continue;
                  if (TWO) {
                    acc_dbg[tok * d + c + e] = acc_read(acc[i][2 * jj][4 * a + e]);
                    acc_dbg[M * d + tok * d + c + e] = acc_read(acc[i][2 * jj + 1][4 * a + e]);
                  } else if (F == F_P16N) {  // the high plane (all zero) and the low plane
                    acc_dbg[tok * d + c + e] = 0;
                    acc_dbg[M * d + tok * d + c + e] = acc_read(acc[i][2 * p + jj][4 * a + e]);
                  } else {
                    const int v = acc_read(acc[i][2 * p + jj][4 * a + e]);
                    acc_dbg[tok * d + c + e] = F == F_INT4 ? (v >> 4) : v;
                  }
                }
              }
            }
          }
        }
        // (a wave's LDS accesses complete in order: its reads below see its writes)
        // 32 tokens x 64 outputs, read back row-contiguously: 8 lanes x 16 bytes per row
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int row = s4 * 8 + (lane >> 3);
          const int col8 = 8 * (lane & 7);
          const int64_t tok = t0 + wm * 128 + i * 32 + row;
          const int64_t c = o0 + (TWO ? wn * 64 : wn * 128 + 64 * p) + col8;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + row * EPI_RS + 2 * col8);
          if (tok < M && c < d) {
            uint16_t* Yp = Y + tok * d + c;
            if (vec_ok && c + 7 < d) {
              *reinterpret_cast<uint4*>(Yp) = v;
            } else {
              const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (c + e < d) Yp[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
    }
    // the next tile streams in; the one after it becomes "next"
    a_cur = a_nxt;
    b_cur = b_nxt;
    ab_cur = ab_nxt;
    bb_cur = bb_nxt;
    tile_ptrs(lt + 2, a_nxt, ab_nxt, b_nxt, bb_nxt);
    if (F == F_UW4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) zpc[u] = zpn[u];
    }
  }
  wait_vmcnt<0>();  // trailing (zero-reading) loads land before the block's LDS is released
}

template <int F, bool KTAIL>
__global__ __launch_bounds__(lin::kThreads, 1) void k_linear(int64_t M, int64_t d, int64_t n,
                                                            const int8_t* __restrict__ xq,
                                                            const float* __restrict__ sx,
                                                            const int32_t* __restrict__ rowsum,
                                                            const uint8_t* __restrict__ m,
                                                            const uint8_t* __restrict__ split,
                                                            const float* __restrict__ sbar, uint16_t* __restrict__ Y,
                                                            int32_t* __restrict__ acc_dbg, int tiles_m, int tiles_n,
                                                            int64_t wdelta, const int32_t* __restrict__ zbar_p,
                                                            const int32_t* __restrict__ zw_p) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  linear_body<F, KTAIL>(lds, M, d, n, xq, sx, rowsum, m, split, sbar, Y, acc_dbg, tiles_m, tiles_n, wdelta, zbar_p,
                        zw_p);
}

// Byte-plane merged integers: when every row's plane code is 0 (all high bytes zero) and
// the host allows it, the launch multiplies the low planes alone as int8 weights (256
// outputs per tile, the high planes never loaded); otherwise both planes, with the bias
// correction on the rows whose code says so.  Every block reads the codes and votes
// before its first load.  Both bodies give the same integers and outputs; the host
// allows the low-plane body only where its fewer, wider tiles take fewer rounds of the
// persistent grid (with equal rounds the two-plane tiles are as fast or faster: half of
// their products multiply the zero high plane).
template <bool KTAIL>
__global__ __launch_bounds__(lin::kThreads, 1) void k_linear_planes(int64_t M, int64_t d, int64_t n,
                                                                   const int8_t* __restrict__ xq,
                                                                   const float* __restrict__ sx,
                                                                   const int32_t* __restrict__ rowsum,
                                                                   const uint8_t* __restrict__ m,
                                                                   const uint8_t* __restrict__ code,
                                                                   const float* __restrict__ sbar,
                                                                   uint16_t* __restrict__ Y,
                                                                   int32_t* __restrict__ acc_dbg, int tiles_m,
                                                                   int allow_narrow) {
  using namespace lin;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  __shared__ int vote[4];
  const int tid = threadIdx.x;
  const int fl = any_code(code, d);
  if ((tid & 63) == 0) vote[tid >> 6] = 0;
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(fl != 0) != 0 && (tid & 63) == 0) vote[tid >> 6] = 1;
  __syncthreads();
  const bool narrow = allow_narrow && (vote[0] | vote[1] | vote[2] | vote[3]) == 0;
  if (narrow)
    linear_body<F_P16N, KTAIL>(lds, M, d, n, xq, sx, rowsum, m, code, sbar, Y, acc_dbg, tiles_m,
                               (int)((d + Cfg<F_P16N>::OUT - 1) / Cfg<F_P16N>::OUT), 0, nullptr, nullptr);
  else
    linear_body<F_P16T, KTAIL>(lds, M, d, n, xq, sx, rowsum, m, code, sbar, Y, acc_dbg, tiles_m,
                               (int)((d + Cfg<F_P16T>::OUT - 1) / Cfg<F_P16T>::OUT), 0, nullptr, nullptr);
}

// ---------------------------------------------------------------------------------
// Few-token linear layer (M <= 16 TT tokens: decode), bound by streaming the weights.
// A block owns 16 output rows and its 4 waves split K into quarters.  Each 64-deep K
// step is one v_mfma_i32_16x16x64_i8 per plane and token tile, with the weights as the
// A operand (lane l: row l % 16, K 16 (l / 16) .. + 15 of the step) and 16 tokens as B
// (lane l: token l % 16, same K); lane l, register v of the result hold output row
// 4 (l / 16) + v and token l % 16.  Formats as in the tiled kernel: INT16 through the
// same byte split (one split per block of 16 rows, from their split codes), INT4 through the
// same 16 w unpack.  Loads run four steps ahead from clamped (always valid) addresses;
// K chunks past n, and the steps that pad a wave's quarter to a multiple of four, are
// zeroed on the token side.  The four waves' int32 sums are added
// through LDS (exact) and the epilogue is the tiled kernel's.
// ---------------------------------------------------------------------------------
namespace sk {
constexpr int kAhead = 4;  // K steps in flight per wave
}

// Byte planes: P16T multiplies both planes (a row whose plane code has bit 1 set is in
// the bias split); P16N the low planes alone (every high byte of the call is zero).
template <int F, int TT>
__device__ __forceinline__ void skinny_body(int64_t M, int64_t d, int64_t n, const int8_t* __restrict__ xq,
                                            const float* __restrict__ sx, const int32_t* __restrict__ rowsum,
                                            const uint8_t* __restrict__ m, const uint8_t* __restrict__ split,
                                            const float* __restrict__ sbar, uint16_t* __restrict__ Y,
                                            int32_t* __restrict__ acc_dbg, int64_t wdelta,
                                            const int32_t* __restrict__ zbar_p, const int32_t* __restrict__ zw_p) {
  constexpr int PL = (F == F_INT16 || F == F_UW4 || F == F_P16T) ? 2 : 1;  // byte planes
  __shared__ int red[4][PL * TT][4][64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t i0 = (int64_t)blockIdx.x * 16;
  const int rl = lane & 15, kg = lane >> 4;
  const int64_t wr = i0 + rl < d ? i0 + rl : d - 1;  // rows past d: loaded, never stored
  const int64_t KT = (n + 63) / 64;
  const int64_t per = (KT + 3) / 4;
  const int64_t s0 = (int64_t)wid * per;
  const int64_t s1 = s0 + per < KT ? s0 + per : KT;
  const int64_t wrow = (F == F_INT16 || planar(F)) ? 2 * n : (F == F_INT8 ? n : n / 2);
  // UW4: the base codes lie wdelta bytes after U's; the lane's row zero points are fixed
  uint32_t zb2 = 0, zw2 = 0;
  if (F == F_UW4) {
    const uint32_t zb = (uint32_t)zbar_p[wr], zw = (uint32_t)zw_p[wr];
    zb2 = zb | (zb << 16);
    zw2 = zw | (zw << 16);
  }

  struct Step {
    v4i w[2];
    v4i x[TT];
  };
  // loads of step st (clamped into [0, KT) and the matrices; the caller never uses a
  // step outside [s0, s1))
  auto load = [&](int64_t st, Step& S) {
    st = st < KT ? st : KT - 1;
    int64_t k = st * 64 + 16 * kg;
    k = k < n ? k : n - 16;  // n is a multiple of 32: chunks are whole
    if (F == F_INT16) {  // 16 int16
      const v4i* pw = reinterpret_cast<const v4i*>(m + wr * wrow + 2 * k);
      S.w[0] = pw[0];
      S.w[1] = pw[1];
    } else if (F == F_P16T) {  // 16 high bytes, and the same columns' 16 low bytes
      S.w[0] = *reinterpret_cast<const v4i*>(m + wr * wrow + k);
      S.w[1] = *reinterpret_cast<const v4i*>(m + wr * wrow + n + k);
    } else if (F == F_P16N) {  // the 16 low bytes
      S.w[0] = *reinterpret_cast<const v4i*>(m + wr * wrow + n + k);
      S.w[1] = v4i{0, 0, 0, 0};
    } else if (F == F_INT8) {
      S.w[0] = *reinterpret_cast<const v4i*>(m + wr * wrow + k);
      S.w[1] = v4i{0, 0, 0, 0};
    } else if (F == F_UW4) {
      const uint2 qu = *reinterpret_cast<const uint2*>(m + wr * wrow + (k >> 1));
      const uint2 qw = *reinterpret_cast<const uint2*>(
          reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(m) + (uintptr_t)wdelta) + wr * wrow + (k >> 1));
      S.w[0] = v4i{(int)qu.x, (int)qu.y, 0, 0};
      S.w[1] = v4i{(int)qw.x, (int)qw.y, 0, 0};
    } else {
      const uint2 q = *reinterpret_cast<const uint2*>(m + wr * wrow + (k >> 1));
      S.w[0] = v4i{(int)q.x, (int)q.y, 0, 0};
      S.w[1] = v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int64_t t = 16 * tt + rl < M ? 16 * tt + rl : M - 1;  // tokens past M: never stored
      S.x[tt] = *reinterpret_cast<const v4i*>(xq + t * n + k);
    }
  };

  // INT16: the split of the block's own 16 rows (their outputs depend on nothing else):
  // bias when some row's code is 1, or when there are no codes.  Every wave reads the
  // same 16 codes, so the choice is uniform over the block.
  bool bias = false;
  if (F == F_INT16) {
    const int c = split == nullptr ? 1 : (i0 + rl < d ? (int)split[i0 + rl] : 0);
    bias = __builtin_amdgcn_ballot_w64(c != 0) != 0;
  }
  v4i acc[PL][TT];
#pragma unroll
  for (int p = 0; p < PL; ++p)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[p][tt] = v4i{0, 0, 0, 0};

  auto compute = [&](int64_t st, const Step& S, auto bias_tag) {
    constexpr bool BIAS = decltype(bias_tag)::value;
    const bool kin = st < s1 && st * 64 + 16 * kg < n;  // padded steps past the quarter add zeros
    v4i a[PL];
    if (F == F_INT16) {
      const uint32_t x[8] = {(uint32_t)S.w[0].x, (uint32_t)S.w[0].y, (uint32_t)S.w[0].z, (uint32_t)S.w[0].w,
                             (uint32_t)S.w[1].x, (uint32_t)S.w[1].y, (uint32_t)S.w[1].z, (uint32_t)S.w[1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 hl = split16<BIAS>(x[2 * e], x[2 * e + 1]);
        a[0][e] = (int)hl.x;
        a[PL - 1][e] = (int)hl.y;
      }
    } else if (F == F_UW4) {  // m = (u - z_bar)(w - z), balanced split (|m| <= 225)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 mm = uw4_m((uint32_t)S.w[0][e >> 1], (uint32_t)S.w[1][e >> 1], zb2, zw2, e & 1);
        const uint2 hl = split16<false>(mm.x, mm.y);
        a[0][e] = (int)hl.x;
        a[PL - 1][e] = (int)hl.y;
      }
    } else if (F == F_P16T) {
      a[0] = S.w[0];
      a[PL - 1] = S.w[1];
    } else if (F == F_INT8 || F == F_P16N) {
      a[0] = S.w[0];
    } else {
      uint32_t o0, o1, o2, o3;
      unpack4((uint32_t)S.w[0].x, o0, o1);
      unpack4((uint32_t)S.w[0].y, o2, o3);
      a[0] = v4i{(int)o0, (int)o1, (int)o2, (int)o3};
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const v4i xv = kin ? S.x[tt] : v4i{0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < PL; ++p) acc[p][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[p], xv, acc[p][tt], 0, 0, 0);
    }
  };

  // a ring of kAhead steps: each step's buffer is refilled with the step kAhead later
  // as soon as it has been used (no branch in the body, so the loads stay in flight)
  auto k_loop = [&](auto bias_tag) {
    Step buf[sk::kAhead];
#pragma unroll
    for (int q = 0; q < sk::kAhead; ++q) load(s0 + q, buf[q]);
    for (int64_t st = s0; st < s1; st += sk::kAhead) {
#pragma unroll
      for (int q = 0; q < sk::kAhead; ++q) {
        compute(st + q, buf[q], bias_tag);
        load(st + q + sk::kAhead, buf[q]);
      }
    }
  };
  if (F == F_INT16 && bias)
    k_loop(std::true_type{});
  else
    k_loop(std::false_type{});

  // the four K quarters, added in LDS (exact)
#pragma unroll
  for (int p = 0; p < PL; ++p)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wid][p * TT + tt][v][lane] = acc[p][tt][v];
  __syncthreads();
  for (int x = tid; x < TT * 4 * 64; x += 256) {
    const int tt = x / 256, v = (x / 64) & 3, l = x & 63;
    const int64_t row = i0 + 4 * (l >> 4) + v;
    const int64_t t = 16 * tt + (l & 15);
    if (row >= d || t >= M) continue;
    int pv[PL];
#pragma unroll
    for (int p = 0; p < PL; ++p)
      pv[p] = red[0][p * TT + tt][v][l] + red[1][p * TT + tt][v][l] + red[2][p * TT + tt][v][l] +
              red[3][p * TT + tt][v][l];
    float y;
    if (F == F_INT16 || F == F_UW4 || F == F_P16T) {
      const bool brow = F == F_P16T ? ((split[row] >> 1) & 1u) != 0 : bias;
      const double rs128 = brow ? 128.0 * (double)rowsum[t] : 0.0;
      const double ex = fma(256.0, (double)pv[0], (double)pv[PL - 1]) + rs128;
      y = ((float)ex * sx[t]) * sbar[row];
    } else {
      y = ((float)(F == F_INT4 ? (pv[0] >> 4) : pv[0]) * sx[t]) * sbar[row];
    }
    const uint32_t b2 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){y, y}, bf2));
    Y[t * d + row] = (uint16_t)(b2 & 0xFFFFu);
    if (acc_dbg) {
      if (F == F_P16N) {  // the high plane (all zero) and the low plane
        acc_dbg[t * d + row] = 0;
        acc_dbg[M * d + t * d + row] = pv[0];
      } else {
#pragma unroll
        for (int p = 0; p < PL; ++p) acc_dbg[(int64_t)p * M * d + t * d + row] = F == F_INT4 ? (pv[p] >> 4) : pv[p];
      }
    }
  }
}

template <int F, int TT>
__global__ __launch_bounds__(256) void k_linear_skinny(int64_t M, int64_t d, int64_t n, const int8_t* __restrict__ xq,
                                                      const float* __restrict__ sx,
                                                      const int32_t* __restrict__ rowsum,
                                                      const uint8_t* __restrict__ m,
                                                      const uint8_t* __restrict__ split,
                                                      const float* __restrict__ sbar, uint16_t* __restrict__ Y,
                                                      int32_t* __restrict__ acc_dbg, int64_t wdelta,
                                                      const int32_t* __restrict__ zbar_p,
                                                      const int32_t* __restrict__ zw_p) {
  skinny_body<F, TT>(M, d, n, xq, sx, rowsum, m, split, sbar, Y, acc_dbg, wdelta, zbar_p, zw_p);
}

// Byte planes at few tokens: a block multiplies the low planes alone when the plane codes
// of its 16 rows are all 0.
template <int TT>
__global__ __launch_bounds__(256) void k_linear_skinny_planes(int64_t M, int64_t d, int64_t n,
                                                             const int8_t* __restrict__ xq,
                                                             const float* __restrict__ sx,
                                                             const int32_t* __restrict__ rowsum,
                                                             const uint8_t* __restrict__ m,
                                                             const uint8_t* __restrict__ code,
                                                             const float* __restrict__ sbar, uint16_t* __restrict__ Y,
                                                             int32_t* __restrict__ acc_dbg) {
  // the plane codes of the block's own 16 rows (read by every wave: a uniform choice)
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  const int c = r < d ? (int)code[r] : 0;
  if (__builtin_amdgcn_ballot_w64(c != 0) == 0)
    skinny_body<F_P16N, TT>(M, d, n, xq, sx, rowsum, m, code, sbar, Y, acc_dbg, 0, nullptr, nullptr);
  else
    skinny_body<F_P16T, TT>(M, d, n, xq, sx, rowsum, m, code, sbar, Y, acc_dbg, 0, nullptr, nullptr);
}

// Blocks of the persistent grid for `tiles` tiles of K depth KT: one per compute unit,
// except that when the tiles take more than one round and some block count between
// 3/4 of the units and all of them divides the tiles into the same number of whole
// rounds, that count is used (every block then owns the same number of tiles, and the
// idle units draw no power while the others run).  A short K (fewer than 3 stages) runs
// one block per tile.
static unsigned persistent_grid(int tiles, int KT, int cus) {
  if (KT < 3 || tiles <= cus) return (unsigned)tiles;
  const int rounds = (tiles + cus - 1) / cus;
  for (int c = cus; c >= cus * 3 / 4; --c)
    if (tiles % c == 0 && tiles / c == rounds) return (unsigned)c;
  return (unsigned)cus;
}

static int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

static hipError_t set_linear_attrs() {
  using namespace lin;
  static bool attr_set = false;
  if (attr_set) return hipSuccess;
  const void* fns[10] = {reinterpret_cast<const void*>(&k_linear<F_INT8, false>),
                        reinterpret_cast<const void*>(&k_linear<F_INT8, true>),
                        reinterpret_cast<const void*>(&k_linear<F_INT4, false>),
                        reinterpret_cast<const void*>(&k_linear<F_INT4, true>),
                        reinterpret_cast<const void*>(&k_linear<F_INT16, false>),
                        reinterpret_cast<const void*>(&k_linear<F_INT16, true>),
                        reinterpret_cast<const void*>(&k_linear<F_UW4, false>),
                        reinterpret_cast<const void*>(&k_linear<F_UW4, true>),
                        reinterpret_cast<const void*>(&k_linear_planes<false>),
                        reinterpret_cast<const void*>(&k_linear_planes<true>)};
  static_assert(Cfg<F_P16T>::LDS >= Cfg<F_P16N>::LDS, "the planes kernel sizes its LDS for both forms");
  const int lds_of[10] = {Cfg<F_INT8>::LDS, Cfg<F_INT8>::LDS, Cfg<F_INT4>::LDS, Cfg<F_INT4>::LDS,
                          Cfg<F_INT16>::LDS, Cfg<F_INT16>::LDS, Cfg<F_UW4>::LDS, Cfg<F_UW4>::LDS,
                          Cfg<F_P16T>::LDS, Cfg<F_P16T>::LDS};
  for (int k = 0; k < 10; ++k) {
    const hipError_t e = hipFuncSetAttribute(fns[k], hipFuncAttributeMaxDynamicSharedMemorySize, lds_of[k]);
    if (e != hipSuccess) return e;
  }
  attr_set = true;
  return hipSuccess;
}

// One block per compute unit, each streaming several tiles; with fewer than three K
// stages per tile the stream cannot span tiles, so every block takes one tile.
template <int FMT>
static hipError_t launch_fmt(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx,
                             const int32_t* rowsum, const uint8_t* mb, const uint8_t* split, const float* sbar,
                             uint16_t* Y, int32_t* acc_dbg, int64_t wdelta, const int32_t* zbar,
                             const int32_t* zw, hipStream_t st) {
  using namespace lin;
  const hipError_t e = set_linear_attrs();
  if (e != hipSuccess) return e;
  if (M <= 32) {  // few tokens: weight streaming
    const dim3 g((unsigned)((d + 15) / 16));
    if (M <= 16)
      hipLaunchKernelGGL((k_linear_skinny<FMT, 1>), g, dim3(256), 0, st, M, d, n, xq, sx, rowsum, mb, split, sbar, Y,
                         acc_dbg, wdelta, zbar, zw);
    else
      hipLaunchKernelGGL((k_linear_skinny<FMT, 2>), g, dim3(256), 0, st, M, d, n, xq, sx, rowsum, mb, split, sbar, Y,
                         acc_dbg, wdelta, zbar, zw);
    return hipGetLastError();
  }
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((d + Cfg<FMT>::OUT - 1) / Cfg<FMT>::OUT);
  const int ntile = tiles_m * tiles_n;
  const int KT = (int)((n + BK - 1) / BK);
  const int cus = device_cus();
  const dim3 grid(persistent_grid(ntile, KT, cus));
  if ((n % BK) != 0)
    hipLaunchKernelGGL((k_linear<FMT, true>), grid, dim3(kThreads), Cfg<FMT>::LDS, st, M, d, n, xq, sx, rowsum, mb,
                       split, sbar, Y, acc_dbg, tiles_m, tiles_n, wdelta, zbar, zw);
  else
    hipLaunchKernelGGL((k_linear<FMT, false>), grid, dim3(kThreads), Cfg<FMT>::LDS, st, M, d, n, xq, sx, rowsum, mb,
                       split, sbar, Y, acc_dbg, tiles_m, tiles_n, wdelta, zbar, zw);
  return hipGetLastError();
}

// Byte-plane merged integers: the grid is sized for the two-plane tiles (128 outputs);
// the low-plane form has half as many tiles and the extra blocks find none.
static hipError_t launch_planes(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx,
                                const int32_t* rowsum, const uint8_t* mb, const uint8_t* code, const float* sbar,
                                uint16_t* Y, int32_t* acc_dbg, hipStream_t st) {
  using namespace lin;
  const hipError_t e = set_linear_attrs();
  if (e != hipSuccess) return e;
  if (M <= 32) {
    const dim3 g((unsigned)((d + 15) / 16));
    if (M <= 16)
      hipLaunchKernelGGL((k_linear_skinny_planes<1>), g, dim3(256), 0, st, M, d, n, xq, sx, rowsum, mb, code, sbar, Y,
                         acc_dbg);
    else
      hipLaunchKernelGGL((k_linear_skinny_planes<2>), g, dim3(256), 0, st, M, d, n, xq, sx, rowsum, mb, code, sbar, Y,
                         acc_dbg);
    return hipGetLastError();
  }
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int ntile = tiles_m * (int)((d + Cfg<F_P16T>::OUT - 1) / Cfg<F_P16T>::OUT);
  const int ntile_n = tiles_m * (int)((d + Cfg<F_P16N>::OUT - 1) / Cfg<F_P16N>::OUT);
  const int KT = (int)((n + BK - 1) / BK);
  const int cus = device_cus();
  // the low-plane body only where its wider tiles take fewer rounds of a full grid
  const int gf = KT >= 3 && ntile > cus ? cus : ntile;
  const int allow_narrow = (ntile_n + gf - 1) / gf < (ntile + gf - 1) / gf ? 1 : 0;
  const dim3 grid(persistent_grid(allow_narrow ? ntile_n : ntile, KT, cus));
  if ((n % BK) != 0)
    hipLaunchKernelGGL((k_linear_planes<true>), grid, dim3(kThreads), Cfg<F_P16T>::LDS, st, M, d, n, xq, sx, rowsum,
                       mb, code, sbar, Y, acc_dbg, tiles_m, allow_narrow);
  else
    hipLaunchKernelGGL((k_linear_planes<false>), grid, dim3(kThreads), Cfg<F_P16T>::LDS, st, M, d, n, xq, sx, rowsum,
                       mb, code, sbar, Y, acc_dbg, tiles_m, allow_narrow);
  return hipGetLastError();
}

hipError_t launch_linear(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx, const int32_t* rowsum,
                         int wfmt, const void* m, const uint8_t* split, const float* sbar, uint16_t* Y,
                         int32_t* acc_dbg, hipStream_t st) {
  const uint8_t* mb = static_cast<const uint8_t*>(m);
  switch (wfmt) {
    case F_P16T:
      return launch_planes(M, d, n, xq, sx, rowsum, mb, split, sbar, Y, acc_dbg, st);
    case F_INT8:
      return launch_fmt<F_INT8>(M, d, n, xq, sx, rowsum, mb, split, sbar, Y, acc_dbg, 0, nullptr, nullptr, st);
    case F_INT4:
      return launch_fmt<F_INT4>(M, d, n, xq, sx, rowsum, mb, split, sbar, Y, acc_dbg, 0, nullptr, nullptr, st);
    default:
      return launch_fmt<F_INT16>(M, d, n, xq, sx, rowsum, mb, split, sbar, Y, acc_dbg, 0, nullptr, nullptr, st);
  }
}

hipError_t launch_linear_codes(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx,
                               const uint8_t* ucode, const uint8_t* wcode, const int32_t* z, const int32_t* zbar,
                               const float* sbar, uint16_t* Y, int32_t* acc_dbg, hipStream_t st) {
  const int64_t wdelta = (int64_t)(reinterpret_cast<uintptr_t>(wcode) - reinterpret_cast<uintptr_t>(ucode));
  return launch_fmt<F_UW4>(M, d, n, xq, sx, nullptr, ucode, nullptr, sbar, Y, acc_dbg, wdelta, zbar, z, st);
}

}  // namespace intlora
