// Internal launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace intlora {

struct AdaptArgs {
  int64_t d, n;
  int r, w_bits;
  uint64_t seed;
  uint32_t layer_id;
  const uint8_t* wround;
  const int32_t* z;
  const float* s;
  const float* c;
  const float* A;
  const float* B;
  float* U;
  int* pmin;  // order keys of the U range per (partial column, row), column-major: pmin[col * d + row]
  int* pmax;
  unsigned long long* sat_zero;  // zeroed by the adaptation kernel (nullable)
  bool ptq;                      // x = (s w + R*) + AB for every element (comparison path) instead of U
  bool force_generic;
  int dist;                      // auxiliary-matrix distribution (kAuxLaplace ... kAuxStudentT2)
  int64_t row0 = 0;              // global index of row 0 of these pointers (R's counter uses i + row0)
};

// Fused single-pass MUL merge (no scratch); hipErrorInvalidValue for n > 16384.
hipError_t launch_merge_fused(const AdaptArgs& a, int u_bits, int16_t* m, float* sbar, int32_t* zbar,
                              uint8_t* split, uint8_t* uround_dbg, unsigned long long* sat, hipStream_t st);

// Upper bound of the number of column tiles of the adaptation kernel (sizes the
// workspace of row partials).
int adapt_max_ntiles(int64_t n);

hipError_t launch_gen_r(int64_t d, int64_t n, uint64_t seed, uint32_t layer_id, const float* c, float* out, int dist,
                        hipStream_t st);
hipError_t launch_ln_odd(int64_t count, const uint32_t* G, float* out, hipStream_t st);
hipError_t launch_debug_mfma_chain(int form, int64_t d, int64_t n, int r, const float* A, const float* B, float* out,
                                   hipStream_t st);
hipError_t launch_aux_debug(int64_t blocks, const uint32_t* words, int dist, float* out, hipStream_t st);
hipError_t launch_sigma_w(int64_t d, int64_t n, const float* W, float* sigma, hipStream_t st);
hipError_t launch_vmc_scale(int64_t d, const float* sigma, double alpha, float* c, int dist, hipStream_t st);
hipError_t launch_base_quant(int64_t d, int64_t n, int bits, uint64_t seed, uint32_t layer_id, const float* W,
                             const float* c, uint8_t* wround, int32_t* z, float* s, int dist, hipStream_t st);
hipError_t launch_quant_act(int64_t M, int64_t n, const float* X, int8_t* xq, float* sx, int32_t* rowsum,
                            hipStream_t st);
hipError_t launch_adapt(const AdaptArgs& a, int* ntiles_out, hipStream_t st);
hipError_t launch_row_range(int64_t d, int ntiles, const int* pmin, const int* pmax, float* umin, float* umax,
                            uint8_t* split, hipStream_t st);
// Per-row MUL quantizer parameters (range, s_bar, z_bar, RN(1/s_bar), small-row flag);
// umin_in / umax_in: the caller's range, or NULL to reduce the partials.
hipError_t launch_mul_params(int64_t d, int ntiles, const int* pmin, const int* pmax, const float* umin_in,
                             const float* umax_in, float* umin_out, float* umax_out, int u_bits, int w_bits,
                             const int32_t* z, float* sbar, int32_t* zbar, float* rs, int* small, uint8_t* split,
                             bool planes, hipStream_t st);
// m: int16 d x n, or (planes) the byte-plane layout d x 2n with split = the plane codes.
hipError_t launch_quant_mul(int64_t d, int64_t n, int w_bits, int u_bits, const uint8_t* wround, const int32_t* z,
                            const float* U, const float* sbar, const int32_t* zbar, const float* rs,
                            const int* small, void* m, uint8_t* split, uint8_t* uround_dbg,
                            unsigned long long* sat, uint8_t* ucode, bool planes, hipStream_t st);
hipError_t launch_quant_ptq(int64_t d, int64_t n, int bits, const float* X, const float* xmin, const float* xmax,
                            uint8_t* code, float* s_out, int32_t* z_out, hipStream_t st);
hipError_t launch_quant_shift(int64_t d, int64_t n, int w_bits, int v_bits, const uint8_t* wround, const int32_t* z,
                              const float* U, const float* umin, const float* umax, uint8_t* m, float* sbar,
                              uint8_t* shift_dbg, unsigned long long* sat, hipStream_t st);
// Straight-through backward (ste.hip): launch geometry, workspace and launcher.
struct SteSplits {
  int S;                   // column chunks (partial sums of dA)
  int64_t cols_per_split;  // the chunk width
  int S2;                  // row ranges (partial sums of dB)
  int64_t rows_per_split;  // a multiple of the row tile
};
SteSplits ste_splits(int64_t d, int64_t n, int r);
size_t ste_ws_bytes(int64_t d, int64_t n, int r);
hipError_t launch_ste_backward(int64_t d, int64_t n, int r, int w_bits, const uint8_t* wround, const int32_t* z,
                               const float* A, const float* B, const float* G, float* dA, float* dB, void* ws,
                               hipStream_t st);
hipError_t launch_linear(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx, const int32_t* rowsum,
                         int wfmt, const void* m, const uint8_t* split, const float* sbar, uint16_t* Y,
                         int32_t* acc_dbg, hipStream_t st);
hipError_t launch_linear_codes(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* sx,
                               const uint8_t* ucode, const uint8_t* wcode, const int32_t* z, const int32_t* zbar,
                               const float* sbar, uint16_t* Y, int32_t* acc_dbg, hipStream_t st);

}  // namespace intlora
