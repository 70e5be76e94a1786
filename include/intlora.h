/*
 * intlora.h -- C ABI of libintlora.so: the IntLoRA integer merge and the W8A8 / W4A8
 * integer linear layer that consumes the merged integers, on AMD Instinct MI355X
 * (gfx950).
 *
 * Method: "IntLoRA: Integral Low-rank Adaptation of Quantized Diffusion Models"
 * (Paper-Notes, ICML 2025):
 *   section "1. AQS"  W' = Q[W - sg(R)] + sg(R) + AB; R regenerated from statistics
 *                     and a fixed seed, so it is never stored;
 *   section "2. MLA"  W' = [s I + (R + AB) / (W_round - z)] (.) (W_round - z);
 *   section "3. VMC"  R* = r^alpha R with r = sigma_W / sigma_R;
 *   section "two implementation variants":
 *                     MUL   W' = s_bar (U_round - z_bar) (.) (W_round - z),
 *                     SHIFT W' = sign(V) (.) [(W_round - z) >> shift];
 *   section "training and inference efficiency": the merged integers are the
 *                     deployed W8A8 / W4A8 weights, with no post-training quantization.
 * The Laplace law of R follows the auxiliary-matrix ablation of the atlas.scime.ai
 * summary of the same paper; per-token activation scales with per-channel weight
 * scales follow "implementation details" of the SVDQuant article (8-bit setting).
 *
 * Conventions shared by every entry point
 *  - W is d x n (out_features x in_features), row-major.  "Row" = output channel.
 *  - All array pointers are DEVICE pointers owned by the caller, except `desc`
 *    and the `intlora_base` / `intlora_lora` structs themselves (host structs holding
 *    device pointers).  The library allocates no memory and keeps no state between
 *    calls; scratch memory is the caller's workspace (`ws`, `ws_bytes`, sized by
 *    intlora_workspace_bytes()).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *    call only enqueues work; outputs are valid after the caller synchronizes the
 *    stream.  The status reports host-side validation and launch errors.
 *  - Sizes are int64; 0 rows / 0 tokens are valid no-ops (n must be >= 1).
 *  - Codes: 8-bit codes are one uint8 per element; 4-bit codes are packed two per
 *    byte, low nibble = even column, row stride n/2 bytes (n must be even).
 *  - Pointers must be 16-byte aligned (INTLORA_EALIGN otherwise).
 *  - Results are deterministic and independent of launch geometry: R depends only
 *    on (seed, layer_id, i, j), so any row block regenerates the same values.
 *  - Readings of points the pages leave open (the quantizer form, the w == 0
 *    convention, the SHIFT scale, the counter layout of R, ...) are stated at each
 *    entry point below.
 *  - On error the call enqueues nothing and intlora_last_error() returns a
 *    thread-local description.
 */
#ifndef INTLORA_H
#define INTLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum intlora_status {
  INTLORA_OK = 0,
  INTLORA_EINVAL = 1,     /* null pointer or argument out of range (bit width, rank, alpha, mode) */
  INTLORA_ESHAPE = 2,     /* unsupported or inconsistent sizes                                   */
  INTLORA_EALIGN = 3,     /* a pointer is not 16-byte aligned                                    */
  INTLORA_EWORKSPACE = 4, /* workspace missing or smaller than intlora_workspace_bytes()         */
  INTLORA_EDEVICE = 5,    /* no usable gfx950 device                                             */
  INTLORA_ELAUNCH = 6     /* a kernel launch failed (hipGetLastError)                            */
};

/* intlora_stats modes */
enum { INTLORA_SIGMA_W = 0, INTLORA_U_MINMAX = 1 };

/* merged-weight formats for intlora_linear_fwd */
enum {
  INTLORA_W_INT4 = 4,  /* SHIFT, b_W = 4: packed signed nibbles (two's complement)            */
  INTLORA_W_INT8 = 8,  /* SHIFT, b_W = 8: int8                                                */
  INTLORA_W_INT16 = 16, /* MUL: int16 merged integers (U_round - z_bar) * (W_round - z)       */
  INTLORA_W_INT16_PLANES = 17 /* MUL: the same integers stored as their two int8 byte planes,
                                 as intlora_merge_mul_planes writes them                      */
};

/* operations for intlora_workspace_bytes */
enum {
  INTLORA_OP_STATS_UMINMAX = 1,
  INTLORA_OP_MERGE_MUL = 2,
  INTLORA_OP_MERGE_SHIFT = 3,
  INTLORA_OP_LINEAR = 4,
  INTLORA_OP_BASE_QUANT = 5,
  INTLORA_OP_MERGE_PTQ = 6,
  INTLORA_OP_STE_BACKWARD = 7
};

/* Auxiliary-matrix distributions (the pages' IntLoRA ablation on the law of R, summary
 * table "Measured effects": Laplace against Gaussian, Cauchy and Student-t samples).
 * Laplace is the method's choice and the default (0). */
enum {
  INTLORA_AUX_LAPLACE = 0,   /* Laplace(0, 1)                                                  */
  INTLORA_AUX_GAUSS = 1,     /* N(0, 1), Box-Muller                                            */
  INTLORA_AUX_CAUCHY = 2,    /* Cauchy(0, 1)                                                   */
  INTLORA_AUX_STUDENT_T2 = 3 /* Student-t with 2 degrees of freedom                            */
};

/* One pretrained layer.  r is the LoRA rank (1..128); w_bits the base code width
 * (4 or 8); (seed, layer_id) select the auxiliary-matrix stream and aux_dist its law. */
typedef struct intlora_desc {
  int64_t d;         /* out_features (rows)                             */
  int64_t n;         /* in_features (columns)                           */
  int32_t r;         /* LoRA rank                                       */
  int32_t w_bits;    /* 4 or 8                                          */
  uint64_t seed;     /* Philox key                                      */
  uint32_t layer_id; /* Philox counter word 2                           */
  uint32_t aux_dist; /* INTLORA_AUX_*; other values give INTLORA_EINVAL */
} intlora_desc;

/* Stored state of a quantized base layer (AQS: Q[W - R*] with R* regenerated). */
typedef struct intlora_base {
  const void* w_round;  /* codes of W - R*: uint8 d x n (w_bits 8) or packed d x n/2 (w_bits 4) */
  const int32_t* z;     /* [d] zero points, each in [0, 2^w_bits - 1] as intlora_base_quant
                           writes them.  The merges stay exact for any int32 z (rows whose z
                           is outside [0, 255] take the IEEE division); the merge-on-load
                           linear layer needs z in [0, 15].                                 */
  const float* s;       /* [d] scales                                                            */
  const float* vmc_c;   /* [d] VMC scale c_i = (sigma_W,i / sigma_R)^alpha, from intlora_vmc_scale */
} intlora_base;

/* LoRA factors in fp32 (floating point during tuning). */
typedef struct intlora_lora {
  const float* A; /* d x r row-major */
  const float* B; /* r x n row-major */
} intlora_lora;

/* ---------------------------------------------------------------------------- */
const char* intlora_status_string(int status);
/* Thread-local text of the last error returned on this thread ("" if none). */
const char* intlora_last_error(void);
/* Library ABI version (major * 100 + minor). */
int intlora_version(void);

/* Workspace bytes needed by `op` for a layer (M tokens for INTLORA_OP_LINEAR).
 * Returns 0 for ops that need none.  MUL/SHIFT merge and U statistics: the fp32
 * adaptation term U (4 d n bytes) plus per-tile row partials. */
size_t intlora_workspace_bytes(int op, const intlora_desc* desc, int64_t M);

/* ---------------------------------------------------------------------------- */
/* Auxiliary matrix (section "1. AQS" with section "3. VMC"):
 *   R*_ij = c_i * L_ij,  L_ij ~ Laplace(0, 1) by the inverse CDF
 *   L = -sign(v) ln(1 - 2|v|), v = u - 1/2, u = (2 floor(x / 2^9) + 1) 2^-24,
 *   x = word (q & 3) of Philox4x32-10 with counter (q >> 2 [64 bits], layer_id, 0)
 *   and key (seed low, seed high), q = i*n + j.  ln is correctly rounded to binary32,
 *   R* = RN32(c_i * L).  r_out: d x n fp32.  Uses desc->d, n, seed, layer_id, aux_dist.
 * The other laws (desc->aux_dist) take the same u of each element; every step below is
 * one binary32 rounding of the exact value (ln, cos, sin, tan correctly rounded):
 *   Gaussian: Box-Muller within word pairs (0, 1) and (2, 3) of the block: with u1 from
 *     the pair's first word and u2 from its second, S = sqrt(-2 ln u1), element 2p gets
 *     S cos(2 pi u2) and element 2p + 1 gets S sin(2 pi u2);
 *   Cauchy: tan(pi (u - 1/2));
 *   Student-t(2): (2u - 1) / sqrt(2u (1 - u)), its inverse distribution function. */
int intlora_gen_r(const intlora_desc* desc, const float* vmc_c, float* r_out, void* stream);

/* Per-row statistics.
 *  INTLORA_SIGMA_W:  out0[d] = population std of each row of the fp32 weight W
 *                    (binary64 accumulation, rounded to binary32; base/lora unused).
 *                    The VMC statistic of section "3. VMC", per output channel.
 *  INTLORA_U_MINMAX: out0[d] = U_min, out1[d] = U_max of the adaptation term
 *                    U = s + (R* + AB) / w over the row's valid elements
 *                    (w = W_round - z != 0); +inf / -inf for a row with none.
 *                    Needs base, lora and the workspace. */
int intlora_stats(const intlora_desc* desc, int mode, const float* W, const intlora_base* base,
                  const intlora_lora* lora, float* out0, float* out1, void* ws, size_t ws_bytes, void* stream);

/* VMC scale (section "3. VMC"): c_out[i] = RN32((sigma_w[i] / sqrt(2))^alpha); sigma_R =
 * sqrt(2) is the standard deviation of the unit Laplace law.  alpha in [0, 8]. */
int intlora_vmc_scale(int64_t d, const float* sigma_w, double alpha, float* c_out, void* stream);

/* The same for the auxiliary law aux_dist (the IntLoRA summary's distribution ablation;
 * section "3. VMC" for the scale): c_out[i] = RN32((sigma_w[i] / sigma_R)^alpha) in
 * binary64, sigma_R = sqrt(2) for Laplace and 1 for the others (the Gaussian's standard
 * deviation; the unit scale of the Cauchy and Student-t(2) laws, which have no finite
 * variance).  sigma_w and c_out: d fp32 device values, caller-owned.  INTLORA_EINVAL for
 * an unknown law or alpha outside [0, 8]; d = 0 returns INTLORA_OK without touching the
 * device. */
int intlora_vmc_scale_dist(int64_t d, const float* sigma_w, double alpha, uint32_t aux_dist, float* c_out,
                           void* stream);

/* Base quantization Q[W - R*] (section "1. AQS"), per row, asymmetric with a range
 * that always contains 0:  x = W - R*, lo = min(0, min x), hi = max(0, max x),
 * s = (hi - lo) / (2^b - 1) (1 if that is 0), z = clamp(rint(-lo / s), 0, 2^b - 1),
 * W_round = clamp(rint(x / s) + z, 0, 2^b - 1); rint = half to even; every step IEEE
 * binary32.  Outputs w_round (uint8 d x n, or packed d x n/2), z_out[d], s_out[d].
 * n <= 32768 (the row is staged in LDS).  No workspace. */
int intlora_base_quant(const intlora_desc* desc, const float* W, const float* vmc_c, void* w_round_out,
                       int32_t* z_out, float* s_out, void* stream);

/* IntLoRA_MUL merge (section "two implementation variants", MUL).  Per element with
 * w = W_round - z != 0: acc = fma chain of A[i,k] B[k,j] for k = 0..r-1 from +0,
 * U = s_i + (R*_ij + acc) / w (binary32, IEEE division).  Per row, over the range
 * (U_min, U_max) -- the least and greatest valid U of the row, or, when the caller
 * passes u_min and u_max ([d] fp32 each; both or neither), those values instead (for
 * a caller that already holds the range, e.g. from intlora_stats): lo = min(U_min, 0),
 * hi = max(U_max, 0), s_bar = (hi - lo) / (2^u_bits - 1) (1 unless positive),
 * z_bar = clamp(rint(-lo / s_bar), 0, 2^u_bits - 1); U_round = clamp(rint(U / s_bar) +
 * z_bar, 0, 2^u_bits - 1); m = (U_round - z_bar) * w stored as int16, saturating
 * (counted).  Reading for w == 0 (zero MLA denominator): excluded from the range,
 * U_round = z_bar, m = 0.  The merged weight is s_bar_i * m_ij.
 * Outputs: m (int16 d x n), s_bar[d], z_bar[d]; optional (NULL to skip):
 * m_split[d] (uint8 per row: 1 if some m of the row is >= 32640, else 0 -- the split
 * codes intlora_linear_fwd takes), u_round_dbg (uint8 d x n), sat_count (one uint64,
 * overwritten with the number of saturated elements).  u_bits in [2, 8].
 * Workspace: INTLORA_OP_MERGE_MUL. */
int intlora_merge_mul(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int u_bits,
                      const float* u_min, const float* u_max, int16_t* m, float* s_bar, int32_t* z_bar,
                      uint8_t* m_split, uint8_t* u_round_dbg, unsigned long long* sat_count, void* ws,
                      size_t ws_bytes, void* stream);

/* MUL merge writing the merged integers already split into the two int8 planes the
 * integer linear layer multiplies ([IntLoRA notes] "two implementation variants", MUL;
 * the int16 merged integers go through the int8 matrix cores as two byte planes), so
 * the layer reads them without any conversion (format INTLORA_W_INT16_PLANES).  The
 * same computation as intlora_merge_mul up to m; then, per row, the split is chosen
 * before any element is written, from a bound on the row's merged integers:
 *   bound_i = max(|z_i|, |2^w_bits - 1 - z_i|) * max(z_bar_i, 2^u_bits - 1 - z_bar_i);
 *   bound_i <= 32639: balanced split hi = (m + 128) >> 8, lo = m - 256 hi (m = 256 hi + lo);
 *   otherwise:        bias split hi = m >> 8, lo = (m & 0xFF) - 128 (m = 256 hi + lo + 128).
 * Layout m_planes (uint8, d x 2n): per row, the row's n high bytes in column order,
 * then its n low bytes (two's complement), so that a call whose high planes are all
 * zero streams whole runs of low bytes.  plane_code[d] (uint8):
 * 0 = balanced and every high byte of the row is zero (-128 <= m <= 127: the high plane adds
 * nothing), 1 = balanced, 3 = bias split.  n must be a multiple of 16 (INTLORA_ESHAPE).
 * Other arguments, outputs and workspace as intlora_merge_mul (whose split codes
 * plane_code replaces). */
int intlora_merge_mul_planes(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora,
                             int u_bits, const float* u_min, const float* u_max, uint8_t* m_planes, float* s_bar,
                             int32_t* z_bar, uint8_t* plane_code, uint8_t* u_round_dbg,
                             unsigned long long* sat_count, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free MUL merge, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The same computation and outputs, bit for bit, as intlora_merge_mul
 * (every argument as there), with the scratch taken from a 64 MiB array the library
 * holds on each device until the process ends; nothing is allocated.  Layers whose
 * scratch does not fit are merged in row chunks (R depends on (seed, layer_id, i, j)
 * only, so a chunk regenerates its own rows).  INTLORA_ESHAPE when 32 rows do not fit
 * (n above about 500 000).  Every call on a device shares that device's array, so
 * calls that overlap on one device (other streams, other host threads) race and give
 * wrong results; calls ordered on one stream are safe.  The first call on a device
 * looks the array's address up (hipGetSymbolAddress). */
int intlora_merge_mul_noalloc(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora,
                              int u_bits, const float* u_min, const float* u_max, int16_t* m, float* s_bar,
                              int32_t* z_bar, uint8_t* m_split, uint8_t* u_round_dbg, unsigned long long* sat_count,
                              void* stream);

/* Fused single-pass MUL merge with no scratch memory: the same outputs, bit for bit, as
 * intlora_merge_mul ([IntLoRA notes] "1. AQS", "2. MLA", "两种实现版本" MUL), computed
 * by one kernel in which a block keeps whole rows of U on chip, so U is never written
 * to memory and no workspace is taken.  The rank-r term runs on the vector ALU (the
 * same fma chain as the definition).  n <= 16384 (INTLORA_ESHAPE otherwise); other
 * arguments as intlora_merge_mul. */
int intlora_merge_mul_fused(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int u_bits,
                            int16_t* m, float* s_bar, int32_t* z_bar, uint8_t* m_split, uint8_t* u_round_dbg,
                            unsigned long long* sat_count, void* stream);

/* MUL merge that keeps U's codes instead of the merged integers, for the merge-on-load
 * linear layer (intlora_linear_fwd_codes): the same computation as intlora_merge_mul up
 * to U_round ([IntLoRA notes] "两种实现版本", MUL), which is stored as packed nibbles
 * (u_code d x n/2, low nibble = even column; z_bar where w = 0), with s_bar[d] and
 * z_bar[d].  The merged integers are m = (U_round - z_bar) (W_round - z); with u_bits
 * <= 4 and 4-bit base codes |m| <= 225.  u_bits in [2, 4]; n even.  Workspace:
 * INTLORA_OP_MERGE_MUL.  Serving several adapters on one base stores one u_code per
 * adapter (half a byte per weight) next to the shared base codes. */
int intlora_merge_mul_codes(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int u_bits,
                            uint8_t* u_code, float* s_bar, int32_t* z_bar, void* ws, size_t ws_bytes, void* stream);

/* IntLoRA_SHIFT merge (section "two implementation variants", SHIFT).  U as for MUL.
 * Reading: s_bar = max(|U_min|, |U_max|), the largest |U| over the row's valid elements
 * (1 for an empty or all-zero row), with (U_min, U_max) the row's range or the caller's
 * u_min / u_max (both or neither, as for MUL); V = U / s_bar, so |V| <= 1 for every U in
 * the range and only right shifts occur;
 * shift = clamp(-round(log2 |V|), 0, 2^v_bits - 1), exact from the bits (no ties);
 * m = sign(V) * (w >> shift), ">>" arithmetic (floor); V == 0 gives m = 0 and the
 * largest shift code; m saturates to the signed w_bits range (counted); w == 0 gives
 * m = 0 and shift code 255.  The merged weight is s_bar_i * m_ij.
 * Outputs: m (int8 d x n for w_bits 8; packed signed nibbles d x n/2 for w_bits 4),
 * s_bar[d]; optional shift_dbg (uint8 d x n), sat_count.  v_bits in [1, 8].
 * Workspace: INTLORA_OP_MERGE_SHIFT. */
int intlora_merge_shift(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int v_bits,
                        const float* u_min, const float* u_max, void* m, float* s_bar, uint8_t* shift_dbg,
                        unsigned long long* sat_count, void* ws, size_t ws_bytes, void* stream);

/* QLoRA-style comparison path: the flow IntLoRA removes ([IntLoRA notes] research
 * background; its PTQ step is what "training and inference efficiency" says IntLoRA
 * avoids).  Per element, in binary32 and in this order:
 *   x = (s_i * (W_round - z_i) + R*_ij) + acc,  acc = the fma chain of A[i,k] B[k,j]
 *   over k from +0 (the same product as the MLA term);
 * then the base quantizer of "1. AQS" on each row of x at `bits` (4 or 8): lo =
 * min(0, min x), hi = max(0, max x), s' = (hi - lo)/(2^b - 1) (1 unless positive),
 * z' = clamp(rint(-lo / s')), code = clamp(rint(x / s') + z') (IEEE division).  Every
 * element takes part.  Outputs: code (uint8 d x n for 8 bits; packed nibbles d x n/2,
 * low nibble = even column, for 4 bits), s_out[d], z_out[d].  The requantized weight
 * is s'_i (code - z'_i).  Workspace: INTLORA_OP_MERGE_PTQ (x as fp32 scratch). */
int intlora_merge_ptq(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int bits,
                      void* code, float* s_out, int32_t* z_out, void* ws, size_t ws_bytes, void* stream);

/* Straight-through backward of the MUL / SHIFT fake-quant merge to the LoRA factors
 * ([IntLoRA notes] "two implementation variants": training back-propagates through the
 * quantizers with the STE; "1. AQS": R takes no gradient).  Reading: the roundings
 * pass gradients unchanged and s_bar, z_bar are constants, so the merged weight acts as
 * U (.) w = s w + R* + AB where w = W_round - z != 0 and as the constant 0 where w = 0.
 * With G = dL/dW' (fp32 d x n) and D = G (.) [w != 0]:
 *   dA = D B^T (fp32 d x r),  dB = A^T D (fp32 r x n),
 * accumulated in binary32 on the matrix cores in an order fixed by (d, n, r) alone
 * (deterministic; each output within the binary32 summation bound of its exact value).
 * w_round: the base codes (uint8 d x n, or packed d x n/2 for w_bits 4), z[d]; A d x r,
 * B r x n (as for the merge).  r <= 128.  Workspace: INTLORA_OP_STE_BACKWARD (partial
 * sums; 0 bytes for small shapes). */
int intlora_ste_backward(const intlora_desc* desc, const void* w_round, const int32_t* z, const float* A,
                         const float* B, const float* G, float* dA, float* dB, void* ws, size_t ws_bytes,
                         void* stream);

/* Per-token symmetric int8 activation quantization, the activation side of the W8A8 /
 * W4A8 layer: the IntLoRA notes ("training and inference efficiency") keep the
 * activations' quantization conventional, and the SVDQuant article ("5 Experiments",
 * "Setups", 8-bit implementation details) takes per-token dynamic activation scales.
 *   s_x[t] = max_j |X[t,j]| / 127 (1 for an all-zero token),
 *   xq = clamp(rint(X / s_x), -127, 127) (rint half to even, IEEE division),
 *   x_rowsum[t] = sum_j xq[t,j] (x_rowsum may be NULL).
 * X: M x n fp32 row-major; xq: M x n int8; s_x: [M] fp32; x_rowsum: [M] int32; all
 * caller-owned device memory.  M = 0 is a no-op; INTLORA_ESHAPE for M < 0 or n < 1. */
int intlora_quant_act(int64_t M, int64_t n, const float* X, int8_t* xq, float* s_x, int32_t* x_rowsum,
                      void* stream);

/* Integer linear layer on merged integers ([IntLoRA notes] "training and inference
 * efficiency": the merged integers are the deployed W8A8 / W4A8 weights, used with no
 * post-training quantization; "two implementation variants": the merged weight is
 * s_bar_i m_ij; per-token activation and per-channel weight scales as in the SVDQuant
 * article's 8-bit setting):  Y[t, i] for t < M tokens, i < d outputs.
 *   exact = sum_j xq[t,j] * m[i,j] (integer);
 *   y = RN32(RN32(float(exact) * s_x[t]) * s_bar[i]),  Y = bf16 round-to-nearest-even.
 * wfmt INTLORA_W_INT8 / INTLORA_W_INT4 (SHIFT merged integers): one int8 MFMA pass.
 * wfmt INTLORA_W_INT16 (MUL merged integers): two int8 MFMA passes over a byte split
 * of m (x_rowsum required), one split for the whole call (for M <= 32: for each block
 * of 16 consecutive rows), chosen from the split codes m_split[i] (uint8 per row, 0 or
 * 1; NULL = all 1):
 *   some row coded 1 (any int16): bias split hi = m >> 8, lo = (m & 0xFF) - 128,
 *      exact = 256 acc_hi + acc_lo + 128 x_rowsum[t];
 *   every row coded 0 (the caller guarantees each m[i, j] <= 32639, as the codes
 *      written by intlora_merge_mul do): balanced split hi = (m + 128) >> 8,
 *      lo = m - 256 hi, exact = 256 acc_hi + acc_lo;
 * combined exactly (int64-exact binary64).  Both give the same Y; the balanced split
 * leaves the high plane zero for |m| < 128, which the matrix cores run at lower power.
 * Codes of 0 on a matrix holding m >= 32640 give unspecified outputs.
 * m_split must be NULL for the other formats (INTLORA_EINVAL).
 * xq: M x n int8; m: d x n (layout per wfmt); Y_bf16: M x d (bf16 bits, row-major);
 * acc_dbg (optional): planes x M x d int32 raw accumulators (planes = 2 for INT16:
 * hi then lo of the split applied; 1 otherwise).  n must be a multiple of 32 and <= 131071 (no int32
 * overflow).  No workspace. */
int intlora_linear_fwd(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* s_x, const int32_t* x_rowsum,
                       int wfmt, const void* m, const uint8_t* m_split, const float* s_bar, uint16_t* Y_bf16,
                       int32_t* acc_dbg, void* ws, size_t ws_bytes, void* stream);

/* Merge-on-load integer linear layer (MUL with U's codes kept, see
 * intlora_merge_mul_codes; [IntLoRA notes] "两种实现版本", MUL, and "training and
 * inference efficiency"): Y is exactly intlora_linear_fwd's INT16 output for the merged
 * integers m = (U_round - z_bar) (W_round - z), formed per tile after the weights' LDS
 * read and never stored.  u_code, w_round: packed nibbles d x n/2 (low nibble = even
 * column; U's codes of u_bits <= 4, 4-bit base codes); z[d], z_bar[d]: their zero
 * points; s_bar[d].  With these widths |m| <= 225, so the balanced byte split applies
 * (exact = 256 acc_hi + acc_lo) and no row sums are needed.  xq: M x n int8; Y_bf16: M x
 * d; acc_dbg (optional): 2 x M x d int32 (hi then lo plane).  n a multiple of 32 and <=
 * 131071.  No workspace. */
int intlora_linear_fwd_codes(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* s_x,
                             const uint8_t* u_code, const uint8_t* w_round, const int32_t* z, const int32_t* z_bar,
                             const float* s_bar, uint16_t* Y_bf16, int32_t* acc_dbg, void* stream);

/* Diagnostic: the binary32 natural log used by intlora_gen_r, on g = G * 2^-23 for
 * odd G in [1, 2^23) (the only values it is ever given): out[t] = RN32(ln(G[t] 2^-23)).
 * Inputs outside that set give unspecified values. */
int intlora_debug_ln(int64_t count, const uint32_t* G, float* out, void* stream);

/* Diagnostic: the unscaled auxiliary sample (c = 1) of each element of `blocks` given
 * Philox output blocks words[4 t .. 4 t + 3] under law aux_dist: out[4 t + e] is what
 * intlora_gen_r computes for element e of a block with those words.  words (4 * blocks
 * uint32) and out (4 * blocks fp32) are caller-owned device buffers.  INTLORA_EINVAL for
 * an unknown law, INTLORA_ESHAPE for blocks < 0; blocks = 0 returns INTLORA_OK. */
int intlora_debug_aux(int64_t blocks, const uint32_t* words, uint32_t aux_dist, float* out, void* stream);

/* Diagnostic: the rank-r product acc = A B (A: d x r, B: r x n, fp32 row-major; acc:
 * d x n) formed on the matrix cores exactly as the merges form the MLA term's AB
 * ([IntLoRA notes] "2. MLA": an fma chain over k from +0, one rounding per k), one
 * matrix-core instruction per k in increasing k: form 0 is v_mfma_f32_32x32x1f32 taken
 * transposed (the adaptation kernel), form 1 v_mfma_f32_4x4x1f32 (the fused merge).
 * d must be a multiple of 32 (form 0) or 4 (form 1), n of 64; r in [1, 128].  Tests
 * pin it against a plain fmaf chain.  INTLORA_EINVAL / INTLORA_ESHAPE otherwise. */
int intlora_debug_mfma_chain(int form, int64_t d, int64_t n, int r, const float* A, const float* B, float* acc,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INTLORA_H */
