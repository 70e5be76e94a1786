// C ABI of libintlora.so (declared in include/intlora.h): host-side validation,
// workspace layout and kernel dispatch.  No allocation, no state across calls.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/intlora.h"
#include "intlora_internal.h"

// Scratch memory of intlora_merge_mul_noalloc: U and the row partials of one row chunk.
// One copy per device, held until the process ends.  Host code never passes the
// array's name to a kernel: it passes the device address taken once per device with
// hipGetSymbolAddress (scratch_on_device below).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "";

__attribute__((format(printf, 2, 3))) int fail(int status, const char* fmt, ...);
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return INTLORA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(INTLORA_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Largest dynamic LDS any kernel asks for; set once per device before first use.
int ensure_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(INTLORA_EDEVICE, "no HIP device");
  static thread_local int configured_dev = -1;
  if (configured_dev == dev) return INTLORA_OK;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(INTLORA_EDEVICE, "hipGetDeviceProperties failed");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(INTLORA_EDEVICE, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
  configured_dev = dev;
  return INTLORA_OK;
}

constexpr int64_t kMaxDim = int64_t(1) << 31;

int check_desc(const intlora_desc* d, bool need_rank) {
  if (!d) return fail(INTLORA_EINVAL, "desc is NULL");
  if (d->w_bits != 4 && d->w_bits != 8) return fail(INTLORA_EINVAL, "w_bits must be 4 or 8 (got %d)", d->w_bits);
  if (need_rank && (d->r < 1 || d->r > 128)) return fail(INTLORA_EINVAL, "rank r must be in [1, 128] (got %d)", d->r);
  if (d->aux_dist > INTLORA_AUX_STUDENT_T2)
    return fail(INTLORA_EINVAL, "desc.aux_dist must be 0..3 (got %u)", d->aux_dist);
  if (d->d < 0 || d->n < 1 || d->d >= kMaxDim || d->n >= kMaxDim)
    return fail(INTLORA_ESHAPE, "bad shape d=%lld n=%lld", (long long)d->d, (long long)d->n);
  if (d->w_bits == 4 && (d->n & 1)) return fail(INTLORA_ESHAPE, "4-bit codes need an even n (got %lld)", (long long)d->n);
  if ((unsigned long long)d->d * (unsigned long long)d->n >= (1ull << 40))
    return fail(INTLORA_ESHAPE, "d*n too large");
  return INTLORA_OK;
}

int check_ptrs(std::initializer_list<const void*> ps, const char* what) {
  for (const void* p : ps) {
    if (!p) return fail(INTLORA_EINVAL, "%s: NULL pointer", what);
    if (!aligned16(p)) return fail(INTLORA_EALIGN, "%s: pointer %p not 16-byte aligned", what, p);
  }
  return INTLORA_OK;
}

int check_opt(const void* p, const char* what) {
  if (p && !aligned16(p)) return fail(INTLORA_EALIGN, "%s: pointer %p not 16-byte aligned", what, p);
  return INTLORA_OK;
}

// Workspace layout of the merge / U statistics: U (d*n fp32) | pmin | pmax (d*ntiles
// order keys each) | umin | umax | rs | small (d 4-byte values each: the row range, and
// the MUL quantizer's RN(1/s_bar) and small-row flag)
struct MergeWs {
  float* U;
  int* pmin;
  int* pmax;
  float* umin;
  float* umax;
  float* rs;
  int* small;
  int ntiles;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t merge_ws_bytes(int64_t d, int64_t n) {
  const size_t nt = (size_t)intlora::adapt_max_ntiles(n);
  return align256((size_t)d * (size_t)n * 4) + 2 * align256((size_t)d * nt * 4) + 4 * align256((size_t)d * 4);
}

MergeWs carve(void* ws, int64_t d, int64_t n) {
  MergeWs w;
  w.ntiles = intlora::adapt_max_ntiles(n);
  uint8_t* p = static_cast<uint8_t*>(ws);
  w.U = reinterpret_cast<float*>(p);
  p += align256((size_t)d * (size_t)n * 4);
  w.pmin = reinterpret_cast<int*>(p);
  p += align256((size_t)d * (size_t)w.ntiles * 4);  // capacity; the kernels use <= ntiles per row
  w.pmax = reinterpret_cast<int*>(p);
  p += align256((size_t)d * (size_t)w.ntiles * 4);
  w.umin = reinterpret_cast<float*>(p);
  p += align256((size_t)d * 4);
  w.umax = reinterpret_cast<float*>(p);
  p += align256((size_t)d * 4);
  w.rs = reinterpret_cast<float*>(p);
  p += align256((size_t)d * 4);
  w.small = reinterpret_cast<int*>(p);
  return w;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return INTLORA_OK;
  if (!ws) return fail(INTLORA_EWORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned16(ws)) return fail(INTLORA_EALIGN, "workspace not 16-byte aligned");
  if (ws_bytes < need) return fail(INTLORA_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return INTLORA_OK;
}

int run_adapt(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, MergeWs& w,
              unsigned long long* sat_zero, hipStream_t st, bool ptq = false, int64_t row0 = 0) {
  intlora::AdaptArgs a;
  a.d = desc->d;
  a.n = desc->n;
  a.r = desc->r;
  a.w_bits = desc->w_bits;
  a.seed = desc->seed;
  a.layer_id = desc->layer_id;
  a.wround = static_cast<const uint8_t*>(base->w_round);
  a.z = base->z;
  a.s = base->s;
  a.c = base->vmc_c;
  a.A = lora->A;
  a.B = lora->B;
  a.U = w.U;
  a.pmin = w.pmin;
  a.pmax = w.pmax;
  a.sat_zero = sat_zero;
  a.ptq = ptq;
  a.force_generic = false;
  a.dist = (int)desc->aux_dist;
  a.row0 = row0;
  return launch_status(intlora::launch_adapt(a, &w.ntiles, st), "adaptation kernel");
}

int check_base_lora(const intlora_base* base, const intlora_lora* lora) {
  if (!base || !lora) return fail(INTLORA_EINVAL, "base / lora struct is NULL");
  int s = check_ptrs({base->w_round, base->z, base->s, base->vmc_c}, "base");
  if (s) return s;
  return check_ptrs({lora->A, lora->B}, "lora");
}

// The optional caller-supplied row range: both NULL (computed here) or both given.
int check_range(const float* u_min, const float* u_max) {
  if ((u_min == nullptr) != (u_max == nullptr)) return fail(INTLORA_EINVAL, "u_min and u_max: give both or neither");
  if (u_min) return check_ptrs({u_min, u_max}, "u_min / u_max");
  return INTLORA_OK;
}

// Row range of the SHIFT merge: the caller's (u_min, u_max), or the reduction of the
// adaptation kernel's tile partials into the workspace.
int merge_range(int64_t d, const MergeWs& w, const float* u_min, const float* u_max, const float** lo,
                const float** hi, hipStream_t st) {
  if (u_min) {
    *lo = u_min;
    *hi = u_max;
    return INTLORA_OK;
  }
  *lo = w.umin;
  *hi = w.umax;
  return launch_status(intlora::launch_row_range(d, w.ntiles, w.pmin, w.pmax, w.umin, w.umax, nullptr, st),
                       "row range");
}

// The three-kernel MUL merge of rows [0, desc->d) of the pointers given, whose row 0 is
// row `row0` of the layer (R's counter); `sat_zero` is the counter the adaptation
// kernel clears first (NULL: not cleared here).  Arguments are validated by the caller.
// planes: m is the byte-plane layout (d x 2n bytes) and m_split the plane codes.
int merge_mul_rows(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int u_bits,
                   const float* u_min, const float* u_max, void* m, float* s_bar, int32_t* z_bar,
                   uint8_t* m_split, uint8_t* u_round_dbg, unsigned long long* sat_count,
                   unsigned long long* sat_zero, MergeWs& w, int64_t row0, hipStream_t st, bool planes = false) {
  int s = run_adapt(desc, base, lora, w, sat_zero, st, false, row0);
  if (s) return s;
  if ((s = launch_status(intlora::launch_mul_params(desc->d, w.ntiles, w.pmin, w.pmax, u_min, u_max, w.umin, w.umax,
                                                    u_bits, desc->w_bits, base->z, s_bar, z_bar, w.rs, w.small,
                                                    m_split, planes, st),
                         "MUL row parameters")))
    return s;
  return launch_status(intlora::launch_quant_mul(desc->d, desc->n, desc->w_bits, u_bits,
                                                 static_cast<const uint8_t*>(base->w_round), base->z, w.U, s_bar,
                                                 z_bar, w.rs, w.small, m, m_split, u_round_dbg, sat_count, nullptr,
                                                 planes, st),
                       "quant_mul");
}

int check_merge_mul(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int u_bits,
                    const float* u_min, const float* u_max, int16_t* m, float* s_bar, int32_t* z_bar,
                    uint8_t* m_split, uint8_t* u_round_dbg, unsigned long long* sat_count, const char* what) {
  int s = check_desc(desc, true);
  if (s) return s;
  if (u_bits < 2 || u_bits > 8) return fail(INTLORA_EINVAL, "u_bits must be in [2, 8] (got %d)", u_bits);
  if (desc->d == 0) return INTLORA_OK;
  if ((s = check_base_lora(base, lora))) return s;
  if ((s = check_range(u_min, u_max))) return s;
  if ((s = check_ptrs({m, s_bar, z_bar}, what))) return s;
  if ((s = check_opt(m_split, "m_split")) || (s = check_opt(u_round_dbg, "u_round_dbg")) ||
      (s = check_opt(sat_count, "sat_count")))
    return s;
  return INTLORA_OK;
}

// Device address of `scratch` on the current device, looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(INTLORA_EDEVICE, "no HIP device");
  if (dev >= kMaxDevices) return fail(INTLORA_EDEVICE, "device %d: at most %d devices are supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(INTLORA_EDEVICE, "device %d: scratch address: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return INTLORA_OK;
}

// Rows per chunk of the allocation-free merge: the most rows whose workspace fits the
// scratch, a multiple of 32 (one adaptation row tile; it also keeps every row offset of
// the chunked pointers 16-byte aligned) unless the whole layer fits.  0 if not even 32
// rows fit.
int64_t noalloc_rows(int64_t d, int64_t n) {
  if (merge_ws_bytes(d, n) <= kScratchBytes) return d;
  const size_t per_row = (size_t)n * 4 + 8 * (size_t)intlora::adapt_max_ntiles(n) + 16;
  int64_t rows = (int64_t)((kScratchBytes - 7 * 256) / per_row) & ~int64_t(31);
  while (rows > 0 && merge_ws_bytes(rows, n) > kScratchBytes) rows -= 32;
  return rows;
}

}  // namespace

extern "C" {

const char* intlora_status_string(int status) {
  switch (status) {
    case INTLORA_OK: return "ok";
    case INTLORA_EINVAL: return "invalid argument";
    case INTLORA_ESHAPE: return "unsupported shape";
    case INTLORA_EALIGN: return "misaligned pointer";
    case INTLORA_EWORKSPACE: return "workspace too small";
    case INTLORA_EDEVICE: return "no usable device";
    case INTLORA_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* intlora_last_error(void) { return g_err; }

int intlora_version(void) { return 104; }

size_t intlora_workspace_bytes(int op, const intlora_desc* desc, int64_t M) {
  (void)M;
  if (!desc || desc->d < 0 || desc->n < 1) return 0;
  switch (op) {
    case INTLORA_OP_STATS_UMINMAX:
    case INTLORA_OP_MERGE_MUL:
    case INTLORA_OP_MERGE_SHIFT:
    case INTLORA_OP_MERGE_PTQ:
      return merge_ws_bytes(desc->d, desc->n);
    case INTLORA_OP_STE_BACKWARD:
      return intlora::ste_ws_bytes(desc->d, desc->n, desc->r);
    default:
      return 0;
  }
}

int intlora_gen_r(const intlora_desc* desc, const float* vmc_c, float* r_out, void* stream) {
  int s = check_desc(desc, false);
  if (s) return s;
  if (desc->d == 0) return ok();
  if ((s = check_ptrs({vmc_c, r_out}, "gen_r"))) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_gen_r(desc->d, desc->n, desc->seed, desc->layer_id, vmc_c, r_out,
                                             (int)desc->aux_dist, static_cast<hipStream_t>(stream)),
                       "gen_r");
}

int intlora_stats(const intlora_desc* desc, int mode, const float* W, const intlora_base* base,
                  const intlora_lora* lora, float* out0, float* out1, void* ws, size_t ws_bytes, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == INTLORA_SIGMA_W) {
    if (!desc) return fail(INTLORA_EINVAL, "desc is NULL");
    if (desc->d < 0 || desc->n < 1 || desc->d >= kMaxDim || desc->n >= kMaxDim)
      return fail(INTLORA_ESHAPE, "bad shape");
    if (desc->d == 0) return ok();
    int s = check_ptrs({W, out0}, "stats(sigma_w)");
    if (s) return s;
    if ((s = ensure_device())) return s;
    return launch_status(intlora::launch_sigma_w(desc->d, desc->n, W, out0, st), "sigma_w");
  }
  if (mode != INTLORA_U_MINMAX) return fail(INTLORA_EINVAL, "unknown stats mode %d", mode);
  int s = check_desc(desc, true);
  if (s) return s;
  if (desc->d == 0) return ok();
  if ((s = check_base_lora(base, lora))) return s;
  if ((s = check_ptrs({out0, out1}, "stats(u_minmax)"))) return s;
  if ((s = check_ws(ws, ws_bytes, merge_ws_bytes(desc->d, desc->n)))) return s;
  if ((s = ensure_device())) return s;
  MergeWs w = carve(ws, desc->d, desc->n);
  if ((s = run_adapt(desc, base, lora, w, nullptr, st))) return s;
  return launch_status(intlora::launch_row_range(desc->d, w.ntiles, w.pmin, w.pmax, out0, out1, nullptr, st),
                       "row range");
}

int intlora_vmc_scale(int64_t d, const float* sigma_w, double alpha, float* c_out, void* stream) {
  if (d < 0) return fail(INTLORA_ESHAPE, "d < 0");
  if (!(alpha >= 0.0 && alpha <= 8.0)) return fail(INTLORA_EINVAL, "alpha must be in [0, 8]");
  if (d == 0) return ok();
  int s = check_ptrs({sigma_w, c_out}, "vmc_scale");
  if (s) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_vmc_scale(d, sigma_w, alpha, c_out, INTLORA_AUX_LAPLACE,
                                                 static_cast<hipStream_t>(stream)),
                       "vmc_scale");
}

int intlora_vmc_scale_dist(int64_t d, const float* sigma_w, double alpha, uint32_t aux_dist, float* c_out,
                           void* stream) {
  if (d < 0) return fail(INTLORA_ESHAPE, "d < 0");
  if (!(alpha >= 0.0 && alpha <= 8.0)) return fail(INTLORA_EINVAL, "alpha must be in [0, 8]");
  if (aux_dist > INTLORA_AUX_STUDENT_T2) return fail(INTLORA_EINVAL, "aux_dist must be 0..3 (got %u)", aux_dist);
  if (d == 0) return ok();
  int s = check_ptrs({sigma_w, c_out}, "vmc_scale_dist");
  if (s) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_vmc_scale(d, sigma_w, alpha, c_out, (int)aux_dist,
                                                 static_cast<hipStream_t>(stream)),
                       "vmc_scale_dist");
}

int intlora_base_quant(const intlora_desc* desc, const float* W, const float* vmc_c, void* w_round_out,
                       int32_t* z_out, float* s_out, void* stream) {
  int s = check_desc(desc, false);
  if (s) return s;
  if (desc->n > 32768) return fail(INTLORA_ESHAPE, "base_quant supports n <= 32768 (got %lld)", (long long)desc->n);
  if (desc->d == 0) return ok();
  if ((s = check_ptrs({W, vmc_c, w_round_out, z_out, s_out}, "base_quant"))) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_base_quant(desc->d, desc->n, desc->w_bits, desc->seed, desc->layer_id, W, vmc_c,
                                                  static_cast<uint8_t*>(w_round_out), z_out, s_out, (int)desc->aux_dist,
                                                  static_cast<hipStream_t>(stream)),
                       "base_quant");
}


int intlora_merge_mul(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int u_bits,
                      const float* u_min, const float* u_max, int16_t* m, float* s_bar, int32_t* z_bar,
                      uint8_t* m_split, uint8_t* u_round_dbg, unsigned long long* sat_count, void* ws,
                      size_t ws_bytes, void* stream) {
  int s = check_merge_mul(desc, base, lora, u_bits, u_min, u_max, m, s_bar, z_bar, m_split, u_round_dbg, sat_count,
                          "merge_mul");
  if (s) return s;
  if (desc->d == 0) return ok();
  if ((s = check_ws(ws, ws_bytes, merge_ws_bytes(desc->d, desc->n)))) return s;
  if ((s = ensure_device())) return s;
  MergeWs w = carve(ws, desc->d, desc->n);
  if ((s = merge_mul_rows(desc, base, lora, u_bits, u_min, u_max, m, s_bar, z_bar, m_split, u_round_dbg, sat_count,
                          sat_count, w, 0, static_cast<hipStream_t>(stream))))
    return s;
  return ok();
}

int intlora_merge_mul_planes(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora,
                             int u_bits, const float* u_min, const float* u_max, uint8_t* m_planes, float* s_bar,
                             int32_t* z_bar, uint8_t* plane_code, uint8_t* u_round_dbg,
                             unsigned long long* sat_count, void* ws, size_t ws_bytes, void* stream) {
  int s = check_merge_mul(desc, base, lora, u_bits, u_min, u_max, reinterpret_cast<int16_t*>(m_planes), s_bar, z_bar,
                          plane_code, u_round_dbg, sat_count, "merge_mul_planes");
  if (s) return s;
  if (desc->n % 16 != 0)
    return fail(INTLORA_ESHAPE, "merge_mul_planes: n must be a multiple of 16 (got %lld)", (long long)desc->n);
  if (desc->d == 0) return ok();
  if ((s = check_ptrs({plane_code}, "merge_mul_planes plane_code"))) return s;
  if ((s = check_ws(ws, ws_bytes, merge_ws_bytes(desc->d, desc->n)))) return s;
  if ((s = ensure_device())) return s;
  MergeWs w = carve(ws, desc->d, desc->n);
  if ((s = merge_mul_rows(desc, base, lora, u_bits, u_min, u_max, m_planes, s_bar, z_bar, plane_code, u_round_dbg,
                          sat_count, sat_count, w, 0, static_cast<hipStream_t>(stream), true)))
    return s;
  return ok();
}

int intlora_merge_mul_noalloc(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora,
                              int u_bits, const float* u_min, const float* u_max, int16_t* m, float* s_bar,
                              int32_t* z_bar, uint8_t* m_split, uint8_t* u_round_dbg, unsigned long long* sat_count,
                              void* stream) {
  int s = check_merge_mul(desc, base, lora, u_bits, u_min, u_max, m, s_bar, z_bar, m_split, u_round_dbg, sat_count,
                          "merge_mul_noalloc");
  if (s) return s;
  if (desc->d == 0) return ok();
  const int64_t d = desc->d, n = desc->n;
  const int64_t rows = noalloc_rows(d, n);
  if (rows <= 0)
    return fail(INTLORA_ESHAPE,
                "merge_mul_noalloc: 32 rows of n = %lld need %zu bytes of scratch; the library holds %zu per device",
                (long long)n, merge_ws_bytes(32, n), kScratchBytes);
  if ((s = ensure_device())) return s;
  void* sp = nullptr;
  if ((s = scratch_on_device(&sp))) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t code_row = desc->w_bits == 4 ? n / 2 : n;  // bytes per row of base codes
  for (int64_t r0 = 0; r0 < d; r0 += rows) {
    const int64_t dc = d - r0 < rows ? d - r0 : rows;
    intlora_desc dk = *desc;
    dk.d = dc;
    intlora_base bk = *base;
    bk.w_round = static_cast<const uint8_t*>(base->w_round) + r0 * code_row;
    bk.z = base->z + r0;
    bk.s = base->s + r0;
    bk.vmc_c = base->vmc_c + r0;
    intlora_lora lk = *lora;
    lk.A = lora->A + r0 * desc->r;
    MergeWs w = carve(sp, dc, n);
    // the first chunk's adaptation kernel clears the saturation counter; later chunks add
    s = merge_mul_rows(&dk, &bk, &lk, u_bits, u_min ? u_min + r0 : nullptr, u_max ? u_max + r0 : nullptr,
                       m + r0 * n, s_bar + r0, z_bar + r0, m_split ? m_split + r0 : nullptr,
                       u_round_dbg ? u_round_dbg + r0 * n : nullptr, sat_count, r0 == 0 ? sat_count : nullptr, w, r0,
                       st);
    if (s) return s;
  }
  return ok();
}

int intlora_merge_mul_fused(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int u_bits,
                            int16_t* m, float* s_bar, int32_t* z_bar, uint8_t* m_split, uint8_t* u_round_dbg,
                            unsigned long long* sat_count, void* stream) {
  int s = check_desc(desc, true);
  if (s) return s;
  if (u_bits < 2 || u_bits > 8) return fail(INTLORA_EINVAL, "u_bits must be in [2, 8] (got %d)", u_bits);
  if (desc->n > 16384)
    return fail(INTLORA_ESHAPE, "merge_mul_fused keeps whole rows on chip: n <= 16384 (got %lld)",
                (long long)desc->n);
  if (desc->d == 0) return ok();
  if ((s = check_base_lora(base, lora))) return s;
  if ((s = check_ptrs({m, s_bar, z_bar}, "merge_mul_fused"))) return s;
  if ((s = check_opt(m_split, "m_split")) || (s = check_opt(u_round_dbg, "u_round_dbg")) ||
      (s = check_opt(sat_count, "sat_count")))
    return s;
  if ((s = ensure_device())) return s;
  intlora::AdaptArgs a;
  a.d = desc->d;
  a.n = desc->n;
  a.r = desc->r;
  a.w_bits = desc->w_bits;
  a.seed = desc->seed;
  a.layer_id = desc->layer_id;
  a.wround = static_cast<const uint8_t*>(base->w_round);
  a.z = base->z;
  a.s = base->s;
  a.c = base->vmc_c;
  a.A = lora->A;
  a.B = lora->B;
  a.U = nullptr;
  a.pmin = a.pmax = nullptr;
  a.sat_zero = nullptr;
  a.ptq = false;
  a.force_generic = false;
  a.dist = (int)desc->aux_dist;
  return launch_status(intlora::launch_merge_fused(a, u_bits, m, s_bar, z_bar, m_split, u_round_dbg, sat_count,
                                                   static_cast<hipStream_t>(stream)),
                       "merge_mul_fused");
}

int intlora_merge_mul_codes(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int u_bits,
                            uint8_t* u_code, float* s_bar, int32_t* z_bar, void* ws, size_t ws_bytes, void* stream) {
  int s = check_desc(desc, true);
  if (s) return s;
  if (u_bits < 2 || u_bits > 4) return fail(INTLORA_EINVAL, "merge_mul_codes: u_bits must be in [2, 4] (got %d)", u_bits);
  if (desc->n & 1) return fail(INTLORA_ESHAPE, "merge_mul_codes: packed 4-bit codes need an even n");
  if (desc->d == 0) return ok();
  if ((s = check_base_lora(base, lora))) return s;
  if ((s = check_ptrs({u_code, s_bar, z_bar}, "merge_mul_codes"))) return s;
  if ((s = check_ws(ws, ws_bytes, merge_ws_bytes(desc->d, desc->n)))) return s;
  if ((s = ensure_device())) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MergeWs w = carve(ws, desc->d, desc->n);
  if ((s = run_adapt(desc, base, lora, w, nullptr, st))) return s;
  if ((s = launch_status(intlora::launch_mul_params(desc->d, w.ntiles, w.pmin, w.pmax, nullptr, nullptr, w.umin,
                                                    w.umax, u_bits, desc->w_bits, base->z, s_bar, z_bar, w.rs,
                                                    w.small, nullptr, false, st),
                         "MUL row parameters")))
    return s;
  return launch_status(intlora::launch_quant_mul(desc->d, desc->n, desc->w_bits, u_bits,
                                                 static_cast<const uint8_t*>(base->w_round), base->z, w.U, s_bar,
                                                 z_bar, w.rs, w.small, nullptr, nullptr, nullptr, nullptr, u_code,
                                                 false, st),
                       "quant_mul codes");
}

int intlora_merge_shift(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int v_bits,
                        const float* u_min, const float* u_max, void* m, float* s_bar, uint8_t* shift_dbg,
                        unsigned long long* sat_count, void* ws, size_t ws_bytes, void* stream) {
  int s = check_desc(desc, true);
  if (s) return s;
  if (v_bits < 1 || v_bits > 8) return fail(INTLORA_EINVAL, "v_bits must be in [1, 8] (got %d)", v_bits);
  if (desc->d == 0) return ok();
  if ((s = check_base_lora(base, lora))) return s;
  if ((s = check_range(u_min, u_max))) return s;
  if ((s = check_ptrs({m, s_bar}, "merge_shift"))) return s;
  if ((s = check_opt(shift_dbg, "shift_dbg")) || (s = check_opt(sat_count, "sat_count"))) return s;
  if ((s = check_ws(ws, ws_bytes, merge_ws_bytes(desc->d, desc->n)))) return s;
  if ((s = ensure_device())) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MergeWs w = carve(ws, desc->d, desc->n);
  if ((s = run_adapt(desc, base, lora, w, sat_count, st))) return s;
  const float *lo, *hi;
  if ((s = merge_range(desc->d, w, u_min, u_max, &lo, &hi, st))) return s;
  return launch_status(intlora::launch_quant_shift(desc->d, desc->n, desc->w_bits, v_bits,
                                                   static_cast<const uint8_t*>(base->w_round), base->z, w.U, lo, hi,
                                                   static_cast<uint8_t*>(m), s_bar, shift_dbg, sat_count, st),
                       "quant_shift");
}

int intlora_merge_ptq(const intlora_desc* desc, const intlora_base* base, const intlora_lora* lora, int bits,
                      void* code, float* s_out, int32_t* z_out, void* ws, size_t ws_bytes, void* stream) {
  int s = check_desc(desc, true);
  if (s) return s;
  if (bits != 4 && bits != 8) return fail(INTLORA_EINVAL, "bits must be 4 or 8 (got %d)", bits);
  if (bits == 4 && (desc->n & 1)) return fail(INTLORA_ESHAPE, "4-bit codes need even n");
  if (desc->d == 0) return ok();
  if ((s = check_base_lora(base, lora))) return s;
  if ((s = check_ptrs({code, s_out, z_out}, "merge_ptq"))) return s;
  if ((s = check_ws(ws, ws_bytes, merge_ws_bytes(desc->d, desc->n)))) return s;
  if ((s = ensure_device())) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MergeWs w = carve(ws, desc->d, desc->n);
  if ((s = run_adapt(desc, base, lora, w, nullptr, st, true))) return s;
  if ((s = launch_status(intlora::launch_row_range(desc->d, w.ntiles, w.pmin, w.pmax, w.umin, w.umax, nullptr, st),
                         "row range")))
    return s;
  return launch_status(intlora::launch_quant_ptq(desc->d, desc->n, bits, w.U, w.umin, w.umax,
                                                 static_cast<uint8_t*>(code), s_out, z_out, st),
                       "quant_ptq");
}

int intlora_ste_backward(const intlora_desc* desc, const void* w_round, const int32_t* z, const float* A,
                         const float* B, const float* G, float* dA, float* dB, void* ws, size_t ws_bytes,
                         void* stream) {
  int s = check_desc(desc, true);
  if (s) return s;
  if (desc->d == 0) return ok();
  if ((s = check_ptrs({w_round, z, A, B, G, dA, dB}, "ste_backward"))) return s;
  if ((s = check_ws(ws, ws_bytes, intlora::ste_ws_bytes(desc->d, desc->n, desc->r)))) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_ste_backward(desc->d, desc->n, desc->r, desc->w_bits,
                                                    static_cast<const uint8_t*>(w_round), z, A, B, G, dA, dB, ws,
                                                    static_cast<hipStream_t>(stream)),
                       "ste_backward");
}

int intlora_quant_act(int64_t M, int64_t n, const float* X, int8_t* xq, float* s_x, int32_t* x_rowsum,
                      void* stream) {
  if (M < 0 || n < 1 || M >= kMaxDim || n >= kMaxDim) return fail(INTLORA_ESHAPE, "bad shape M=%lld n=%lld",
                                                                 (long long)M, (long long)n);
  if (M == 0) return ok();
  int s = check_ptrs({X, xq, s_x}, "quant_act");
  if (s) return s;
  if ((s = check_opt(x_rowsum, "x_rowsum"))) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_quant_act(M, n, X, xq, s_x, x_rowsum, static_cast<hipStream_t>(stream)),
                       "quant_act");
}

int intlora_linear_fwd(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* s_x, const int32_t* x_rowsum,
                       int wfmt, const void* m, const uint8_t* m_split, const float* s_bar, uint16_t* Y_bf16,
                       int32_t* acc_dbg, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (wfmt != INTLORA_W_INT4 && wfmt != INTLORA_W_INT8 && wfmt != INTLORA_W_INT16 && wfmt != INTLORA_W_INT16_PLANES)
    return fail(INTLORA_EINVAL, "wfmt must be INTLORA_W_INT4, _INT8, _INT16 or _INT16_PLANES (got %d)", wfmt);
  if (M < 0 || d < 0 || n < 1 || M >= kMaxDim || d >= kMaxDim) return fail(INTLORA_ESHAPE, "bad shape");
  if (n % 32 != 0 || n > 131071)
    return fail(INTLORA_ESHAPE, "linear needs n a multiple of 32 and <= 131071 (got %lld)", (long long)n);
  if ((int64_t)((M + 255) / 256) * (int64_t)((d + 127) / 128) >= (int64_t(1) << 31))
    return fail(INTLORA_ESHAPE, "too many tiles");
  if (M == 0 || d == 0) return ok();
  int s = check_ptrs({xq, s_x, m, s_bar, Y_bf16}, "linear_fwd");
  if (s) return s;
  if ((wfmt == INTLORA_W_INT16 || wfmt == INTLORA_W_INT16_PLANES) &&
      (s = check_ptrs({x_rowsum}, "linear_fwd x_rowsum (INT16)")))
    return s;
  if (wfmt == INTLORA_W_INT16_PLANES && (s = check_ptrs({m_split}, "linear_fwd plane codes (INT16_PLANES)"))) return s;
  if ((s = check_opt(acc_dbg, "acc_dbg")) || (s = check_opt(m_split, "m_split"))) return s;
  if (m_split && wfmt != INTLORA_W_INT16 && wfmt != INTLORA_W_INT16_PLANES)
    return fail(INTLORA_EINVAL, "m_split applies to INTLORA_W_INT16 and _INT16_PLANES only");
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_linear(M, d, n, xq, s_x, x_rowsum, wfmt, m, m_split, s_bar, Y_bf16, acc_dbg,
                                              static_cast<hipStream_t>(stream)),
                       "linear");
}

int intlora_linear_fwd_codes(int64_t M, int64_t d, int64_t n, const int8_t* xq, const float* s_x,
                             const uint8_t* u_code, const uint8_t* w_round, const int32_t* z, const int32_t* z_bar,
                             const float* s_bar, uint16_t* Y_bf16, int32_t* acc_dbg, void* stream) {
  if (M < 0 || d < 0 || n < 1 || M >= kMaxDim || d >= kMaxDim) return fail(INTLORA_ESHAPE, "bad shape");
  if (n % 32 != 0 || n > 131071)
    return fail(INTLORA_ESHAPE, "linear_fwd_codes needs n a multiple of 32 and <= 131071 (got %lld)", (long long)n);
  if ((int64_t)((M + 255) / 256) * (int64_t)((d + 127) / 128) >= (int64_t(1) << 31))
    return fail(INTLORA_ESHAPE, "too many tiles");
  if (M == 0 || d == 0) return ok();
  int s = check_ptrs({xq, s_x, u_code, w_round, z, z_bar, s_bar, Y_bf16}, "linear_fwd_codes");
  if (s) return s;
  if ((s = check_opt(acc_dbg, "acc_dbg"))) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_linear_codes(M, d, n, xq, s_x, u_code, w_round, z, z_bar, s_bar, Y_bf16,
                                                    acc_dbg, static_cast<hipStream_t>(stream)),
                       "linear_codes");
}

int intlora_debug_ln(int64_t count, const uint32_t* G, float* out, void* stream) {
  if (count < 0) return fail(INTLORA_ESHAPE, "count < 0");
  if (count == 0) return ok();
  int s = check_ptrs({G, out}, "debug_ln");
  if (s) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_ln_odd(count, G, out, static_cast<hipStream_t>(stream)), "debug_ln");
}

int intlora_debug_mfma_chain(int form, int64_t d, int64_t n, int r, const float* A, const float* B, float* acc,
                             void* stream) {
  if (form != 0 && form != 1) return fail(INTLORA_EINVAL, "form must be 0 (32x32x1) or 1 (4x4x1) (got %d)", form);
  if (r < 1 || r > 128) return fail(INTLORA_EINVAL, "rank r must be in [1, 128] (got %d)", r);
  const int64_t rows = form == 0 ? 32 : 4;
  if (d < 0 || n < 0 || d % rows != 0 || n % 64 != 0 || d >= kMaxDim || n >= kMaxDim || d / rows > 65535)
    return fail(INTLORA_ESHAPE, "debug_mfma_chain: d a multiple of %lld (tiles <= 65535), n of 64", (long long)rows);
  if (d == 0 || n == 0) return ok();
  int s = check_ptrs({A, B, acc}, "debug_mfma_chain");
  if (s) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_debug_mfma_chain(form, d, n, r, A, B, acc, static_cast<hipStream_t>(stream)),
                       "debug_mfma_chain");
}

int intlora_debug_aux(int64_t blocks, const uint32_t* words, uint32_t aux_dist, float* out, void* stream) {
  if (blocks < 0) return fail(INTLORA_ESHAPE, "blocks < 0");
  if (aux_dist > INTLORA_AUX_STUDENT_T2) return fail(INTLORA_EINVAL, "aux_dist must be 0..3 (got %u)", aux_dist);
  if (blocks == 0) return ok();
  int s = check_ptrs({words, out}, "debug_aux");
  if (s) return s;
  if ((s = ensure_device())) return s;
  return launch_status(intlora::launch_aux_debug(blocks, words, (int)aux_dist, out, static_cast<hipStream_t>(stream)),
                       "debug_aux");
}

}  // extern "C"
