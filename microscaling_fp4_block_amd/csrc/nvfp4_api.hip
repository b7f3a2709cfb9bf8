// nvfp4_api.hip -- the C ABI declared in include/nvfp4.h: host-side argument
// checks (made before anything is enqueued, so they run without a GPU) and
// kernel launches on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>
#include <mutex>

#include "../../include/mxfp4.h"
#include "../../include/nvfp4.h"
#include "nvfp4_internal.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxBlocks = 1ll << 29;  // 32-bit chunk and block indices never overflow

// A C caller may pass any int as an enum argument; read it as an int, so that an
// out-of-range value is rejected without being loaded as the C++ enum type.
template <class E>
int enum_int(const E &e) {
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}
bool dtype_ok(const nvfp4_dtype &d) {
  const int v = enum_int(d);
  return v == NVFP4_F32 || v == NVFP4_BF16;
}
// a * b <= lim for a, b >= 0, decided without forming a product that could overflow
bool prod_le(int64_t a, int64_t b, int64_t lim) { return a == 0 || b <= lim / a; }
constexpr int64_t k2p31 = 1ll << 31;
bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

size_t workspace_needed() { return (size_t)kMaxAmaxGroups * sizeof(uint32_t); }

nvfp4_status hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP; }

int amax_groups(uint64_t nblocks, bool bf16) {
  const uint64_t chunks = nblocks * (bf16 ? 2u : 4u);
  uint64_t g = (chunks + 4ull * kThreads - 1) / (4ull * kThreads);
  if (g < 1) g = 1;
  if (g > (uint64_t)kMaxAmaxGroups) g = kMaxAmaxGroups;
  return (int)g;
}

RegionMap plain_map(int64_t rows, int64_t cols) {
  RegionMap m{};
  m.nblocks = (uint32_t)(rows * (cols / 16));
  m.bpr = (uint32_t)(cols / 16);
  m.div_bpr = make_fastdiv(m.bpr ? m.bpr : 1);
  m.segments = 0;
  m.tm = 1;
  m.div_tm = make_fastdiv(1);
  m.cols = (uint32_t)cols;
  return m;
}

// Global amax pass: one partial maximum per workgroup into the workspace.
// Returns the number of partials (0 on a launch error).
int run_amax(const void *x, bool bf16, bool hadamard, const HadamardSigns &hs, const RegionMap &m,
             void *ws, hipStream_t s, const Balance &bal = Balance{nullptr, 1}) {
  AmaxArgs a{x, (uint32_t *)ws, m, hs, bal};
  int groups;
  hipError_t e;
  if (hadamard) {
    groups = amax_hadamard_groups(m.nblocks);
    e = launch_amax_hadamard(a, groups, s);
  } else {
    groups = amax_groups(m.nblocks, bf16);
    e = launch_amax(a, bf16, groups, s);
  }
  return e == hipSuccess ? groups : 0;
}

// Global amax + finalize into gscale (the tensor scale alone).
nvfp4_status run_global_scale(const void *x, bool bf16, bool hadamard, const HadamardSigns &hs,
                              const RegionMap &m, float *gscale, void *ws, hipStream_t s,
                              const Balance &bal = Balance{nullptr, 1}) {
  const int groups = run_amax(x, bf16, hadamard, hs, m, ws, s, bal);
  if (groups == 0) return NVFP4_EHIP;
  return hip_status(launch_finalize((const uint32_t *)ws, groups, gscale, s));
}

hipError_t run_quantize(const QuantArgs &q, bool bf16, bool hadamard, hipStream_t s) {
  return hadamard ? launch_quantize_hadamard(q, s) : launch_quantize(q, bf16, s);
}

// Quantize a region: the amax pass (unless the tensor scale is given), then the
// search kernel, which reduces the partials to S_g in its prologue. An empty
// region still gets its tensor scale.
nvfp4_status run_quantize_region(const void *x, bool bf16, bool had, const HadamardSigns &hs,
                                 bool given, const RegionMap &m, int f_lo, int f_hi,
                                 uint8_t *codes, uint8_t *scales, float *gscale, void *ws,
                                 hipStream_t s, const Balance &bal = Balance{nullptr, 1}) {
  if (m.nblocks == 0)
    return given ? NVFP4_OK : run_global_scale(x, bf16, had, hs, m, gscale, ws, s, bal);
  int np = 0;
  if (!given) {
    np = run_amax(x, bf16, had, hs, m, ws, s, bal);
    if (np == 0) return NVFP4_EHIP;
  }
  QuantArgs q{x, codes, scales, gscale, (const uint32_t *)ws, np, m, f_lo, f_hi, hs, bal};
  return hip_status(run_quantize(q, bf16, had, s));
}


HadamardSigns make_signs(const uint32_t *signs) {
  HadamardSigns h{};
  if (signs) {
    h.on = 1;
    for (int i = 0; i < 4; ++i) h.w[i] = signs[i];
  }
  return h;
}

nvfp4_status check_offsets(int block, int f_lo, int f_hi) {
  if (block != 16) return NVFP4_EINVAL;
  if (f_lo > 0 || f_hi < 0 || f_lo < -126 || f_hi > 126) return NVFP4_EINVAL;
  return NVFP4_OK;
}

nvfp4_status check_shape(int64_t rows, int64_t cols, uint32_t flags, const nvfp4_dtype &dt) {
  if (rows < 0 || cols <= 0 || cols % 16) return NVFP4_ESHAPE;
  if (cols > (1ll << 30) || (rows > 0 && rows > kMaxBlocks / (cols / 16))) return NVFP4_ESHAPE;
  if (flags & ~(NVFP4_HADAMARD128 | NVFP4_GSCALE_GIVEN)) return NVFP4_EINVAL;
  if (flags & NVFP4_HADAMARD128) {
    if (enum_int(dt) != NVFP4_BF16) return NVFP4_EINVAL;
    if (cols % 128) return NVFP4_ESHAPE;
  }
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char *nvfp4_status_str(nvfp4_status s) {
  switch (enum_int(s)) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument";
    case NVFP4_ESHAPE: return "invalid shape";
    case NVFP4_EALIGN: return "misaligned pointer";
    case NVFP4_EWORKSPACE: return "workspace missing or too small";
    case NVFP4_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

size_t nvfp4_workspace_bytes(int64_t rows, int64_t cols, uint32_t flags) {
  (void)rows;
  (void)cols;
  (void)flags;
  return workspace_needed();
}

}  // extern "C"

namespace {

// The entry points below with signs == nullptr (plain transform or none), and
// the *_rht entry points with the caller's signs and the transform forced on.

nvfp4_status global_scale_impl(const void *x, const nvfp4_dtype &xdt, int64_t rows, int64_t cols,
                               uint32_t flags, const uint32_t *signs, float *global_scale,
                               void *workspace, size_t workspace_bytes, void *stream) {
  if (!global_scale || !dtype_ok(xdt)) return NVFP4_EINVAL;
  nvfp4_status st = check_shape(rows, cols, flags & ~NVFP4_GSCALE_GIVEN, xdt);
  if (st) return st;
  if (rows > 0 && !x) return NVFP4_EINVAL;
  if (!aligned(x, 16)) return NVFP4_EALIGN;
  if (!workspace || workspace_bytes < workspace_needed() || !aligned(workspace, 4))
    return NVFP4_EWORKSPACE;
  return run_global_scale(x, enum_int(xdt) == NVFP4_BF16, flags & NVFP4_HADAMARD128, make_signs(signs),
                          plain_map(rows, cols), global_scale, workspace, (hipStream_t)stream);
}

nvfp4_status quantize_impl(const void *x, const nvfp4_dtype &xdt, int64_t rows, int64_t cols, int block,
                           int f_lo, int f_hi, uint32_t flags, const uint32_t *signs,
                           uint8_t *codes, uint8_t *scales, float *global_scale, void *workspace,
                           size_t workspace_bytes, void *stream) {
  if (!global_scale || !dtype_ok(xdt)) return NVFP4_EINVAL;
  nvfp4_status st = check_offsets(block, f_lo, f_hi);
  if (st) return st;
  st = check_shape(rows, cols, flags, xdt);
  if (st) return st;
  if (rows > 0 && (!x || !codes || !scales)) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8)) return NVFP4_EALIGN;
  const bool given = flags & NVFP4_GSCALE_GIVEN;
  if (!given && (!workspace || workspace_bytes < workspace_needed() || !aligned(workspace, 4)))
    return NVFP4_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = enum_int(xdt) == NVFP4_BF16;
  const bool had = flags & NVFP4_HADAMARD128;
  return run_quantize_region(x, bf16, had, make_signs(signs), given, plain_map(rows, cols), f_lo,
                             f_hi, codes, scales, global_scale, workspace, s);
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_global_scale(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                                uint32_t flags, float *global_scale, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return global_scale_impl(x, xdt, rows, cols, flags, nullptr, global_scale, workspace,
                           workspace_bytes, stream);
}

nvfp4_status nvfp4_global_scale_rht(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                                    uint32_t flags, const uint32_t *signs, float *global_scale,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  if (!signs) return NVFP4_EINVAL;
  return global_scale_impl(x, xdt, rows, cols, flags | NVFP4_HADAMARD128, signs, global_scale,
                           workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_quantize(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                            int block, int f_lo, int f_hi, uint32_t flags, uint8_t *codes,
                            uint8_t *scales, float *global_scale, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return quantize_impl(x, xdt, rows, cols, block, f_lo, f_hi, flags, nullptr, codes, scales,
                       global_scale, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free quantize: the partial maxima of the global amax pass live in a
// file-scope device array instead of a caller workspace. Each GPU holds its own
// copy; its address is looked up once per device (with that device current) and
// only that address is handed to the kernels. All calls on one GPU share it, so
// calls that overlap in time on one GPU race. Every call writes each partial it
// later reads (one per amax workgroup), so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
namespace {

constexpr int kScratchWords = kMaxAmaxGroups;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxScratchDevices];

// The device address of `scratch` on the device that runs `stream` (the current
// device for the null stream); nullptr if it cannot be found.
void *scratch_address(hipStream_t stream) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (scratch_dev[dev]) return scratch_dev[dev];
  if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (dev != cur) (void)hipSetDevice(cur);
  if (e != hipSuccess || !p) return nullptr;
  scratch_dev[dev] = p;
  return p;
}

}  // namespace

extern "C" {

size_t nvfp4_noalloc_scratch_bytes(void) { return sizeof(scratch); }

nvfp4_status nvfp4_quantize_noalloc(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                                    int block, int f_lo, int f_hi, uint32_t flags,
                                    uint8_t *codes, uint8_t *scales, float *global_scale,
                                    void *stream) {
  if (workspace_needed() > sizeof(scratch)) return NVFP4_EWORKSPACE;
  // argument checks first, so that an invalid call touches no device state
  if (!global_scale || !dtype_ok(xdt)) return NVFP4_EINVAL;
  nvfp4_status st = check_offsets(block, f_lo, f_hi);
  if (st) return st;
  st = check_shape(rows, cols, flags, xdt);
  if (st) return st;
  if (rows > 0 && (!x || !codes || !scales)) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8)) return NVFP4_EALIGN;
  void *ws = nullptr;
  if (!(flags & NVFP4_GSCALE_GIVEN)) {
    ws = scratch_address((hipStream_t)stream);
    if (!ws) return NVFP4_EHIP;
  }
  return quantize_impl(x, xdt, rows, cols, block, f_lo, f_hi, flags, nullptr, codes, scales,
                       global_scale, ws, ws ? sizeof(scratch) : 0, stream);
}

nvfp4_status nvfp4_quantize_rht(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                                int block, int f_lo, int f_hi, uint32_t flags,
                                const uint32_t *signs, uint8_t *codes, uint8_t *scales,
                                float *global_scale, void *workspace, size_t workspace_bytes,
                                void *stream) {
  if (!signs) return NVFP4_EINVAL;
  return quantize_impl(x, xdt, rows, cols, block, f_lo, f_hi, flags | NVFP4_HADAMARD128, signs,
                       codes, scales, global_scale, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales,
                              const float *global_scale, int64_t rows, int64_t cols, int block,
                              void *y, nvfp4_dtype ydt, void *stream) {
  if (!global_scale || !dtype_ok(ydt)) return NVFP4_EINVAL;
  if (block != 16) return NVFP4_EINVAL;
  nvfp4_status st = check_shape(rows, cols, 0, ydt);
  if (st) return st;
  if (rows > 0 && (!codes || !scales || !y)) return NVFP4_EINVAL;
  if (!aligned(codes, 8) || !aligned(y, 16)) return NVFP4_EALIGN;
  DequantArgs a{codes, scales, global_scale, y, (uint32_t)(rows * (cols / 16))};
  if (a.nblocks == 0) return NVFP4_OK;
  return hip_status(launch_dequantize(a, enum_int(ydt) == NVFP4_BF16, (hipStream_t)stream));
}

}  // extern "C"

namespace {

nvfp4_status kv_sink_impl(const void *kv, const nvfp4_dtype &dt, int64_t B, int64_t H, int64_t T,
                          int64_t D, int64_t n_first, int64_t n_last, int block, int f_lo,
                          int f_hi, uint32_t flags, const uint32_t *signs, uint8_t *codes,
                          uint8_t *scales, float *global_scale, void *sink, void *workspace,
                          size_t workspace_bytes, void *stream) {
  if (!global_scale || !dtype_ok(dt)) return NVFP4_EINVAL;
  nvfp4_status st = check_offsets(block, f_lo, f_hi);
  if (st) return st;
  if (B < 0 || H < 0 || T < 0 || D <= 0 || n_first < 0 || n_last < 0) return NVFP4_ESHAPE;
  if (T > k2p31 || n_first > T || n_last > T || !prod_le(B, H, k2p31)) return NVFP4_ESHAPE;
  if (n_first + n_last > T) return NVFP4_ESHAPE;
  const int64_t BH = B * H, NS = n_first + n_last, Tm = T - NS;
  if (BH * T > 0 && !kv) return NVFP4_EINVAL;
  if (BH * NS > 0 && !sink) return NVFP4_EINVAL;
  if (BH * Tm > 0 && (!codes || !scales)) return NVFP4_EINVAL;
  st = check_shape(BH * T, D, flags, dt);
  if (st) return st;
  if (!aligned(kv, 16) || !aligned(codes, 8) || !aligned(sink, 16)) return NVFP4_EALIGN;
  const bool given = flags & NVFP4_GSCALE_GIVEN;
  if (!given && (!workspace || workspace_bytes < workspace_needed() || !aligned(workspace, 4)))
    return NVFP4_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = enum_int(dt) == NVFP4_BF16;
  const bool had = flags & NVFP4_HADAMARD128;
  const uint32_t es = bf16 ? 2u : 4u;

  if (BH > 0 && NS > 0) {
    SinkArgs c{};
    c.src = kv;
    c.dst = sink;
    c.bh = (uint32_t)BH;
    c.T = (uint32_t)T;
    c.D = (uint32_t)D;
    c.n_first = (uint32_t)n_first;
    c.n_last = (uint32_t)n_last;
    c.chunks_per_row = (uint32_t)(D * es / 16);
    c.nchunks = (uint32_t)(BH * NS) * c.chunks_per_row;
    c.div_cpr = make_fastdiv(c.chunks_per_row);
    c.div_ns = make_fastdiv((uint32_t)NS);
    hipError_t e = launch_sink_copy(c, bf16, s);
    if (e != hipSuccess) return NVFP4_EHIP;
  }

  RegionMap m{};
  m.bpr = (uint32_t)(D / 16);
  m.nblocks = (uint32_t)(BH * Tm) * m.bpr;
  m.div_bpr = make_fastdiv(m.bpr);
  m.segments = (uint32_t)BH;
  m.tm = (uint32_t)(Tm > 0 ? Tm : 1);
  m.div_tm = make_fastdiv(m.tm);
  m.seg_tokens = (uint32_t)T;
  m.n_first = (uint32_t)n_first;
  m.cols = (uint32_t)D;
  return run_quantize_region(kv, bf16, had, make_signs(signs), given, m, f_lo, f_hi, codes, scales,
                             global_scale, workspace, s);
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_quantize_kv_sink(const void *kv, nvfp4_dtype dt, int64_t B, int64_t H,
                                    int64_t T, int64_t D, int64_t n_first, int64_t n_last,
                                    int block, int f_lo, int f_hi, uint32_t flags,
                                    uint8_t *codes, uint8_t *scales, float *global_scale,
                                    void *sink, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  return kv_sink_impl(kv, dt, B, H, T, D, n_first, n_last, block, f_lo, f_hi, flags, nullptr,
                      codes, scales, global_scale, sink, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_quantize_kv_sink_rht(const void *kv, nvfp4_dtype dt, int64_t B, int64_t H,
                                        int64_t T, int64_t D, int64_t n_first, int64_t n_last,
                                        int block, int f_lo, int f_hi, uint32_t flags,
                                        const uint32_t *signs, uint8_t *codes, uint8_t *scales,
                                        float *global_scale, void *sink, void *workspace,
                                        size_t workspace_bytes, void *stream) {
  if (!signs) return NVFP4_EINVAL;
  return kv_sink_impl(kv, dt, B, H, T, D, n_first, n_last, block, f_lo, f_hi,
                      flags | NVFP4_HADAMARD128, signs, codes, scales, global_scale, sink,
                      workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_dequantize_kv_sink(const uint8_t *codes, const uint8_t *scales,
                                      const float *global_scale, const void *sink,
                                      nvfp4_dtype sink_dt, int64_t B, int64_t H, int64_t T,
                                      int64_t D, int64_t n_first, int64_t n_last, int block,
                                      void *y, nvfp4_dtype ydt, void *stream) {
  if (!global_scale || !dtype_ok(sink_dt) || !dtype_ok(ydt)) return NVFP4_EINVAL;
  if (block != 16) return NVFP4_EINVAL;
  if (B < 0 || H < 0 || T < 0 || D <= 0 || D % 16 || n_first < 0 || n_last < 0)
    return NVFP4_ESHAPE;
  if (T > k2p31 || n_first > T || n_last > T || !prod_le(B, H, k2p31)) return NVFP4_ESHAPE;
  if (n_first + n_last > T) return NVFP4_ESHAPE;
  const int64_t BH = B * H, NS = n_first + n_last, Tm = T - NS;
  nvfp4_status st = check_shape(BH * T, D, 0, ydt);
  if (st) return st;
  if (BH * T > 0 && !y) return NVFP4_EINVAL;
  if (BH * NS > 0 && !sink) return NVFP4_EINVAL;
  if (BH * Tm > 0 && (!codes || !scales)) return NVFP4_EINVAL;
  if (!aligned(codes, 8) || !aligned(sink, 16) || !aligned(y, 16)) return NVFP4_EALIGN;
  DequantKvArgs a{};
  a.codes = codes;
  a.scales = scales;
  a.gscale = global_scale;
  a.sink = sink;
  a.y = y;
  a.bpr = (uint32_t)(D / 16);
  a.nblocks = (uint32_t)(BH * T) * a.bpr;
  a.div_bpr = make_fastdiv(a.bpr);
  a.div_T = make_fastdiv((uint32_t)(T > 0 ? T : 1));
  a.T = (uint32_t)T;
  a.n_first = (uint32_t)n_first;
  a.n_last = (uint32_t)n_last;
  if (a.nblocks == 0) return NVFP4_OK;
  return hip_status(
      launch_dequantize_kv(a, enum_int(sink_dt) == NVFP4_BF16, enum_int(ydt) == NVFP4_BF16, (hipStream_t)stream));
}

}  // extern "C"

namespace {

nvfp4_status kv_append_impl(const void *kv_new, const nvfp4_dtype &dt, int64_t B, int64_t H, int64_t T,
                            int64_t t_new, int64_t D, int64_t n_first, int64_t n_last,
                            int64_t cap, int block, int f_lo, int f_hi, uint32_t flags,
                            const uint32_t *signs, const float *global_scale, void *head,
                            void *tail, uint8_t *codes, uint8_t *scales, void *stream) {
  if (!global_scale || !dtype_ok(dt)) return NVFP4_EINVAL;
  nvfp4_status st = check_offsets(block, f_lo, f_hi);
  if (st) return st;
  if (flags & ~(NVFP4_HADAMARD128 | NVFP4_GSCALE_GIVEN)) return NVFP4_EINVAL;
  if (B < 0 || H < 0 || T < 0 || t_new < 0 || D <= 0 || D % 16 || n_first < 0 || n_last < 0 ||
      cap < 0)
    return NVFP4_ESHAPE;
  if (T > k2p31 || t_new > k2p31 || n_first > k2p31 || n_last > k2p31 || cap > k2p31 ||
      !prod_le(B, H, k2p31))
    return NVFP4_ESHAPE;
  if (T + t_new > k2p31) return NVFP4_ESHAPE;
  const bool had = flags & NVFP4_HADAMARD128;
  if (had && (enum_int(dt) != NVFP4_BF16)) return NVFP4_EINVAL;
  if (had && D % 128) return NVFP4_ESHAPE;
  const int64_t BH = B * H, T2 = T + t_new;
  // tokens entering the middle: [lo, hi); the middle must hold rows up to hi - n_first
  const int64_t lo = n_first > T - n_last ? n_first : T - n_last;
  const int64_t hi = n_first > T2 - n_last ? n_first : T2 - n_last;
  const int64_t npos = hi > lo ? hi - lo : 0;
  if (hi - n_first > cap) return NVFP4_ESHAPE;
  st = check_shape(BH * (npos > 0 ? npos : 0), D, 0, dt);
  if (st) return st;
  st = check_shape(BH * (cap > 0 ? cap : 0), D, 0, dt);
  if (st) return st;
  if (BH * t_new > 0 && !kv_new) return NVFP4_EINVAL;
  if (BH * n_first > 0 && !head) return NVFP4_EINVAL;
  if (BH * n_last > 0 && !tail) return NVFP4_EINVAL;
  if (BH * cap > 0 && (!codes || !scales)) return NVFP4_EINVAL;
  if (!aligned(kv_new, 16) || !aligned(head, 16) || !aligned(tail, 16) || !aligned(codes, 8))
    return NVFP4_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = enum_int(dt) == NVFP4_BF16;
  const uint32_t es = bf16 ? 2u : 4u;

  // 1. code the tokens that leave the recent window (before the ring is overwritten)
  QuantArgs q{};
  if (BH > 0 && npos > 0) {
    RegionMap m{};
    m.bpr = (uint32_t)(D / 16);
    m.nblocks = (uint32_t)(BH * npos) * m.bpr;
    m.div_bpr = make_fastdiv(m.bpr);
    m.segments = (uint32_t)BH;
    m.tm = (uint32_t)npos;
    m.div_tm = make_fastdiv(m.tm);
    m.cols = (uint32_t)D;
    m.n_first = (uint32_t)n_first;
    m.append = 1;
    m.lo = (uint32_t)lo;
    m.t_old = (uint32_t)T;
    m.n_last = (uint32_t)n_last;
    m.t_new = (uint32_t)t_new;
    m.cap = (uint32_t)cap;
    m.div_nlast = make_fastdiv((uint32_t)(n_last > 0 ? n_last : 1));
    m.ring = tail;
    q = QuantArgs{kv_new, codes, scales, (float *)global_scale, nullptr, 0, m, f_lo, f_hi,
                  make_signs(signs)};
  }
  // 2. store the new tokens that stay in full precision
  AdmitArgs c{};
  if (BH > 0 && t_new > 0) {
    c.src = kv_new;
    c.head = head;
    c.tail = tail;
    c.t_old = (uint32_t)T;
    c.t_new = (uint32_t)t_new;
    c.n_first = (uint32_t)n_first;
    c.n_last = (uint32_t)n_last;
    c.chunks_per_row = (uint32_t)(D * es / 16);
    c.nchunks = (uint32_t)(BH * t_new) * c.chunks_per_row;
    c.div_cpr = make_fastdiv(c.chunks_per_row);
    c.div_tnew = make_fastdiv((uint32_t)t_new);
    c.div_nlast = make_fastdiv((uint32_t)(n_last > 0 ? n_last : 1));
  }
  if (q.map.nblocks == 0 && c.nchunks == 0) return NVFP4_OK;
  if (!had && q.map.nblocks <= kSmallAppendBlocks && c.nchunks <= kSmallAppendChunks) {
    q.gscale = (float *)global_scale;
    return hip_status(launch_kv_append_small(q, c, nullptr, bf16, s));
  }
  if (q.map.nblocks > 0 && run_quantize(q, bf16, had, s) != hipSuccess) return NVFP4_EHIP;
  if (c.nchunks > 0 && launch_admit(c, bf16, s) != hipSuccess) return NVFP4_EHIP;
  return NVFP4_OK;
}

// The append at a device-resident length: the kernels read t_old from *length
// when they run and the last one advances it; an append that would overflow
// the cache (t_old + t_new > n_first + cap + n_last) leaves cache and length
// unchanged. Host checks cover everything that does not depend on t_old.
// With `plan` given, the checks run and the launch arguments are returned
// there instead of being launched (the paired K and V append).
struct KvAppendPlan {
  QuantArgs q;
  AdmitArgs c;
  bool empty, small;
};

nvfp4_status kv_append_dev_impl(const void *kv_new, const nvfp4_dtype &dt, int64_t B, int64_t H,
                                int64_t t_new, int64_t D, int64_t n_first, int64_t n_last,
                                int64_t cap, int block, int f_lo, int f_hi, uint32_t flags,
                                const uint32_t *signs, const float *global_scale, void *head,
                                void *tail, uint8_t *codes, uint8_t *scales, int64_t *length,
                                void *stream, KvAppendPlan *plan = nullptr) {
  if (!global_scale || !length || !dtype_ok(dt)) return NVFP4_EINVAL;
  nvfp4_status st = check_offsets(block, f_lo, f_hi);
  if (st) return st;
  if (flags & ~(NVFP4_HADAMARD128 | NVFP4_GSCALE_GIVEN)) return NVFP4_EINVAL;
  if (B < 0 || H < 0 || t_new < 0 || D <= 0 || D % 16 || n_first < 0 || n_last < 0 || cap < 0)
    return NVFP4_ESHAPE;
  if (t_new > k2p31 || n_first > k2p31 || n_last > k2p31 || cap > k2p31 || !prod_le(B, H, k2p31))
    return NVFP4_ESHAPE;
  const int64_t total = n_first + cap + n_last;
  if (total > k2p31) return NVFP4_ESHAPE;
  const bool had = flags & NVFP4_HADAMARD128;
  if (had && (enum_int(dt) != NVFP4_BF16)) return NVFP4_EINVAL;
  if (had && D % 128) return NVFP4_ESHAPE;
  const int64_t BH = B * H;
  st = check_shape(BH * t_new, D, 0, dt);
  if (st) return st;
  st = check_shape(BH * cap, D, 0, dt);
  if (st) return st;
  if (BH * t_new > 0 && !kv_new) return NVFP4_EINVAL;
  if (BH * n_first > 0 && !head) return NVFP4_EINVAL;
  if (BH * n_last > 0 && !tail) return NVFP4_EINVAL;
  if (BH * cap > 0 && (!codes || !scales)) return NVFP4_EINVAL;
  if (!aligned(kv_new, 16) || !aligned(head, 16) || !aligned(tail, 16) || !aligned(codes, 8) ||
      !aligned(length, 8))
    return NVFP4_EALIGN;
  if (plan) plan->empty = t_new == 0;
  if (t_new == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = enum_int(dt) == NVFP4_BF16;
  const uint32_t es = bf16 ? 2u : 4u;
  QuantArgs q{};
  q.gscale = (float *)global_scale;
  AdmitArgs c{};
  c.len_dev = length;
  c.t_new = (uint32_t)t_new;
  c.total = (uint32_t)total;
  if (BH > 0) {
    // 1. code the tokens that leave the recent window: at most t_new rows per segment
    RegionMap m{};
    m.bpr = (uint32_t)(D / 16);
    m.nblocks = (uint32_t)(BH * t_new) * m.bpr;
    m.div_bpr = make_fastdiv(m.bpr);
    m.segments = (uint32_t)BH;
    m.tm = (uint32_t)t_new;
    m.div_tm = make_fastdiv(m.tm);
    m.cols = (uint32_t)D;
    m.n_first = (uint32_t)n_first;
    m.append = 1;
    m.n_last = (uint32_t)n_last;
    m.t_new = (uint32_t)t_new;
    m.cap = (uint32_t)cap;
    m.div_nlast = make_fastdiv((uint32_t)(n_last > 0 ? n_last : 1));
    m.ring = tail;
    m.len_dev = length;
    m.total = (uint32_t)total;
    q = QuantArgs{kv_new, codes, scales, (float *)global_scale, nullptr, 0, m, f_lo, f_hi,
                  make_signs(signs)};
    // 2. store the new tokens that stay in full precision
    c.src = kv_new;
    c.head = head;
    c.tail = tail;
    c.t_new = (uint32_t)t_new;
    c.n_first = (uint32_t)n_first;
    c.n_last = (uint32_t)n_last;
    c.chunks_per_row = (uint32_t)(D * es / 16);
    c.nchunks = (uint32_t)(BH * t_new) * c.chunks_per_row;
    c.div_cpr = make_fastdiv(c.chunks_per_row);
    c.div_tnew = make_fastdiv((uint32_t)t_new);
    c.div_nlast = make_fastdiv((uint32_t)(n_last > 0 ? n_last : 1));
  }
  // small appends (a decode step's): all three steps in one workgroup
  const bool small =
      !had && q.map.nblocks <= kSmallAppendBlocks && c.nchunks <= kSmallAppendChunks;
  if (plan) {  // checked, nothing launched
    plan->q = q;
    plan->c = c;
    plan->small = small;
    return NVFP4_OK;
  }
  if (small) return hip_status(launch_kv_append_small(q, c, length, bf16, s));
  if (BH > 0) {
    if (run_quantize(q, bf16, had, s) != hipSuccess) return NVFP4_EHIP;
    if (launch_admit(c, bf16, s) != hipSuccess) return NVFP4_EHIP;
  }
  // 3. advance the length (after both kernels read it)
  return hip_status(launch_advance_length(length, (uint32_t)t_new, (uint32_t)total, s));
}

nvfp4_status hadamard_impl(const void *x, const nvfp4_dtype &xdt, int64_t rows, const uint32_t *signs,
                           float *y, void *stream) {
  if (enum_int(xdt) != NVFP4_BF16) return NVFP4_EINVAL;
  if (rows < 0 || rows > kMaxBlocks / 8) return NVFP4_ESHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!x || !y) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16)) return NVFP4_EALIGN;
  return hip_status(launch_hadamard((const uint16_t *)x, y, (uint32_t)rows, make_signs(signs),
                                    Balance{nullptr, 1}, (hipStream_t)stream));
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_kv_append(const void *kv_new, nvfp4_dtype dt, int64_t B, int64_t H,
                             int64_t T, int64_t t_new, int64_t D, int64_t n_first,
                             int64_t n_last, int64_t cap, int block, int f_lo, int f_hi,
                             uint32_t flags, const float *global_scale, void *head, void *tail,
                             uint8_t *codes, uint8_t *scales, void *stream) {
  return kv_append_impl(kv_new, dt, B, H, T, t_new, D, n_first, n_last, cap, block, f_lo, f_hi,
                        flags, nullptr, global_scale, head, tail, codes, scales, stream);
}

nvfp4_status nvfp4_kv_append_rht(const void *kv_new, nvfp4_dtype dt, int64_t B, int64_t H,
                                 int64_t T, int64_t t_new, int64_t D, int64_t n_first,
                                 int64_t n_last, int64_t cap, int block, int f_lo, int f_hi,
                                 uint32_t flags, const uint32_t *signs, const float *global_scale,
                                 void *head, void *tail, uint8_t *codes, uint8_t *scales,
                                 void *stream) {
  if (!signs) return NVFP4_EINVAL;
  return kv_append_impl(kv_new, dt, B, H, T, t_new, D, n_first, n_last, cap, block, f_lo, f_hi,
                        flags | NVFP4_HADAMARD128, signs, global_scale, head, tail, codes, scales,
                        stream);
}

nvfp4_status nvfp4_kv_append_dev(const void *kv_new, nvfp4_dtype dt, int64_t B, int64_t H,
                                 int64_t t_new, int64_t D, int64_t n_first, int64_t n_last,
                                 int64_t cap, int block, int f_lo, int f_hi, uint32_t flags,
                                 const uint32_t *signs, const float *global_scale, void *head,
                                 void *tail, uint8_t *codes, uint8_t *scales, int64_t *length,
                                 void *stream) {
  return kv_append_dev_impl(kv_new, dt, B, H, t_new, D, n_first, n_last, cap, block, f_lo, f_hi,
                            signs ? (flags | NVFP4_HADAMARD128) : flags, signs, global_scale,
                            head, tail, codes, scales, length, stream);
}

nvfp4_status nvfp4_kv_append2_dev(const nvfp4_kv_cache_ref *k, const nvfp4_kv_cache_ref *v,
                                  nvfp4_dtype dt, int64_t B, int64_t H, int64_t t_new, int64_t D,
                                  int64_t n_first, int64_t n_last, int64_t cap, int block,
                                  int f_lo, int f_hi, void *stream) {
  if (!k || !v) return NVFP4_EINVAL;
  if (k->length && k->length == v->length) return NVFP4_EINVAL;  // one length each
  const nvfp4_kv_cache_ref *r[2] = {k, v};
  KvAppendPlan plan[2];
  for (int i = 0; i < 2; ++i) {  // every check first: nothing runs unless both pass
    const nvfp4_kv_cache_ref &c = *r[i];
    const nvfp4_status st = kv_append_dev_impl(
        c.kv_new, dt, B, H, t_new, D, n_first, n_last, cap, block, f_lo, f_hi,
        c.signs ? (c.flags | NVFP4_HADAMARD128) : c.flags, c.signs, c.global_scale, c.head,
        c.tail, c.codes, c.scales, c.length, stream, &plan[i]);
    if (st) return st;
  }
  if (plan[0].empty) return NVFP4_OK;
  if (plan[0].small && plan[1].small) {
    KvAppendPair p{};
    for (int i = 0; i < 2; ++i) {
      p.q[i] = plan[i].q;
      p.c[i] = plan[i].c;
      p.len[i] = r[i]->length;
    }
    p.row_bytes = plan[0].c.chunks_per_row * 16u;
    return hip_status(launch_kv_append_small_pair(p, enum_int(dt) == NVFP4_BF16, (hipStream_t)stream));
  }
  for (int i = 0; i < 2; ++i) {
    const nvfp4_kv_cache_ref &c = *r[i];
    const nvfp4_status st = kv_append_dev_impl(
        c.kv_new, dt, B, H, t_new, D, n_first, n_last, cap, block, f_lo, f_hi,
        c.signs ? (c.flags | NVFP4_HADAMARD128) : c.flags, c.signs, c.global_scale, c.head,
        c.tail, c.codes, c.scales, c.length, stream);
    if (st) return st;
  }
  return NVFP4_OK;
}

nvfp4_status nvfp4_hadamard128(const void *x, nvfp4_dtype xdt, int64_t rows, float *y,
                               void *stream) {
  return hadamard_impl(x, xdt, rows, nullptr, y, stream);
}

nvfp4_status nvfp4_hadamard128_rht(const void *x, nvfp4_dtype xdt, int64_t rows,
                                   const uint32_t *signs, float *y, void *stream) {
  if (!signs) return NVFP4_EINVAL;
  return hadamard_impl(x, xdt, rows, signs, y, stream);
}

nvfp4_status mxfp4_quantize(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                            int block, int f_lo, int f_hi, uint8_t *codes, uint8_t *scales,
                            void *stream) {
  if (!dtype_ok(xdt) || block != 32) return NVFP4_EINVAL;
  if (f_lo > 0 || f_hi < 0 || f_lo < -8 || f_hi > 8) return NVFP4_EINVAL;
  if (rows < 0 || cols <= 0 || cols % 32) return NVFP4_ESHAPE;
  if (cols > (1ll << 30) || (rows > 0 && rows > kMaxBlocks / (cols / 16))) return NVFP4_ESHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!x || !codes || !scales) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16)) return NVFP4_EALIGN;
  MxArgs a{x, codes, scales, (uint32_t)(rows * (cols / 32)), f_lo, f_hi};
  return hip_status(launch_mx_quantize(a, enum_int(xdt) == NVFP4_BF16, (hipStream_t)stream));
}

nvfp4_status mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                              int64_t cols, int block, void *y, nvfp4_dtype ydt, void *stream) {
  if (!dtype_ok(ydt) || block != 32) return NVFP4_EINVAL;
  if (rows < 0 || cols <= 0 || cols % 32) return NVFP4_ESHAPE;
  if (cols > (1ll << 30) || (rows > 0 && rows > kMaxBlocks / (cols / 16))) return NVFP4_ESHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!codes || !scales || !y) return NVFP4_EINVAL;
  if (!aligned(codes, 16) || !aligned(y, 16)) return NVFP4_EALIGN;
  MxDequantArgs a{codes, scales, y, (uint32_t)(rows * (cols / 32))};
  return hip_status(launch_mx_dequantize(a, enum_int(ydt) == NVFP4_BF16, (hipStream_t)stream));
}

nvfp4_status nvfp4_attention(const uint8_t *q_codes, const uint8_t *q_scales,
                             const float *q_gscale, const uint8_t *k_codes,
                             const uint8_t *k_scales, const float *k_gscale,
                             const uint8_t *v_codes, const uint8_t *v_scales,
                             const float *v_gscale, int64_t B, int64_t Hq, int64_t Hkv,
                             int64_t Nq, int64_t Nk, int64_t D, int causal, void *out,
                             nvfp4_dtype out_dt, void *stream) {
  if (!dtype_ok(out_dt)) return NVFP4_EINVAL;
  if (D != 128) return NVFP4_ESHAPE;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Nq < 0 || Nk < 0) return NVFP4_ESHAPE;
  if (!prod_le(B, Hq, 65535) || Nq > (1ll << 30) || Nk > (1ll << 30)) return NVFP4_ESHAPE;
  if (B * Hq * Nq > kMaxBlocks / 8 || B * Hkv * Nk > kMaxBlocks / 8) return NVFP4_ESHAPE;
  if (B * Nq == 0) return NVFP4_OK;
  if (!q_codes || !q_scales || !q_gscale || !k_gscale || !v_gscale || !out) return NVFP4_EINVAL;
  if (Nk > 0 && (!k_codes || !k_scales || !v_codes || !v_scales)) return NVFP4_EINVAL;
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(out, 16) ||
      !aligned(q_scales, 8) || !aligned(k_scales, 8) || !aligned(v_scales, 8))
    return NVFP4_EALIGN;
  AttnArgs a{};
  a.qc = q_codes;
  a.qs = q_scales;
  a.kc = k_codes;
  a.ks = k_scales;
  a.vc = v_codes;
  a.vs = v_scales;
  a.qg = q_gscale;
  a.kg = k_gscale;
  a.vg = v_gscale;
  a.o = out;
  a.B = (uint32_t)B;
  a.Hq = (uint32_t)Hq;
  a.Hkv = (uint32_t)Hkv;
  a.Nq = (uint32_t)Nq;
  a.Nk = (uint32_t)Nk;
  a.causal = causal ? 1u : 0u;
  a.tau_log2e = (float)(1.4426950408889634 / sqrt(128.0));
  return hip_status(launch_attention(a, enum_int(out_dt) == NVFP4_BF16, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Attention over the sink cache with T tokens, or (len_dev set) with the token
// count read from that device word when the kernel runs (clamped to the
// cache's n_first + cap + n_last); checks that need T are then made on the
// cache's capacity instead.
// Units of a split cache attention sized for a middle of `cap` tokens: the
// head, the tail and ceil(cap / split) pieces.
int64_t split_units(int64_t cap, int64_t split) { return 2 + (cap + split - 1) / split; }

nvfp4_status attention_kv_cache_impl(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, const nvfp4_dtype &cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    int64_t T, const int64_t *len_dev, int64_t D, int64_t n_first, int64_t n_last, int64_t cap,
    int64_t split, void *workspace, size_t workspace_bytes, void *out, const nvfp4_dtype &out_dt,
    void *stream) {
  if (!dtype_ok(out_dt) || enum_int(cache_dt) != NVFP4_BF16) return NVFP4_EINVAL;
  if (split < 0 || split % 32 || split > (1ll << 30)) return NVFP4_EINVAL;
  if (D != 128) return NVFP4_ESHAPE;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Nq < 0 || T < 0 || n_first < 0 || n_last < 0 ||
      cap < 0)
    return NVFP4_ESHAPE;
  if (!prod_le(B, Hq, 65535) || Nq > (1ll << 30) || T > (1ll << 30) || cap > (1ll << 30) ||
      n_first > (1ll << 30) || n_last > (1ll << 30))
    return NVFP4_ESHAPE;
  const int64_t mid = len_dev ? cap : T - n_first - n_last;
  if (mid > cap) return NVFP4_ESHAPE;
  if (B * Hq * Nq > kMaxBlocks / 8 || B * Hkv * cap > kMaxBlocks / 8) return NVFP4_ESHAPE;
  if (B * Nq == 0) return NVFP4_OK;
  if (!q_codes || !q_scales || !q_gscale || !k_gscale || !v_gscale || !out) return NVFP4_EINVAL;
  const int64_t span = len_dev ? n_first + cap + n_last : T;  // tokens that may be read
  if (n_first > 0 && span > 0 && (!k_head || !v_head)) return NVFP4_EINVAL;
  if (n_last > 0 && span > n_first && (!k_tail || !v_tail)) return NVFP4_EINVAL;
  if (mid > 0 && (!k_codes || !k_scales || !v_codes || !v_scales)) return NVFP4_EINVAL;
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_head, 16) || !aligned(k_tail, 16) || !aligned(v_head, 16) ||
      !aligned(v_tail, 16) || !aligned(out, 16) || !aligned(len_dev, 8) ||
      !aligned(q_scales, 8) || !aligned(k_scales, 8) || !aligned(v_scales, 8))
    return NVFP4_EALIGN;
  if (split > 0) {
    if (split_units(cap, split) > 65535) return NVFP4_ESHAPE;
    const size_t need = nvfp4_attention_split_workspace_bytes(B, Hq, Nq, cap, split);
    if (!workspace || need == 0 || workspace_bytes < need) return NVFP4_EWORKSPACE;
    if (!aligned(workspace, 16)) return NVFP4_EALIGN;
  }
  AttnArgs a{};
  a.qc = q_codes;
  a.qs = q_scales;
  a.kc = k_codes;
  a.ks = k_scales;
  a.vc = v_codes;
  a.vs = v_scales;
  a.qg = q_gscale;
  a.kg = k_gscale;
  a.vg = v_gscale;
  a.o = out;
  a.B = (uint32_t)B;
  a.Hq = (uint32_t)Hq;
  a.Hkv = (uint32_t)Hkv;
  a.Nq = (uint32_t)Nq;
  a.Nk = (uint32_t)T;
  a.causal = 0u;
  a.tau_log2e = (float)(1.4426950408889634 / sqrt(128.0));
  a.cache = 1u;
  a.kh = (const uint16_t *)k_head;
  a.kt = (const uint16_t *)k_tail;
  a.vh = (const uint16_t *)v_head;
  a.vt = (const uint16_t *)v_tail;
  a.nf = (uint32_t)n_first;
  a.nl = (uint32_t)n_last;
  a.cap = (uint32_t)cap;
  a.nk_dev = len_dev;
  if (split > 0) {
    const int64_t part = split_units(cap, split) * B * Hq * Nq * 128;
    a.split = (uint32_t)split;
    a.ustride = (uint32_t)split_units(cap, split);
    a.part = (float *)workspace;
    a.ml = (float2 *)((float *)workspace + part);
  }
  return hip_status(launch_attention(a, enum_int(out_dt) == NVFP4_BF16, (hipStream_t)stream));
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_attention_kv_cache(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, nvfp4_dtype cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    int64_t T, int64_t D, int64_t n_first, int64_t n_last, int64_t cap, void *out,
    nvfp4_dtype out_dt, void *stream) {
  return attention_kv_cache_impl(q_codes, q_scales, q_gscale, k_head, k_tail, k_codes, k_scales,
                                 k_gscale, v_head, v_tail, v_codes, v_scales, v_gscale, cache_dt,
                                 B, Hq, Hkv, Nq, T, nullptr, D, n_first, n_last, cap, 0, nullptr,
                                 0, out, out_dt, stream);
}

nvfp4_status nvfp4_attention_kv_cache_dev(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, nvfp4_dtype cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    const int64_t *length, int64_t D, int64_t n_first, int64_t n_last, int64_t cap, void *out,
    nvfp4_dtype out_dt, void *stream) {
  if (!length) return NVFP4_EINVAL;
  return attention_kv_cache_impl(q_codes, q_scales, q_gscale, k_head, k_tail, k_codes, k_scales,
                                 k_gscale, v_head, v_tail, v_codes, v_scales, v_gscale, cache_dt,
                                 B, Hq, Hkv, Nq, 0, length, D, n_first, n_last, cap, 0, nullptr,
                                 0, out, out_dt, stream);
}

size_t nvfp4_attention_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t cap,
                                             int64_t split) {
  if (B < 0 || Hq <= 0 || Nq < 0 || cap < 0 || cap > (1ll << 30) || split <= 0 || split % 32 ||
      split > (1ll << 30) || !prod_le(B, Hq, 65535) || Nq > (1ll << 30))
    return 0;
  const int64_t units = split_units(cap, split), rows = B * Hq * Nq;
  if (units > 65535 || rows > kMaxBlocks / 8) return 0;
  // per unit and row: 128 FP32 accumulator values, then (max, sum)
  return (size_t)(units * rows) * (128 * sizeof(float) + 2 * sizeof(float));
}

nvfp4_status nvfp4_attention_kv_cache_split(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, nvfp4_dtype cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    int64_t T, int64_t D, int64_t n_first, int64_t n_last, int64_t cap, int64_t split,
    void *workspace, size_t workspace_bytes, void *out, nvfp4_dtype out_dt, void *stream) {
  if (split <= 0) return NVFP4_EINVAL;
  return attention_kv_cache_impl(q_codes, q_scales, q_gscale, k_head, k_tail, k_codes, k_scales,
                                 k_gscale, v_head, v_tail, v_codes, v_scales, v_gscale, cache_dt,
                                 B, Hq, Hkv, Nq, T, nullptr, D, n_first, n_last, cap, split,
                                 workspace, workspace_bytes, out, out_dt, stream);
}

nvfp4_status nvfp4_attention_kv_cache_split_dev(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, nvfp4_dtype cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    const int64_t *length, int64_t D, int64_t n_first, int64_t n_last, int64_t cap, int64_t split,
    void *workspace, size_t workspace_bytes, void *out, nvfp4_dtype out_dt, void *stream) {
  if (!length || split <= 0) return NVFP4_EINVAL;
  return attention_kv_cache_impl(q_codes, q_scales, q_gscale, k_head, k_tail, k_codes, k_scales,
                                 k_gscale, v_head, v_tail, v_codes, v_scales, v_gscale, cache_dt,
                                 B, Hq, Hkv, Nq, 0, length, D, n_first, n_last, cap, split,
                                 workspace, workspace_bytes, out, out_dt, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The balancing pair of incoherence processing (ScaleSearch summary page,
// ScaleSearchAttention, 非干渉処理（IP）と絶対値低減): Q' = Q diag(2^-e),
// K' = K diag(2^e), before the Hadamard transform when one is used.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kMaxBalanceCols = 2048;

size_t balance_ws(int64_t cols) {
  return (size_t)2 * kColSumGroups * (size_t)cols * sizeof(double);
}

Balance make_balance(const int8_t *e, uint32_t flags) {
  return Balance{e, (flags & NVFP4_PAIR_Q) ? -1 : 1};
}

}  // namespace

extern "C" {

size_t nvfp4_balance_workspace_bytes(int64_t cols) {
  return (cols > 0 && cols <= kMaxBalanceCols) ? balance_ws(cols) : 0;
}

nvfp4_status nvfp4_balance_exponents(const void *q, const void *k, nvfp4_dtype dt, int64_t rows_q,
                                     int64_t rows_k, int64_t cols, int8_t *chan_exp,
                                     void *workspace, size_t workspace_bytes, void *stream) {
  if (!dtype_ok(dt) || !chan_exp) return NVFP4_EINVAL;
  if (cols <= 0 || cols % 16 || cols > kMaxBalanceCols || rows_q < 0 || rows_k < 0 ||
      rows_q >= k2p31 || rows_k >= k2p31)
    return NVFP4_ESHAPE;
  if ((rows_q > 0 && !q) || (rows_k > 0 && !k)) return NVFP4_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16)) return NVFP4_EALIGN;
  if (!workspace || workspace_bytes < balance_ws(cols) || !aligned(workspace, 8))
    return NVFP4_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = enum_int(dt) == NVFP4_BF16;
  double *qp = (double *)workspace, *kp = qp + (size_t)kColSumGroups * (size_t)cols;
  if (launch_colsumsq(ColSumArgs{q, (uint32_t)rows_q, (uint32_t)cols, qp}, bf16, s) != hipSuccess)
    return NVFP4_EHIP;
  if (launch_colsumsq(ColSumArgs{k, (uint32_t)rows_k, (uint32_t)cols, kp}, bf16, s) != hipSuccess)
    return NVFP4_EHIP;
  return hip_status(launch_balance_exponents(qp, kp, (uint32_t)cols, chan_exp, s));
}

nvfp4_status nvfp4_quantize_balanced(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                                     int block, int f_lo, int f_hi, uint32_t flags,
                                     const int8_t *chan_exp, const uint32_t *signs,
                                     uint8_t *codes, uint8_t *scales, float *global_scale,
                                     void *workspace, size_t workspace_bytes, void *stream) {
  if (!global_scale || !dtype_ok(xdt) || !chan_exp) return NVFP4_EINVAL;
  if (flags & ~(NVFP4_HADAMARD128 | NVFP4_GSCALE_GIVEN | NVFP4_PAIR_Q)) return NVFP4_EINVAL;
  const bool had = flags & NVFP4_HADAMARD128;
  if (signs && !had) return NVFP4_EINVAL;
  nvfp4_status st = check_offsets(block, f_lo, f_hi);
  if (st) return st;
  st = check_shape(rows, cols, flags & ~NVFP4_PAIR_Q, xdt);
  if (st) return st;
  if (had && cols != 128) return NVFP4_ESHAPE;
  if (rows > 0 && (!x || !codes || !scales)) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(chan_exp, 16)) return NVFP4_EALIGN;
  const bool given = flags & NVFP4_GSCALE_GIVEN;
  if (!given && (!workspace || workspace_bytes < workspace_needed() || !aligned(workspace, 4)))
    return NVFP4_EWORKSPACE;
  return run_quantize_region(x, enum_int(xdt) == NVFP4_BF16, had, make_signs(signs), given,
                             plain_map(rows, cols), f_lo, f_hi, codes, scales, global_scale,
                             workspace, (hipStream_t)stream, make_balance(chan_exp, flags));
}

nvfp4_status nvfp4_hadamard128_balanced(const void *x, nvfp4_dtype xdt, int64_t rows,
                                        const int8_t *chan_exp, uint32_t flags,
                                        const uint32_t *signs, float *y, void *stream) {
  if (enum_int(xdt) != NVFP4_BF16 || !chan_exp || (flags & ~NVFP4_PAIR_Q)) return NVFP4_EINVAL;
  if (rows < 0 || rows > kMaxBlocks / 8) return NVFP4_ESHAPE;
  if (!aligned(chan_exp, 16)) return NVFP4_EALIGN;
  if (rows == 0) return NVFP4_OK;
  if (!x || !y) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16)) return NVFP4_EALIGN;
  return hip_status(launch_hadamard((const uint16_t *)x, y, (uint32_t)rows, make_signs(signs),
                                    make_balance(chan_exp, flags), (hipStream_t)stream));
}

}  // extern "C"
