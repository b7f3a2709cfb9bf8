// nvfp4_kernels.hip -- gfx950 kernels of the NVFP4 ScaleSearch quantizer.
//
// What is computed follows the ScaleSearch summary page
// ("技術サマリー：ブロック浮動小数点スケールを検索せよ！", 手法 > ScaleSearch:
// メカニズム, 検索戦略) and the NVFP4 layout of "NVIDIAのFP4推論が50倍の効率を実現"
// (超低精度推論を支えるアーキテクチャ): E2M1 codes, one UE4M3 scale per 16
// elements, an FP32 tensor scale. Every rounding point matches the CPU oracle
// bit for bit; this file must be compiled with -ffp-contract=off so that no
// product is fused into a following add.
//
// Kernels:
//   amax      global max |x| as a max over absolute-value bit patterns
//             (exact, order-free): 16-byte coalesced loads, DPP wave reduce,
//             one partial per workgroup.
//   finalize  one workgroup: partial maxima -> tensor scale S_g.
//   quantize  one lane per 16-element block: block amax, default pattern, the
//             candidate search held in VGPRs, then 8 code bytes + 1 scale byte.
//   dequantize, sink copy, KV reassembly.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

// Input offset (in elements) of block b of the quantized region.
__device__ __forceinline__ uint64_t block_offset(const RegionMap &m, uint32_t b) {
  if (m.segments == 0) return (uint64_t)b * 16u;
  uint32_t r = fastdiv(b, m.div_bpr);
  uint32_t j = b - r * m.bpr;
  uint32_t g = fastdiv(r, m.div_tm);
  uint32_t t = r - g * m.tm;
  uint64_t row = (uint64_t)g * m.seg_tokens + m.n_first + t;
  return row * m.cols + (uint64_t)j * 16u;
}

// Source address and destination block of block b of a quantize region;
// valid is false for a row past the end of a device-length append.
struct BlockIO {
  const char *src;
  uint64_t dst;
  bool valid;
};

// t_dev: the value of *m.len_dev when the map has one (read once by the caller).
__device__ __forceinline__ BlockIO block_io(const void *x, const RegionMap &m, uint32_t b,
                                            uint32_t esize, uint32_t t_dev) {
  if (!m.append) return BlockIO{(const char *)x + block_offset(m, b) * esize, b, true};
  const uint32_t r = fastdiv(b, m.div_bpr);
  const uint32_t j = b - r * m.bpr;
  const uint32_t g = fastdiv(r, m.div_tm);
  uint32_t t_old = m.t_old, lo = m.lo;
  bool valid = true;
  if (m.len_dev) {
    t_old = t_dev;
    const uint32_t t2 = t_old + m.t_new;
    lo = max(m.n_first, t_old > m.n_last ? t_old - m.n_last : 0u);
    const uint32_t hi = max(m.n_first, t2 > m.n_last ? t2 - m.n_last : 0u);
    valid = t2 <= m.total && lo + (r - g * m.tm) < hi;
  }
  const uint32_t pos = lo + (r - g * m.tm);
  if (!valid) return BlockIO{(const char *)x, 0, false};
  uint64_t row;
  const char *base;
  if (pos < t_old) {
    const uint32_t q = fastdiv(pos, m.div_nlast);
    row = (uint64_t)g * m.n_last + (pos - q * m.n_last);
    base = (const char *)m.ring;
  } else {
    row = (uint64_t)g * m.t_new + (pos - t_old);
    base = (const char *)x;
  }
  const uint64_t dst = ((uint64_t)g * m.cap + (pos - m.n_first)) * m.bpr + j;
  return BlockIO{base + (row * m.cols + (uint64_t)j * 16u) * esize, dst, true};
}

// The device-resident token count of an append map (0 when there is none).
__device__ __forceinline__ uint32_t map_length(const RegionMap &m) {
  return m.len_dev ? (uint32_t)*m.len_dev : 0u;
}

// Wave64 max with DPP: xor-1 and xor-2 quad permutes, half-row and row
// mirrors give every lane its row-of-16 maximum; row broadcasts 15 and 31
// then fold the four rows into lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  __shared__ uint32_t red[kThreads / 64];
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  uint32_t m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = max(m, red[w]);
  return m;
}

// Load one 16-element block as FP32 (bf16 widening is exact: a 16-bit shift).
template <bool BF16>
__device__ __forceinline__ void load_block_at(const void *src, float (&v)[16]) {
  if (BF16) {
    const uint4 *p = (const uint4 *)src;
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float4 *p = (const float4 *)src;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float4 a = p[k];
      v[4 * k] = a.x;
      v[4 * k + 1] = a.y;
      v[4 * k + 2] = a.z;
      v[4 * k + 3] = a.w;
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void load_block(const void *x, uint64_t off, float (&v)[16]) {
  load_block_at<BF16>((const char *)x + off * (BF16 ? 2u : 4u), v);
}

// ---------------------------------------------------------------------------
// Global amax pass.
// ---------------------------------------------------------------------------

// Max of the absolute-value bit patterns of one 16-byte chunk.
template <bool BF16>
__device__ __forceinline__ uint32_t chunk_absmax(uint4 c) {
  if (BF16) {
    uint32_t m = 0;
    uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max((w[k] << 16) & 0x7FFFFFFFu, w[k] & 0x7FFF0000u));
    return m;
  }
  return max(max(c.x & 0x7FFFFFFFu, c.y & 0x7FFFFFFFu), max(c.z & 0x7FFFFFFFu, c.w & 0x7FFFFFFFu));
}

// Lanes take consecutive 16-byte chunks (a block is 2 chunks in bf16, 4 in
// FP32), four independent nontemporal loads in flight per lane; the grid is
// capped at 512 workgroups (fewer concurrent streams read HBM faster here).
// Balancing pair: the exponent side * e (clamped to [-32, 32]) of a signed byte.
__device__ __forceinline__ int bal_exp(uint32_t word, int byte, int side) {
  const int e = side * (int)(int8_t)(uint8_t)(word >> (8 * byte));
  return min(32, max(-32, e));
}

// Max of the absolute-value bit patterns of the scaled values x_i 2^e_i of one
// 16-byte chunk (exponent bytes in ew, one per element).
template <bool BF16>
__device__ __forceinline__ uint32_t chunk_absmax_bal(uint4 c, uint2 ew, int side) {
  uint32_t m = 0;
  if (BF16) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t eww = k < 2 ? ew.x : ew.y;
      const float lo = ldexpf(__uint_as_float(w[k] << 16), bal_exp(eww, 2 * (k & 1), side));
      const float hi = ldexpf(__uint_as_float(w[k] & 0xFFFF0000u), bal_exp(eww, 2 * (k & 1) + 1, side));
      m = max(m, max(__float_as_uint(lo) & 0x7FFFFFFFu, __float_as_uint(hi) & 0x7FFFFFFFu));
    }
  } else {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      m = max(m, __float_as_uint(ldexpf(__uint_as_float(w[k]), bal_exp(ew.x, k, side))) &
                     0x7FFFFFFFu);
  }
  return m;
}

// BAL: the values are those of the balancing pair, x 2^(side e_col) in binary32.
template <bool BF16, bool BAL>
__global__ __launch_bounds__(kThreads) void amax_kernel(AmaxArgs a) {
  constexpr uint32_t CPB = BF16 ? 2 : 4;  // 16-byte chunks per block
  constexpr uint32_t ES = BF16 ? 2 : 4;
  const uint32_t nchunks = a.map.nblocks * CPB;
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t m = 0;
  constexpr int UNROLL = 4;
  for (uint32_t c0 = blockIdx.x * kThreads + threadIdx.x; c0 < nchunks; c0 += UNROLL * stride) {
    uint4 v[UNROLL];
    uint2 ew[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      uint32_t c = c0 + u * stride;
      ew[u] = make_uint2(0, 0);
      if (c < nchunks) {
        uint32_t b = c / CPB, sub = c % CPB;
        const char *p = (const char *)a.x + block_offset(a.map, b) * ES + sub * 16u;
        v[u] = load_stream(p);
        if (BAL) {
          // exponents of the chunk's columns (8 in bf16, 4 in FP32)
          const uint32_t r = fastdiv(b, a.map.div_bpr);
          const uint32_t col = (b - r * a.map.bpr) * 16u + sub * (16u / CPB);
          ew[u] = BF16 ? *(const uint2 *)(a.bal.e + col)
                       : make_uint2(*(const uint32_t *)(a.bal.e + col), 0u);
        }
      } else {
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      m = max(m, BAL ? chunk_absmax_bal<BF16>(v[u], ew[u], a.bal.side) : chunk_absmax<BF16>(v[u]));
  }
  m = group_max_u32(m);
  if (threadIdx.x == 0) a.partials[blockIdx.x] = m;
}

// Tensor (decode) scale from the global amax bit pattern A: S_g = fl(A / 2688),
// 2688 = 6 * 448 (largest E2M1 times largest UE4M3), 1 if that is 0, NaN if
// the region holds a NaN/Inf.
__device__ __forceinline__ float tensor_scale_from_amax(uint32_t m) {
  if (m >= 0x7F800000u) return __uint_as_float(0x7FC00000u);
  const float sg = __uint_as_float(m) / 2688.0f;
  return sg == 0.0f ? 1.0f : sg;
}

__device__ __forceinline__ uint32_t reduce_partials(const uint32_t *partials, int n) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) m = max(m, partials[i]);
  return group_max_u32(m);
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(const uint32_t *partials, int n,
                                                            float *gscale) {
  const uint32_t m = reduce_partials(partials, n);
  if (threadIdx.x == 0) *gscale = tensor_scale_from_amax(m);
}

// The tensor scale for a quantize workgroup: given, or reduced here from the
// amax pass's partials (every workgroup reduces the same values in the same
// way; workgroup 0 also stores the result).
__device__ __forceinline__ float resolve_tensor_scale(const QuantArgs &a) {
  if (a.npartials == 0) return *a.gscale;
  const float sg = tensor_scale_from_amax(reduce_partials(a.partials, a.npartials));
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.gscale = sg;
  return sg;
}

// ---------------------------------------------------------------------------
// ScaleSearch quantize pass.
// ---------------------------------------------------------------------------

// Squared error of one candidate (decode scale d, encode scale r = 1/d; both 0
// for a candidate that codes everything as 0). y = x * r keeps the sign of x,
// so the hardware FP4 convert yields sign-magnitude nibbles directly (round to
// nearest even on the E2M1 grid, saturating at 6); the paired decode gives
// +-V[c]. Element pairs go through one convert each way.
__device__ __forceinline__ float candidate_sse(const float (&x)[16], float d, float r,
                                               uint32_t &c0, uint32_t &c1) {
  // all four pairs of a code word are encoded before any is decoded, so the
  // in-place converts chain without copies; each word starts from the bits of
  // its first product, a value that dies there (the four byte selects
  // overwrite all of it)
  uint32_t cw[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float y0 = x[2 * j] * r;
    const float y1 = x[2 * j + 1] * r;
    const uint32_t old = (j & 3) == 0 ? __float_as_uint(y0) : cw[j >> 2];
    cw[j >> 2] = fp4_encode_pair(old, y0, y1, j);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f32x2 v = fp4_decode_pair(cw[j >> 2], j);
    const float xh0 = v.x * d;
    const float xh1 = v.y * d;
    const float e0 = fabsf(x[2 * j]) - fabsf(xh0);
    const float e1 = fabsf(x[2 * j + 1]) - fabsf(xh1);
    const float q0 = e0 * e0;
    s = s + q0;
    const float q1 = e1 * e1;
    s = s + q1;
  }
  c0 = cw[0];
  c1 = cw[1];
  return s;
}

// Per-workgroup table of every pattern's (decode d, encode r = 1/d); a pattern
// whose r is not finite (p = 0, or 1/d overflows) stores (0, 0) so that the
// candidate codes everything as 0 through the same arithmetic.
__device__ __forceinline__ void build_scale_table(f32x2 *tbl, float sg) {
  if (threadIdx.x < 127) {
    float d = e4m3_value(threadIdx.x) * sg;
    float r = 1.0f / d;
    if (!(r < INFINITY)) {
      d = 0.0f;
      r = 0.0f;
    }
    tbl[threadIdx.x] = f32x2{d, r};
  }
  __syncthreads();
}

// The contract's squared-error term of the block's largest element a under
// candidate (d, r): fl(fl(a - fl(V d))^2), V the E2M1 value of fl(a r).
// The contract's SSE of one candidate from products y formed with its own
// encode scale (SC_LOG2 = 0) or with that of the candidate eight patterns
// below (+1: y / 2) or above (-1: y * 2); the convert's power-of-two scale
// operand applies the factor exactly before rounding.
template <int SC_LOG2>
__device__ __forceinline__ float sse_from_y(const float (&x)[16], const float (&y)[16], float d,
                                            uint32_t &c0, uint32_t &c1) {
  constexpr float sc = SC_LOG2 == 0 ? 1.0f : (SC_LOG2 > 0 ? 2.0f : 0.5f);
  uint32_t cw[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t old = (j & 3) == 0 ? 0u : cw[j >> 2];
    switch (j & 3) {
      case 0: cw[j >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y[2 * j], y[2 * j + 1], sc, 0); break;
      case 1: cw[j >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y[2 * j], y[2 * j + 1], sc, 1); break;
      case 2: cw[j >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y[2 * j], y[2 * j + 1], sc, 2); break;
      default: cw[j >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y[2 * j], y[2 * j + 1], sc, 3); break;
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f32x2 v = fp4_decode_pair(cw[j >> 2], j);
    const float xh0 = v.x * d;
    const float xh1 = v.y * d;
    const float e0 = fabsf(x[2 * j]) - fabsf(xh0);
    const float e1 = fabsf(x[2 * j + 1]) - fabsf(xh1);
    const float q0 = e0 * e0;
    s = s + q0;
    const float q1 = e1 * e1;
    s = s + q1;
  }
  c0 = cw[0];
  c1 = cw[1];
  return s;
}

__device__ __forceinline__ float amax_term(float a, float d, float r) {
  const uint32_t c = fp4_encode_pair(0u, a * r, 0.0f, 0);
  const float e = a - fp4_decode_pair(c, 0).x * d;
  return e * e;
}

// Offset of visiting slot s: slot 0 is f = 0, then FLO, FLO+1, ... without 0.
template <int FLO>
__device__ __forceinline__ constexpr int slot_offset(int s) {
  return s == 0 ? 0 : (FLO + s - 1 < 0 ? FLO + s - 1 : FLO + s);
}

// Evaluation order of the fixed-range searches: candidates in visiting order,
// each followed at once by its in-range twins eight patterns up and down,
// which reuse its products (shift +1: scale 2, -1: scale 1/2, 0: own
// products). slot_of maps an evaluation position back to the visiting slot.
template <int FLO, int FHI>
struct EvalOrder {
  static constexpr int NC = FHI - FLO + 1;
  int off[NC];
  int shift[NC];
  int slot_of[NC];
  constexpr EvalOrder() : off(), shift(), slot_of() {
    bool used[NC] = {};
    int k = 0;
    for (int sl = 0; sl < NC; ++sl) {
      const int f = slot_offset<FLO>(sl);
      if (used[f - FLO]) continue;
      const int grp[3] = {f, f + 8, f - 8};
      const int sh[3] = {0, 1, -1};
      for (int g = 0; g < 3; ++g) {
        const int h = grp[g];
        if (h < FLO || h > FHI || used[h - FLO]) continue;
        used[h - FLO] = true;
        off[k] = h;
        shift[k] = sh[g];
        slot_of[k] = h == 0 ? 0 : (h < 0 ? h - FLO + 1 : h - FLO);
        ++k;
      }
    }
  }
};

// ScaleSearch on one block held in registers: default pattern p0 from the
// block amax, then f = 0, f_lo..f_hi; first strictly smaller SSE wins.
// Writes the chosen pattern (0x7F and zero codes under the non-finite
// contract) and the two code words. A candidate's SSE is a running sum of
// non-negative terms, so it is at least its term for the block's largest
// element; a candidate whose amax term already exceeds the best SSE so far
// cannot win and is skipped when no lane of the wave needs it (exact: the
// result is unchanged).
__device__ __forceinline__ void search_block(const float (&x)[16], float sg, bool sg_ok,
                                             const f32x2 *tbl, int f_lo, int f_hi,
                                             uint32_t &best_p, uint32_t &bc0, uint32_t &bc1) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = max(am, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  best_p = 0x7Fu;
  bc0 = 0u;
  bc1 = 0u;
  if (sg_ok && am < 0x7F800000u) {
    const float amax = __uint_as_float(am);
    const float t = (amax / 6.0f) / sg;
    const uint32_t p0 = e4m3_rne_sat(t);
    f32x2 dr = tbl[p0];
    float best = candidate_sse(x, dr.x, dr.y, bc0, bc1);
    best_p = p0;
    for (int f = f_lo; f <= f_hi; ++f) {
      if (f == 0) continue;
      const int p = (int)p0 + f;
      const bool valid = (unsigned)p <= 126u;
      dr = tbl[valid ? p : (int)p0];
      const bool live = valid && !(amax_term(amax, dr.x, dr.y) > best);
      if (__ballot(live) == 0ull) continue;
      uint32_t c0, c1;
      const float s = candidate_sse(x, dr.x, dr.y, c0, c1);
      const bool win = valid && (s < best);
      best = win ? s : best;
      best_p = win ? (uint32_t)p : best_p;
      bc0 = win ? c0 : bc0;
      bc1 = win ? c1 : bc1;
    }
  }
}

// The same exact search for a fixed offset range, in the evaluation order of
// EvalOrder: a candidate eight patterns from an earlier one takes that one's
// products through the convert's power-of-two scale (exact when the table
// shows d and 1/d differing by exactly 2 between the two patterns, checked
// per lane; a wave with any lane outside that case forms its own products).
// The winner is the least SSE, ties to the earliest visiting slot, which is
// the contract's first strictly smaller SSE in visiting order.
template <int FLO, int FHI>
__device__ __forceinline__ void search_block_twins(const float (&x)[16], float sg, bool sg_ok,
                                                   const f32x2 *tbl, uint32_t &best_p,
                                                   uint32_t &bc0, uint32_t &bc1) {
  constexpr int NC = FHI - FLO + 1;
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = max(am, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  best_p = 0x7Fu;
  bc0 = 0u;
  bc1 = 0u;
  if (!(sg_ok && am < 0x7F800000u)) return;
  const float amax = __uint_as_float(am);
  const float t = (amax / 6.0f) / sg;
  const uint32_t p0 = e4m3_rne_sat(t);
  constexpr EvalOrder<FLO, FHI> ord;
  float best = INFINITY;
  int best_slot = NC;
  float y[16];
  f32x2 db = f32x2{0.0f, 0.0f};  // table entry of the current group's first candidate
  bool have_y = false;           // y holds that candidate's products (wave-uniform)
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int f = ord.off[k], sl = ord.slot_of[k], sh = ord.shift[k];
    const int p = (int)p0 + f;
    const bool valid = p >= 0 && p <= 126;
    const f32x2 dr = tbl[valid ? p : (int)p0];
    const bool live = valid && (k == 0 || !(amax_term(amax, dr.x, dr.y) > best));
    if (sh == 0) {
      db = valid ? dr : f32x2{0.0f, 0.0f};
      have_y = false;
    }
    if (__ballot(live) == 0ull) continue;
    uint32_t c0, c1;
    float sse;
    bool twin = false;
    if (sh != 0 && have_y) {
      const bool rel = sh > 0 ? (dr.x == 2.0f * db.x && dr.y == 0.5f * db.y && db.y != 0.0f)
                              : (db.x == 2.0f * dr.x && db.y == 0.5f * dr.y && dr.y != 0.0f);
      twin = __ballot(live && !rel) == 0ull;
    }
    if (twin) {
      sse = sh > 0 ? sse_from_y<1>(x, y, dr.x, c0, c1) : sse_from_y<-1>(x, y, dr.x, c0, c1);
    } else if (sh == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = x[i] * dr.y;
      have_y = true;
      sse = sse_from_y<0>(x, y, dr.x, c0, c1);
    } else {
      sse = candidate_sse(x, dr.x, dr.y, c0, c1);
    }
    const bool win = valid && (sse < best || (sse == best && sl < best_slot));
    best = win ? sse : best;
    best_slot = win ? sl : best_slot;
    best_p = win ? (uint32_t)p : best_p;
    bc0 = win ? c0 : bc0;
    bc1 = win ? c1 : bc1;
  }
}

// Balancing pair: x_i 2^(side e_i) in binary32 for the block's 16 columns.
__device__ __forceinline__ void balance_block(const Balance &bal, const RegionMap &m, uint32_t b,
                                              float (&x)[16]) {
  const uint32_t r = fastdiv(b, m.div_bpr);
  const uint4 ew = *(const uint4 *)(bal.e + (b - r * m.bpr) * 16u);
  const uint32_t w[4] = {ew.x, ew.y, ew.z, ew.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = ldexpf(x[i], bal_exp(w[i >> 2], i & 3, bal.side));
}

// Max scaling alone (offsets [0, 0]: one candidate, nothing to score) with two
// lanes per 16-element block: each lane loads 8 consecutive elements (16 B of
// bf16 or 32 B of FP32, so a wave's loads are contiguous), the pair exchanges
// its amax over DPP (a block's two lanes are always active together), and
// each lane codes its 8 elements into one 32-bit word.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void quantize_rule_kernel(QuantArgs a) {
  __shared__ f32x2 tbl[128];
  const float sg = resolve_tensor_scale(a);
  const bool sg_ok = (sg > 0.0f) && (sg < INFINITY);
  build_scale_table(tbl, sg);

  const uint32_t nunits = a.map.nblocks * 2u;
  const uint32_t stride = gridDim.x * kThreads;
  const uint32_t t_dev = map_length(a.map);
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < nunits; u += stride) {
    const uint32_t half = u & 1u;
    const BlockIO io = block_io(a.x, a.map, u >> 1, BF16 ? 2u : 4u, t_dev);
    if (!io.valid) continue;  // both lanes of the block skip together
    float x[8];
    uint32_t am = 0u;
    if (BF16) {
      const uint4 v = load_stream((const uint4 *)(io.src + 16u * half));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        am = max(am, (w[k] << 16) & 0x7FFFFFFFu);
        am = max(am, w[k] & 0x7FFF0000u);
      }
    } else {
      const uint4 *p = (const uint4 *)(io.src + 32u * half);
      const uint4 v0 = load_stream(p), v1 = load_stream(p + 1);
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[k] = __uint_as_float(w[k]);
        am = max(am, w[k] & 0x7FFFFFFFu);
      }
    }
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp((int)am, (int)am, 0xB1, 0xF, 0xF, false));
    uint32_t w = 0u, pat = 0x7Fu;
    if (sg_ok && am < 0x7F800000u) {
      pat = e4m3_rne_sat((__uint_as_float(am) / 6.0f) / sg);
      const float r = tbl[pat].y;
#pragma unroll
      for (int j = 0; j < 4; ++j) w = fp4_encode_pair(w, x[2 * j] * r, x[2 * j + 1] * r, j);
    }
    *(uint32_t *)(a.codes + io.dst * 8u + 4u * half) = w;
    if (half == 0u) a.scales[io.dst] = (uint8_t)pat;
  }
}

// ---------------------------------------------------------------------------
// Certified search for bf16 inputs.
//
// The exact search above spends ~105 VALU instructions per candidate on the
// contract's FP32 arithmetic. For bf16 blocks the winner can be established
// with less work and the same result:
//
//  * For candidate f the codes c_i (hence V_i) are computed exactly as in the
//    contract (y = fl(x * r), hardware E2M1 convert). Let a_i = |x_i|,
//    x^_i = V_i d (real product), E_f = sum (a_i - V_i d)^2 (real), and
//    A2 = sum a_i^2. Then E_f = A2 + K_f with K_f = d (d S2 - 2 S1),
//    S1 = sum a_i V_i, S2 = sum V_i^2.
//  * S1 and S2 are exact in FP32 (v_dot2_f32_bf16): V_i is a multiple of 1/2
//    up to 6; an element with V_i > 0 has y > 1/4. When the default pattern
//    is not saturated (amax / (6 S_g) <= 447, so d_0 >= amax / 6.375), a
//    candidate within 8 normal E4M3 steps below it has d >= d_0 / 2, so
//    a_i > amax / 51 > amax / 64: every nonzero product and partial sum is a
//    multiple of 2^(E-14) below 2^(E+8), E the exponent of amax (22 bits). S2
//    is a multiple of 1/4 below 577. (A caller-given S_g can saturate a
//    block's pattern; such blocks take the exact path.)
//  * K_f = 2d (d/2 S2 - S1) is formed in FP32: d/2 and 2d are exact, the
//    fused multiply-add rounds once and the multiply once, so K_f is within
//    2u |K_f| (u = 2^-24), and D_f = K_f - K_0 rounds once more. With
//    |K_0| <= A2 (E_0 <= A2 up to rounding: a nearest code is never farther
//    from the value than 0 is) and |K_f| <= A2 + |D_f|, D_f is within
//    4u A2 + 3u |D_f| of its real value.
//  * The contract's FP32 SSE differs from E_f by at most
//    delta_f <= 2u (sum x^_i^2 / 8 + 14 E_f) (u = 2^-24): per element the
//    rounding of x^, e and e^2 moves e^2 by <= 2u(V_i d |t_i| + t_i^2) to
//    first order, bounded with Cauchy-Schwarz and 2ab <= a^2/8 + 8b^2; the 15
//    sequential adds contribute <= 15u E_f. With sum x^^2 <= 2 (A2 + E_f) and
//    E_f <= |K_f - K_0| + E_0 this is at most
//    2^-23 (0.25 A2 + 14.25 E_0 + 14.25 |D_f|); adding the error of D_f
//    gives a per-candidate margin
//    M_f = 2^-18 |D_f| + 2^-23 (2.3 A2 + 15 E_0), D_f = K_f - K_0
//    (candidate 0 = offset 0 as reference), whose slack also covers the FP32
//    rounding of A2 (8 chained adds), of E_0's bound and of M_f itself.
//  * Winner w = first candidate with least D_f; U_f = D_f + M_f and
//    L_f = D_f - M_f are both increasing in D_f, so w also has the least U.
//    If every other candidate has L_f > U_w (it suffices to test the
//    runner-up in D), its SSE is certainly larger and w is the contract's
//    choice. Otherwise (near-ties, or a block outside the
//    range where the argument holds: non-normal candidate patterns, a
//    saturated default pattern, amax outside [2^-40, 2^60]) the lane
//    evaluates the contract's FP32 SSE
//    exactly for the candidates that could win and applies the visiting-order
//    rule among them.
//
// Offsets with one candidate ([0, 0], max scaling) need no search at all (the
// launcher sends them to quantize_rule_kernel; the kernel still codes them if
// instantiated so).
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x2 fp4_decode_pair_bf16(uint32_t w, int sel) {
  switch (sel & 3) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  }
}

// a . b + 0 in one VOP3P instruction (a chain start without a zeroed
// accumulator register).
__device__ __forceinline__ float dot2_first(bf16x2 a, bf16x2 b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Codes of one candidate and its exact sums S1 = sum x V, S2 = sum V^2 (x and
// V carry the same sign, so S1 = sum |x| |V|; hardware E2M1 decode to bf16,
// which is exact, and v_dot2_f32_bf16), from products y formed with the
// candidate's own encode scale (SC_LOG2 = 0) or with that of the candidate
// eight patterns below (+1) or above (-1): patterns p and p + 8 (both normal)
// have d_{p+8} = 2 d_p and r_{p+8} = r_p / 2 exactly, so y_{p+8} = y_p / 2, and
// the convert's power-of-two scale operand divides by 2^SC_LOG2 exactly before
// rounding. Each code word is converted in place over the candidate's
// previous word (all four byte selects overwrite it).
// A register whose value is never read: the first of a code word's four byte-select
// converts overwrites the byte it selects and the other three fill the rest, so
// the word needs no initial value (and no copy of an older word).
__device__ __forceinline__ uint32_t fresh_word() {
  uint32_t v;
  asm volatile("" : "=v"(v));
  return v;
}

template <int SC_LOG2, int NP>
__device__ __forceinline__ void candidate_stats_parts(const float (&y)[16],
                                                      const uint32_t (&prt)[NP][8],
                                                      uint32_t (&cw)[2], float (&s1)[NP],
                                                      float &s2) {
  constexpr float sc = SC_LOG2 == 0 ? 1.0f : (SC_LOG2 > 0 ? 2.0f : 0.5f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    switch (j & 3) {
      case 0: cw[j >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(fresh_word(), y[2 * j], y[2 * j + 1], sc, 0); break;
      case 1: cw[j >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw[j >> 2], y[2 * j], y[2 * j + 1], sc, 1); break;
      case 2: cw[j >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw[j >> 2], y[2 * j], y[2 * j + 1], sc, 2); break;
      default: cw[j >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw[j >> 2], y[2 * j], y[2 * j + 1], sc, 3); break;
    }
  }
  bf16x2 v = fp4_decode_pair_bf16(cw[0], 0);
  float a[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) a[q] = dot2_first(__builtin_bit_cast(bf16x2, prt[q][0]), v);
  float b = dot2_first(v, v);
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    v = fp4_decode_pair_bf16(cw[j >> 2], j);
#pragma unroll
    for (int q = 0; q < NP; ++q)
      a[q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, prt[q][j]), v, a[q], false);
    b = __builtin_amdgcn_fdot2_f32_bf16(v, v, b, false);
  }
#pragma unroll
  for (int q = 0; q < NP; ++q) s1[q] = a[q];
  s2 = b;
}

// Codes of a single candidate (no scoring).
__device__ __forceinline__ void candidate_codes(const float (&x)[16], float r, uint32_t &c0,
                                                uint32_t &c1) {
  uint32_t cw[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j)
    cw[j >> 2] = fp4_encode_pair(cw[j >> 2], x[2 * j] * r, x[2 * j + 1] * r, j);
  c0 = cw[0];
  c1 = cw[1];
}


// Per pattern: d / 2 and 2 d (both exact) and the encode scale r = 1/d. Rows past
// pattern 126 are zero: a candidate there codes every element to 0 and scores
// K = 0, i.e. the block's full energy, which no eligible block's leader or
// contender can reach (the offset-0 candidate already removes more than
// 0.99 amax^2 of it).
struct CertEntry {
  float hd, td, r, pad;
};
constexpr int kCertRows = 136;

// Max of |x| bit patterns of 16 bf16 values packed in 8 words (packed 16-bit max).
__device__ __forceinline__ uint32_t bf16_block_absmax_bits(const uint32_t (&w)[8]) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int k = 1; k < 8; ++k)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[k] & 0x7FFF7FFFu));
  return (uint32_t)max(m.x, m.y) << 16;
}

// The per-workgroup tables of the certified search (after build_scale_table).
__device__ __forceinline__ void build_cert_table(const f32x2 *tbl, CertEntry *ctbl) {
  if (threadIdx.x < kCertRows) {
    const f32x2 dr = threadIdx.x < 127 ? tbl[threadIdx.x] : f32x2{0.0f, 0.0f};
    ctbl[threadIdx.x] = CertEntry{0.5f * dr.x, 2.0f * dr.x, dr.y, 0.0f};
  }
}

// Default pattern in one multiply: q = fl(am * c6), c6 = 1/(6 S_g) rounded
// once, and the contract's t = fl(fl(am / 6) / S_g) are each within 2^-23
// (relative) of am / (6 S_g), so they differ by at most 4 ulps of q. RNE to
// E4M3 changes only at midpoints (low 20 bits of the binary32 pattern 0x80000
// in E4M3's normal range), so when q is more than 8 ulps from a midpoint, q and
// t give the same pattern. Otherwise (or for q in E4M3's subnormal range, or
// S_g outside [2^-100, 2^100]) t is formed as the contract does.
// On the fast path q is normal in E4M3 (>= 2^-6), where nearest-even onto the
// pattern grid is a rounding of q's binary32 pattern at bit 20 (saturating at
// 126); zero, subnormal and near-midpoint quotients take the contract's steps.
__device__ __forceinline__ uint32_t default_pattern(uint32_t am, float sg, float c6, bool c6_ok) {
  const float q = __uint_as_float(am) * c6;
  const uint32_t b = __float_as_uint(q);
  const bool near_mid = ((b - 0x80000u + 8u) & 0xFFFFFu) <= 16u;
  if (!c6_ok || near_mid || !(q >= 0x1p-6f))
    return e4m3_rne_sat((__uint_as_float(am) / 6.0f) / sg);
  return min(((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - 960u, 126u);
}

// Three-way split of a binary32 block for exact dot products with E2M1 values:
// x = h + m + l with h the top 8 significand bits of x, m the next 8 and l the
// last 8 (fixed bit positions, so m and l are multiples of 2^(e-15) and
// 2^(e-23), e the exponent of x). Each part has at most 8 significant bits and
// is exact in bf16 (its binary32 pattern has zero low half); the parts are
// packed as bf16 pairs (elements 2k, 2k+1).
__device__ __forceinline__ void split3_block(const float (&x)[16], uint32_t (&prt)[3][8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t be = __float_as_uint(x[2 * k]), bo = __float_as_uint(x[2 * k + 1]);
    const float te = __uint_as_float(be & 0xFFFFFF00u), to = __uint_as_float(bo & 0xFFFFFF00u);
    const float me = te - __uint_as_float(be & 0xFFFF0000u);
    const float mo = to - __uint_as_float(bo & 0xFFFF0000u);
    const float le = x[2 * k] - te, lo = x[2 * k + 1] - to;
    prt[0][k] = __builtin_amdgcn_perm(bo, be, 0x07060302u);
    prt[1][k] = __builtin_amdgcn_perm(__float_as_uint(mo), __float_as_uint(me), 0x07060302u);
    prt[2][k] = __builtin_amdgcn_perm(__float_as_uint(lo), __float_as_uint(le), 0x07060302u);
  }
}

// Twin codes identical: candidate patterns p and p + 8 (both normal) reconstruct
// every element alike iff E2M1(y) = 2 E2M1(y / 2) for each product y of the
// finer one, which holds iff no code of the finer candidate is +-0.5 or +-1.5
// (code magnitudes 1 and 3: bit 0 set, bit 2 clear) and its largest product is
// below 7 (7 itself codes to 6 against 2 * 4). Their contract SSEs are then
// equal bit for bit.
__device__ __forceinline__ bool twin_codes_identical(uint32_t c0, uint32_t c1, float ymax) {
  const uint32_t half = (c0 & ~(c0 >> 2)) | (c1 & ~(c1 >> 2));
  return (half & 0x11111111u) == 0u && ymax < 7.0f;
}

// The certified search of one block (bf16 values with NP = 1: parts = the bf16
// words; binary32 values with NP = 3: the three-way split), from the default
// pattern p0. Writes the winner as the exact contract would.
//
// K_f = 2d (d/2 S2 - S1): with one part the fused product d/2 S2 is exact inside
// the FMA, one rounding there and one in the multiply (K within 2u |K|). With
// three parts S1 = S1h + S1m + S1l is not a binary32 value; t = fl(fl(d/2 S2 -
// S1h) - fl(S1m + S1l)) then K = fl(2d t): S1m + S1l < 2^-7 S1, so K is within
// 3.1u (|K| + 2^-6 2d S1) <= 3.2u (A2 + |D|), and D = fl(K - K_0) within
// 6.4u A2 + 4.2u |D|; the margin's A2 coefficient is 3.6 instead of 2.3 and
// the |D| coefficient stays below 2^-18.
//
// TIES (binary32 path): a twin eight patterns above its group's first candidate
// f in [-2, 0] whose codes are identical to the finer one's (twin_codes_identical)
// has the same contract SSE and comes later in visiting order, so it can never
// be the choice; it is dropped (K = inf) instead of contesting.
// PRUNE: candidates with offset <= -4 are skipped wave-wide when no lane can
// need them: the contract SSE is at least its own amax term, and the best
// candidate's contract SSE is at most A2 + K_best + 2^-18 A2 (K error, the
// delta bound and the roundings of the bound itself).
template <int FLO, int FHI, int NP, bool RANGE_FIXED, bool TIES, bool PRUNE>
__device__ __forceinline__ void certified_search(const float (&x)[16],
                                                 const uint32_t (&prt)[NP][8], uint32_t am,
                                                 uint32_t p0, bool unsat, float a2,
                                                 const f32x2 *tbl, const CertEntry *ctbl,
                                                 int f_lo, int f_hi, uint32_t &best_p,
                                                 uint32_t &bc0, uint32_t &bc1) {
  constexpr int NC = FHI - FLO + 1;
  constexpr float kA2Coef = NP == 1 ? 2.3f : 3.6f;
  // certificate applies: every candidate pattern normal, the default pattern
  // not saturated (unsat: amax / (6 S_g) <= 447, so d_0 is within 1/16 of
  // amax / 6; a caller-given S_g can saturate blocks), amax in [2^-40, 2^60];
  // other blocks take the exact path below. Candidates above pattern 126 read
  // the zero rows of the table.
  const bool eligible =
      unsat && ((int)p0 + FLO >= 8) && am >= 0x2B800000u && am <= 0x5D800000u;
  const int p0b = max((int)p0, -FLO);  // keeps table indices >= 0
  const float amax = __uint_as_float(am);

  // Leader = candidate with the least K (first in evaluation order among
  // equal K). D = fl(K - K_0) is non-decreasing in K and the margin is
  // monotone in D, so only the runner-up's K is needed to decide whether
  // any other candidate's L = D - M reaches the leader's U; equal K, or
  // K values whose D rounds equal, contest.
  constexpr EvalOrder<FLO, FHI> ord;
  float kk[NC];  // K by visiting slot
  float k0 = 0.0f;
  float cst = 0.0f;  // block part of the margin
  float best_k = 0.0f, second_k = INFINITY;
  int best_f = 0;
  uint32_t cw[2] = {0u, 0u}, gw[2] = {0u, 0u};
  float y[16];
  float gymax = 0.0f;  // largest product of the group's first candidate
  const CertEntry *crow = ctbl + (p0b + FLO);
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int f = ord.off[k];
    const int sl = ord.slot_of[k];
    const CertEntry ce = crow[f - FLO];
    // a group's first candidate with an offset in [-2, 0] may have an identical twin
    const bool tie_group = TIES && ord.shift[k] == 0 && f >= -2 && f <= 0;
    const bool tie_twin = TIES && ord.shift[k] > 0 && f - 8 >= -2 && f - 8 <= 0;
    if (ord.shift[k] == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = x[i] * ce.r;
      if (tie_group) gymax = amax * ce.r;
    }
    if (PRUNE && k > 0 && f <= -4) {
      const float ub = (a2 + best_k) + a2 * 0x1p-18f;
      const bool live = eligible && !(amax_term(amax, 0.5f * ce.td, ce.r) > ub);
      if (__ballot(live) == 0ull) {
        kk[sl] = INFINITY;
        continue;
      }
    }
    float s1[NP], s2;
    if (ord.shift[k] == 0)
      candidate_stats_parts<0, NP>(y, prt, cw, s1, s2);
    else if (ord.shift[k] > 0)
      candidate_stats_parts<1, NP>(y, prt, cw, s1, s2);
    else
      candidate_stats_parts<-1, NP>(y, prt, cw, s1, s2);
    float kf;
    if constexpr (NP == 1)
      kf = ce.td * __builtin_fmaf(ce.hd, s2, -s1[0]);
    else
      kf = ce.td * (__builtin_fmaf(ce.hd, s2, -s1[0]) - (s1[1] + s1[2]));
    if (k == 0) {
      k0 = kf;
      // E_0 = A2 + K_0 <= A2 (nearest-value codes never do worse than 0),
      // bounded from above with K_0's own error (at most 3.2u A2)
      const float e0ub = fminf(fmaxf(kf + a2 * (1.0f + 0x1p-21f), 0.0f), a2);
      cst = (kA2Coef * a2 + 15.0f * e0ub) * (0x1p-23f * (1.0f + 0x1p-20f)) + 0x1p-120f;
    }
    if (tie_twin && twin_codes_identical(gw[0], gw[1], gymax)) kf = INFINITY;
    if (tie_group) {
      gw[0] = cw[0];
      gw[1] = cw[1];
    }
    if (!RANGE_FIXED && (f < f_lo || f > f_hi)) kf = INFINITY;
    kk[sl] = kf;
    if (k == 0) {
      best_k = kf;
      bc0 = cw[0];
      bc1 = cw[1];
    } else {
      const bool lt = kf < best_k;
      second_k = __builtin_amdgcn_fmed3f(best_k, second_k, kf);
      best_k = lt ? kf : best_k;
      best_f = lt ? f : best_f;
      bc0 = lt ? cw[0] : bc0;
      bc1 = lt ? cw[1] : bc1;
      // select here: keeps each candidate's code words from staying live to the end
      asm volatile("" : "+v"(bc0), "+v"(bc1));
    }
  }
  best_p = (uint32_t)(p0b + best_f);
  const float best_d = best_k - k0, second_d = second_k - k0;
  const float best_u = best_d + __builtin_fmaf(__builtin_fabsf(best_d), 0x1p-18f, cst);
  const bool contested =
      second_d - __builtin_fmaf(__builtin_fabsf(second_d), 0x1p-18f, cst) <= best_u;
  if (!eligible || best_p > 126u || contested) {
    // Exact contract evaluation over the candidates that could win,
    // in visiting order.
    const uint32_t lead = best_p;
    float best = INFINITY;
    bool have = false;
#pragma unroll
    for (int sl = 0; sl < NC; ++sl) {
      const int f = slot_offset<FLO>(sl);
      const int p = (int)p0 + f;
      const bool valid = (RANGE_FIXED || (f >= f_lo && f <= f_hi)) && p >= 0 && p <= 126;
      const float dsl = kk[sl] - k0;
      const float lf = dsl - __builtin_fmaf(__builtin_fabsf(dsl), 0x1p-18f, cst);
      const bool need = valid && (!eligible || (uint32_t)p == lead || lf <= best_u);
      if (need) {
        const f32x2 dr = tbl[p];
        uint32_t c0, c1;
        const float sse = candidate_sse(x, dr.x, dr.y, c0, c1);
        if (!have || sse < best) {
          have = true;
          best = sse;
          best_p = (uint32_t)p;
          bc0 = c0;
          bc1 = c1;
        }
      }
    }
  }
}

// One bf16 block (its 32 bytes as two words of four) through the certified
// search: default pattern, A2, candidates; writes the contract's choice.
template <int FLO, int FHI, bool RANGE_FIXED>
__device__ __forceinline__ void certified_block_bf16(uint4 q0, uint4 q1, float sg, bool sg_ok,
                                                     float c6, bool c6_ok, const f32x2 *tbl,
                                                     const CertEntry *ctbl, int f_lo, int f_hi,
                                                     uint32_t &best_p, uint32_t &bc0,
                                                     uint32_t &bc1) {
  constexpr int NC = FHI - FLO + 1;
  const uint32_t w[1][8] = {{q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w}};
  float x[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = __uint_as_float(w[0][k] << 16);
    x[2 * k + 1] = __uint_as_float(w[0][k] & 0xFFFF0000u);
  }
  const uint32_t am = bf16_block_absmax_bits(w[0]);
  best_p = 0x7Fu;
  bc0 = 0u;
  bc1 = 0u;
  if (!(sg_ok && am < 0x7F800000u)) return;
  const uint32_t p0 = default_pattern(am, sg, c6, c6_ok);
  if (NC == 1) {
    best_p = p0;
    candidate_codes(x, tbl[p0].y, bc0, bc1);
    return;
  }
  // A2 from the bf16 words: exact squares, eight FP32 roundings.
  float a2 = dot2_first(__builtin_bit_cast(bf16x2, w[0][0]), __builtin_bit_cast(bf16x2, w[0][0]));
#pragma unroll
  for (int k = 1; k < 8; ++k)
    a2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[0][k]),
                                         __builtin_bit_cast(bf16x2, w[0][k]), a2, false);
  const bool unsat = c6_ok && __uint_as_float(am) * c6 <= 447.0f;
  certified_search<FLO, FHI, 1, RANGE_FIXED, false, false>(x, w, am, p0, unsat, a2, tbl, ctbl,
                                                            f_lo, f_hi, best_p, bc0, bc1);
}

// RANGE_FIXED: the launch guarantees [f_lo, f_hi] == [FLO, FHI]. Up to nine
// candidates fit in 64 registers: eight waves per SIMD.
template <int FLO, int FHI, bool RANGE_FIXED>
__global__ __launch_bounds__(kThreads, (FHI - FLO + 1 <= 9) ? 8 : 1) void quantize_certified_kernel(
    QuantArgs a) {
  __shared__ f32x2 tbl[128];
  __shared__ CertEntry ctbl[kCertRows];
  const float sg = resolve_tensor_scale(a);
  const bool sg_ok = (sg > 0.0f) && (sg < INFINITY);
  build_scale_table(tbl, sg);
  build_cert_table(tbl, ctbl);
  __syncthreads();
  const float c6 = (float)(1.0 / (6.0 * (double)sg));
  const bool c6_ok = sg_ok && sg >= 0x1p-100f && sg <= 0x1p100f;

  const uint32_t stride = gridDim.x * kThreads;
  const uint32_t t_dev = map_length(a.map);
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < a.map.nblocks; b += stride) {
    const BlockIO io = block_io(a.x, a.map, b, 2u, t_dev);
    if (!io.valid) continue;
    const uint4 q0 = load_stream(io.src), q1 = load_stream(io.src + 16);
    uint32_t best_p, bc0, bc1;
    certified_block_bf16<FLO, FHI, RANGE_FIXED>(q0, q1, sg, sg_ok, c6, c6_ok, tbl, ctbl, a.f_lo,
                                                a.f_hi, best_p, bc0, bc1);
    *(uint2 *)(a.codes + io.dst * 8u) = make_uint2(bc0, bc1);
    a.scales[io.dst] = (uint8_t)best_p;
  }
}

// The certified search for binary32 blocks (the Hadamard path): the split
// makes S1 exact, A2 comes from an FMA chain (within 16u, bounded from above
// by the factor 1 + 2^-19), and blocks with a non-finite element, or whose A2
// overflows, take the exact search.
template <int FLO, int FHI>
__device__ __forceinline__ void search_block_cert32(const float (&x)[16], float sg, bool sg_ok,
                                                    float c6, bool c6_ok, const f32x2 *tbl,
                                                    const CertEntry *ctbl, uint32_t &best_p,
                                                    uint32_t &bc0, uint32_t &bc1) {
  // amax by float max of |x| (a NaN would be skipped; it makes A2 NaN, which
  // sends the block to the exact search)
  float amf = fmaxf(__builtin_fabsf(x[0]), __builtin_fabsf(x[1]));
#pragma unroll
  for (int i = 2; i < 16; ++i) amf = fmaxf(amf, __builtin_fabsf(x[i]));
  const uint32_t am = __float_as_uint(amf);
  float a2 = x[0] * x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) a2 = __builtin_fmaf(x[i], x[i], a2);
  a2 *= 1.0f + 0x1p-19f;
  if (!(sg_ok && am < 0x7F800000u && a2 < INFINITY)) {
    search_block_twins<FLO, FHI>(x, sg, sg_ok, tbl, best_p, bc0, bc1);
    return;
  }
  uint32_t prt[3][8];
  split3_block(x, prt);
  const uint32_t p0 = default_pattern(am, sg, c6, c6_ok);
  const bool unsat = c6_ok && amf * c6 <= 447.0f;
  certified_search<FLO, FHI, 3, true, true, (FLO <= -4)>(x, prt, am, p0, unsat, a2, tbl, ctbl,
                                                          FLO, FHI, best_p, bc0, bc1);
}

// Blocks first, first + stride, ... of the region. FIXED: the launch guarantees
// [f_lo, f_hi] == [FLO, FHI] (certified search on binary32 values); otherwise
// the exact search over [f_lo, f_hi].
template <bool BF16, int FLO, int FHI, bool FIXED, bool BAL = false>
__device__ __forceinline__ void quantize_blocks(const QuantArgs &a, const f32x2 *tbl, float sg,
                                                bool sg_ok, uint32_t first, uint32_t stride,
                                                uint32_t t_dev, const CertEntry *ctbl = nullptr,
                                                float c6 = 0.0f, bool c6_ok = false) {
  for (uint32_t b = first; b < a.map.nblocks; b += stride) {
    float x[16];
    const BlockIO io = block_io(a.x, a.map, b, BF16 ? 2u : 4u, t_dev);
    if (!io.valid) continue;
    load_block_at<BF16>(io.src, x);
    if (BAL) balance_block(a.bal, a.map, b, x);
    uint32_t best_p, bc0, bc1;
    if (FIXED)
      search_block_cert32<FLO, FHI>(x, sg, sg_ok, c6, c6_ok, tbl, ctbl, best_p, bc0, bc1);
    else
      search_block(x, sg, sg_ok, tbl, a.f_lo, a.f_hi, best_p, bc0, bc1);
    *(uint2 *)(a.codes + io.dst * 8u) = make_uint2(bc0, bc1);
    a.scales[io.dst] = (uint8_t)best_p;
  }
}

// BAL: the blocks are those of the balancing pair's scaled values (plain
// regions only), searched as binary32 values.
template <bool BF16, int FLO, int FHI, bool FIXED, bool BAL = false>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  __shared__ f32x2 tbl[128];
  __shared__ CertEntry ctbl[FIXED ? kCertRows : 1];
  const float sg = resolve_tensor_scale(a);
  const bool sg_ok = (sg > 0.0f) && (sg < INFINITY);
  build_scale_table(tbl, sg);
  if (FIXED) {
    build_cert_table(tbl, ctbl);
    __syncthreads();
  }
  const float c6 = (float)(1.0 / (6.0 * (double)sg));
  const bool c6_ok = sg_ok && sg >= 0x1p-100f && sg <= 0x1p100f;
  quantize_blocks<BF16, FLO, FHI, FIXED, BAL>(a, tbl, sg, sg_ok,
                                              blockIdx.x * kThreads + threadIdx.x,
                                              gridDim.x * kThreads, map_length(a.map), ctbl, c6,
                                              c6_ok);
}

// ---------------------------------------------------------------------------
// 128-point Hadamard pre-transform on MFMA (ScaleSearch summary page,
// ScaleSearchAttention, 非干渉処理（IP）と絶対値低減: Hadamard incoherence
// processing of Q and K). y = x H / sqrt(128) per contiguous 128-vector, H the
// Sylvester matrix H[j][k] = (-1)^popcount(j & k).
//
// One wave transforms 32 vectors with v_mfma_f32_32x32x16_bf16 as
// Y^T = H' X^T: B (16 x 32) is a 16-element slice of the 32 vectors straight
// from memory (lane: vector lane & 31, elements 8 (lane >> 5) .. +7 of the
// slice), A (32 x 16) is the matching slice of 32 rows of H (entries +-1,
// exact in bf16), generated in registers. The rows of H are taken in the
// order that makes accumulator v of lane l hold feature 32 t + 16 (l >> 5) + v
// of vector l & 31, i.e. one whole 16-element quantization block per lane and
// per 32-feature tile t. The products are exact; the FP32 accumulation may
// round, and the sum is scaled by the binary32 nearest 2^-3.5 (one more
// rounding), so the transform is within a few FP32 ulps of the exact one.
//
// Randomized variant (random +-1 signs before H, as in QuIP#'s incoherence
// processing): y = (x o s) H / sqrt(128). The signs flip the sign bits of the
// bf16 B operand as it is loaded, so the products stay exact and the result
// is that of the plain transform of x o s.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kInvSqrt128f = 0x1.6a09e6p-4f;  // nearest binary32 to 2^-3.5

// Feature (row of H) held by accumulator row i of tile t.
__device__ __forceinline__ uint32_t hadamard_feature(uint32_t t, uint32_t i) {
  return 32u * t + 16u * ((i >> 2) & 1u) + 4u * (i >> 3) + (i & 3u);
}

struct HadamardLane {
  uint32_t base[4];  // bf16 pairs of H[feat][8g + e] signs for e = 0..7 (feat & 7 part)
  uint32_t lo;       // features of this lane's A row without the tile part
  uint32_t g;        // lane >> 5: which 8 of each 16-element K slice
};

__device__ __forceinline__ HadamardLane hadamard_lane_setup() {
  HadamardLane h;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t i = lane & 31u;
  h.g = lane >> 5;
  h.lo = hadamard_feature(0, i);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t e0 = 2u * q, e1 = 2u * q + 1u;
    const uint32_t s0 = __builtin_popcount(h.lo & e0) & 1u;
    const uint32_t s1 = __builtin_popcount(h.lo & e1) & 1u;
    h.base[q] = (s0 ? 0xBF80u : 0x3F80u) | ((s1 ? 0xBF80u : 0x3F80u) << 16);
  }
  return h;
}

// A operand for tile t and K slice ks: the base signs times
// (-1)^popcount(feat & (16 ks + 8 g)) (the high bits of k; bits 0..2 are in base).
__device__ __forceinline__ bf16x8 hadamard_a(const HadamardLane &h, uint32_t t, uint32_t ks) {
  const uint32_t feat = 32u * t + h.lo;
  const uint32_t neg = __builtin_popcount(feat & (16u * ks + 8u * h.g)) & 1u;
  const uint32_t m = neg ? 0x80008000u : 0u;
  uint4 v = make_uint4(h.base[0] ^ m, h.base[1] ^ m, h.base[2] ^ m, h.base[3] ^ m);
  return __builtin_bit_cast(bf16x8, v);
}

// The A operand of every (tile t, K slice ks) is one of four per-lane quads: the
// sign (-1)^popcount(feat & (16 ks + 8 g)) splits into a per-lane part (feature
// bit 3 with g, feature bit 4 with bit 0 of ks) and a wave-uniform part
// popcount((ks >> 1) & t) (feature bits 5 and 6 are t), so the quads are the
// base signs times the lane part for even and odd ks, and their negations.
struct HadamardAQuads {
  uint4 q[4];  // +even, +odd, -even, -odd
};

__device__ __forceinline__ HadamardAQuads hadamard_a_quads(const HadamardLane &h) {
  const uint32_t i = threadIdx.x & 31u;
  const uint32_t c1 = h.g & ((i >> 4) & 1u), c2 = (i >> 2) & 1u;
  const uint32_t me = c1 ? 0x80008000u : 0u, mo = (c1 ^ c2) ? 0x80008000u : 0u;
  HadamardAQuads a;
  a.q[0] = make_uint4(h.base[0] ^ me, h.base[1] ^ me, h.base[2] ^ me, h.base[3] ^ me);
  a.q[1] = make_uint4(h.base[0] ^ mo, h.base[1] ^ mo, h.base[2] ^ mo, h.base[3] ^ mo);
#pragma unroll
  for (int k = 0; k < 2; ++k)
    a.q[2 + k] = make_uint4(a.q[k].x ^ 0x80008000u, a.q[k].y ^ 0x80008000u,
                            a.q[k].z ^ 0x80008000u, a.q[k].w ^ 0x80008000u);
  return a;
}

// Tile T (compile-time) of the transform from the quads.
template <int T>
__device__ __forceinline__ void hadamard_tile_q(const HadamardAQuads &a, const uint4 (&b)[8],
                                                float (&y)[16]) {
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int u = __builtin_popcount((ks >> 1) & T) & 1;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, a.q[2 * u + (ks & 1)]), __builtin_bit_cast(bf16x8, b[ks]), acc,
        0, 0, 0);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) y[v] = acc[v] * kInvSqrt128f;
}

// Balancing pair folded into the transform: y = (x diag(2^e)) H' = x (diag(2^e) H'),
// so the A operand's entry for input feature k becomes +-2^e_k (still exact in
// bf16, and every product x_k 2^e_k stays exact in FP32). ew holds, per K slice
// ks and lane half g, the bf16 exponent fields of elements 16 ks + 8 g .. +7 in
// pairs (low element in the low half): [ks][g][4] words.
__device__ __forceinline__ void build_balance_bits(const Balance &bal, uint32_t *ew) {
  if (threadIdx.x < 64) {
    const uint32_t ks = threadIdx.x >> 3, g = (threadIdx.x >> 2) & 1u, q = threadIdx.x & 3u;
    const uint32_t k0 = 16u * ks + 8u * g + 2u * q;
    const uint32_t w = *(const uint16_t *)(bal.e + k0);
    const uint32_t lo = (uint32_t)(127 + bal_exp(w, 0, bal.side)) << 7;
    const uint32_t hi = (uint32_t)(127 + bal_exp(w, 1, bal.side)) << 7;
    ew[threadIdx.x] = lo | (hi << 16);
  }
}

__device__ __forceinline__ bf16x8 hadamard_a_bal(const HadamardLane &h, uint32_t t, uint32_t ks,
                                                 const uint4 *ew4) {
  const uint32_t feat = 32u * t + h.lo;
  const uint32_t neg = __builtin_popcount(feat & (16u * ks + 8u * h.g)) & 1u;
  const uint32_t m = neg ? 0x80008000u : 0u;
  const uint4 e = ew4[2u * ks + h.g];
  uint4 v = make_uint4(((h.base[0] ^ m) & 0x80008000u) | e.x, ((h.base[1] ^ m) & 0x80008000u) | e.y,
                       ((h.base[2] ^ m) & 0x80008000u) | e.z, ((h.base[3] ^ m) & 0x80008000u) | e.w);
  return __builtin_bit_cast(bf16x8, v);
}

// bf16 sign-bit mask of elements 16 ks + 8 g .. +7 (two per word, low first).
__device__ __forceinline__ uint4 hadamard_sign_mask(const HadamardSigns &hs, int ks, uint32_t g) {
  const uint32_t bits = (hs.w[ks >> 1] >> (16u * (ks & 1) + 8u * g)) & 0xFFu;
  uint32_t m[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    m[q] = (((bits >> (2 * q)) & 1u) << 15) | (((bits >> (2 * q + 1)) & 1u) << 31);
  return make_uint4(m[0], m[1], m[2], m[3]);
}

// Load this lane's B slices of one 128-vector: elements 16 ks + 8 g .. +7,
// with the random signs applied when SIGNS.
template <bool SIGNS>
__device__ __forceinline__ void hadamard_load(const uint16_t *x, uint64_t off, bool valid,
                                              uint32_t g, const HadamardSigns &hs, uint4 (&b)[8]) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    b[ks] = valid ? *(const uint4 *)(x + off + 16u * ks + 8u * g) : make_uint4(0, 0, 0, 0);
    if (SIGNS) {
      const uint4 m = hadamard_sign_mask(hs, ks, g);
      b[ks] = make_uint4(b[ks].x ^ m.x, b[ks].y ^ m.y, b[ks].z ^ m.z, b[ks].w ^ m.w);
    }
  }
}

// Tile t of the transform: y[v] = feature 32 t + 16 g + v of this lane's vector.
// BAL: with the balancing pair's exponents (ew4, the LDS words of
// build_balance_bits) in the A operand.
template <bool BAL = false>
__device__ __forceinline__ void hadamard_tile(const HadamardLane &h, const uint4 (&b)[8], uint32_t t,
                                              float (&y)[16], const uint4 *ew4 = nullptr) {
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(BAL ? hadamard_a_bal(h, t, ks, ew4)
                                                      : hadamard_a(h, t, ks),
                                                  __builtin_bit_cast(bf16x8, b[ks]), acc, 0, 0, 0);
#pragma unroll
  for (int v = 0; v < 16; ++v) y[v] = acc[v] * kInvSqrt128f;
}

// Quantize with the Hadamard pre-transform (bf16 input, cols % 128 == 0). One
// wave per 32 vectors; each lane codes four blocks of its vector.
template <bool SIGNS, int FLO, int FHI, bool FIXED, bool BAL = false>
__global__ __launch_bounds__(kThreads, 3) void quantize_hadamard_kernel(QuantArgs a) {
  __shared__ f32x2 tbl[128];
  __shared__ CertEntry ctbl[FIXED ? kCertRows : 1];
  __shared__ __attribute__((aligned(16))) uint32_t ew[64];
  if (BAL) build_balance_bits(a.bal, ew);  // the table build below synchronizes
  const float sg = resolve_tensor_scale(a);
  const bool sg_ok = (sg > 0.0f) && (sg < INFINITY);
  build_scale_table(tbl, sg);
  // sign masks of the randomized transform, per lane half and K slice (read
  // through a volatile reference where used, so they are not held in registers)
  __shared__ uint4 smask[FIXED && SIGNS ? 2 : 1][8];
  if (FIXED) {
    build_cert_table(tbl, ctbl);
    if (SIGNS && threadIdx.x < 16) smask[threadIdx.x >> 3][threadIdx.x & 7] =
        hadamard_sign_mask(a.hs, threadIdx.x & 7, threadIdx.x >> 3);
    __syncthreads();
  }
  const float c6 = (float)(1.0 / (6.0 * (double)sg));
  const bool c6_ok = sg_ok && sg >= 0x1p-100f && sg <= 0x1p100f;

  const HadamardLane h = hadamard_lane_setup();
  const uint32_t nvec = a.map.nblocks / 8u;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  const uint32_t t_dev = map_length(a.map);
  // Each wave parks its B operand (the 32 input vectors, 8 KiB) in LDS between
  // the four tiles, so the registers it would hold are free for the search.
  __shared__ uint4 bpark[FIXED ? kThreads / 64 : 1][8][64];
  uint4(&bw)[8][64] = bpark[FIXED ? threadIdx.x >> 6 : 0];
  const HadamardAQuads aq = hadamard_a_quads(h);
  for (uint32_t tile = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); tile * 32u < nvec;
       tile += nwaves) {
    const uint32_t vec = tile * 32u + (lane & 31u);
    const bool valid = vec < nvec;
    uint4 b[8];
    const BlockIO io = block_io(a.x, a.map, valid ? vec * 8u : 0u, 2u, t_dev);
    const bool live = valid && io.valid;  // the 8 blocks of a vector share one row
    hadamard_load<SIGNS && !FIXED>((const uint16_t *)io.src, 0, live, h.g, a.hs, b);
    if (FIXED) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (SIGNS) {
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 m = *(volatile u32x4 *)&smask[SIGNS ? h.g : 0][ks];
          b[ks] = make_uint4(b[ks].x ^ m.x, b[ks].y ^ m.y, b[ks].z ^ m.z, b[ks].w ^ m.w);
        }
        bw[ks][lane] = b[ks];
      }
    }
#pragma unroll 1
    for (uint32_t t = 0; t < 4; ++t) {
      float y[16];
      if (FIXED) {
        uint4 bt[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) bt[ks] = bw[ks][lane];
        if (BAL) {
          hadamard_tile<BAL>(h, bt, t, y, (const uint4 *)ew);  // every lane takes part
        } else {
          switch (t) {
            case 0: hadamard_tile_q<0>(aq, bt, y); break;
            case 1: hadamard_tile_q<1>(aq, bt, y); break;
            case 2: hadamard_tile_q<2>(aq, bt, y); break;
            default: hadamard_tile_q<3>(aq, bt, y); break;
          }
        }
      } else {
        hadamard_tile<BAL>(h, b, t, y, (const uint4 *)ew);
      }
      if (live) {
        uint32_t best_p, bc0, bc1;
        if (FIXED)
          search_block_cert32<FLO, FHI>(y, sg, sg_ok, c6, c6_ok, tbl, ctbl, best_p, bc0, bc1);
        else
          search_block(y, sg, sg_ok, tbl, a.f_lo, a.f_hi, best_p, bc0, bc1);
        const uint64_t blk = io.dst + 2u * t + h.g;
        *(uint2 *)(a.codes + blk * 8u) = make_uint2(bc0, bc1);
        a.scales[blk] = (uint8_t)best_p;
      }
    }
  }
}

// Global amax of the transformed values.
template <bool SIGNS, bool BAL = false>
__global__ __launch_bounds__(kThreads) void amax_hadamard_kernel(AmaxArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t ew[64];
  if (BAL) {
    build_balance_bits(a.bal, ew);
    __syncthreads();
  }
  const HadamardLane h = hadamard_lane_setup();
  const uint32_t nvec = a.map.nblocks / 8u;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  uint32_t m = 0;
  // The next tile's 32 vectors are loaded while this tile is transformed, so each
  // wave keeps one tile's loads in flight through its whole loop.
  auto load_tile = [&](uint32_t tile, uint4 (&b)[8]) {
    const uint32_t vec = tile * 32u + (lane & 31u);
    const bool valid = vec < nvec;
    hadamard_load<SIGNS>((const uint16_t *)a.x, valid ? block_offset(a.map, vec * 8u) : 0, valid,
                         h.g, a.hs, b);
  };
  uint32_t tile = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  uint4 b[8];
  if (tile * 32u < nvec) load_tile(tile, b);
  for (; tile * 32u < nvec; tile += nwaves) {
    uint4 bn[8];
    const uint32_t next = tile + nwaves;
    if (next * 32u < nvec) load_tile(next, bn);
#pragma unroll 1
    for (uint32_t t = 0; t < 4; ++t) {
      float y[16];
      hadamard_tile<BAL>(h, b, t, y, (const uint4 *)ew);
#pragma unroll
      for (int v = 0; v < 16; ++v) m = max(m, __float_as_uint(y[v]) & 0x7FFFFFFFu);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) b[ks] = bn[ks];
  }
  m = group_max_u32(m);
  if (threadIdx.x == 0) a.partials[blockIdx.x] = m;
}

// The transform alone: y[nvec][128] FP32.
template <bool SIGNS, bool BAL = false>
__global__ __launch_bounds__(kThreads) void hadamard_kernel(const uint16_t *x, float *out,
                                                            uint32_t nvec, HadamardSigns hs,
                                                            Balance bal) {
  __shared__ __attribute__((aligned(16))) uint32_t ew[64];
  if (BAL) {
    build_balance_bits(bal, ew);
    __syncthreads();
  }
  const HadamardLane h = hadamard_lane_setup();
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  for (uint32_t tile = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); tile * 32u < nvec;
       tile += nwaves) {
    const uint32_t vec = tile * 32u + (lane & 31u);
    const bool valid = vec < nvec;
    uint4 b[8];
    hadamard_load<SIGNS>(x, (uint64_t)(valid ? vec : 0) * 128u, valid, h.g, hs, b);
#pragma unroll 1
    for (uint32_t t = 0; t < 4; ++t) {
      float y[16];
      hadamard_tile<BAL>(h, b, t, y, (const uint4 *)ew);
      if (valid) {
        float4 *o = (float4 *)(out + (uint64_t)vec * 128u + 32u * t + 16u * h.g);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = make_float4(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantize.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float block_decode_scale(uint32_t p, float sg) {
  const float s = p < 127u ? e4m3_value(p) : __uint_as_float(0x7FC00000u);
  return s * sg;
}

__device__ __forceinline__ void decode_block(uint2 c, float d, float (&o)[16]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = j < 4 ? c.x : c.y;
    const f32x2 v = fp4_decode_pair(w, j);
    o[2 * j] = v.x * d;
    o[2 * j + 1] = v.y * d;
  }
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_block(void *y, uint64_t off, const float (&o)[16]) {
  if (OUT_BF16) {
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      bf16x2 h = __builtin_convertvector((f32x2{o[2 * k], o[2 * k + 1]}), bf16x2);
      w[k] = __builtin_bit_cast(uint32_t, h);
    }
    uint4 *p = (uint4 *)((uint16_t *)y + off);
    p[0] = make_uint4(w[0], w[1], w[2], w[3]);
    p[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    float4 *p = (float4 *)((float *)y + off);
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = make_float4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
  }
}

// One lane writes one contiguous 16-byte output chunk (8 bf16 = half a block,
// or 4 FP32 = a quarter block), so every store instruction of a wave covers
// 1 KiB without gaps; its 4 (2) code bytes and the block's scale byte are
// read directly. Four chunks in flight per lane.
template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantArgs a) {
  constexpr uint32_t EPU = OUT_BF16 ? 8u : 4u;  // elements per chunk
  constexpr uint32_t SHIFT = OUT_BF16 ? 1u : 2u;  // log2(chunks per block)
  constexpr int UNROLL = 4;
  const float sg = *a.gscale;
  const uint32_t nunits = a.nblocks << SHIFT;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t u0 = blockIdx.x * kThreads + threadIdx.x; u0 < nunits; u0 += UNROLL * stride) {
    uint32_t cw[UNROLL];
    uint32_t sp[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const uint32_t u = u0 + k * stride;
      cw[k] = 0u;
      sp[k] = 0u;
      if (u < nunits) {
        const uint32_t b = u >> SHIFT, part = u & ((1u << SHIFT) - 1u);
        if (OUT_BF16)
          cw[k] = *(const uint32_t *)(a.codes + (uint64_t)b * 8u + part * 4u);
        else
          cw[k] = *(const uint16_t *)(a.codes + (uint64_t)b * 8u + part * 2u);
        sp[k] = a.scales[b];
      }
    }
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const uint32_t u = u0 + k * stride;
      if (u < nunits) {
        const float d = block_decode_scale(sp[k], sg);
        float o[EPU];
#pragma unroll
        for (int j = 0; j < (int)EPU / 2; ++j) {
          const f32x2 v = fp4_decode_pair(cw[k], j);
          o[2 * j] = v.x * d;
          o[2 * j + 1] = v.y * d;
        }
        if (OUT_BF16) {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            w[j] = __builtin_bit_cast(uint32_t,
                                      __builtin_convertvector((f32x2{o[2 * j], o[2 * j + 1]}), bf16x2));
          store_stream((uint16_t *)a.y + (uint64_t)u * EPU, w[0], w[1], w[2], w[3]);
        } else {
          store_stream((float *)a.y + (uint64_t)u * EPU, __float_as_uint(o[0]), __float_as_uint(o[1]),
                       __float_as_uint(o[2]), __float_as_uint(o[3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Attention-sink helpers.
// ---------------------------------------------------------------------------

// Copy the sink tokens of kv[BH][T][D] into sink[BH][NS][D], 16 bytes a lane.
__global__ __launch_bounds__(kThreads) void sink_copy_kernel(SinkArgs a, uint32_t esize) {
  const uint32_t ns = a.n_first + a.n_last;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t c = blockIdx.x * kThreads + threadIdx.x; c < a.nchunks; c += stride) {
    const uint32_t row = fastdiv(c, a.div_cpr);  // sink row: g * ns + s
    const uint32_t k = c - row * a.chunks_per_row;
    const uint32_t g = fastdiv(row, a.div_ns);
    const uint32_t s = row - g * ns;
    const uint32_t t = s < a.n_first ? s : a.T - a.n_last + (s - a.n_first);
    const uint64_t src = ((uint64_t)g * a.T + t) * a.D * esize + (uint64_t)k * 16u;
    const uint64_t dst = (uint64_t)row * a.D * esize + (uint64_t)k * 16u;
    *(uint4 *)((char *)a.dst + dst) = *(const uint4 *)((const char *)a.src + src);
  }
}

// New tokens of a KV append into the cache head or tail ring, 16 bytes a lane
// (tokens bound for the middle are coded by the quantize kernel instead).
// Destination of admit chunk c when the cache held t_old tokens before the
// append, or null when its token goes to the coded middle; src is its source.
__device__ __forceinline__ char *admit_dst(const AdmitArgs &a, uint32_t row_bytes,
                                           uint32_t t_old, uint32_t c, const char *&src) {
  const uint32_t tail_from = t_old + a.t_new - min(a.n_last, t_old + a.t_new);
  const uint32_t row = fastdiv(c, a.div_cpr);  // g * t_new + k
  const uint32_t k = c - row * a.chunks_per_row;
  const uint32_t g = fastdiv(row, a.div_tnew);
  const uint32_t pos = t_old + (row - g * a.t_new);
  src = (const char *)a.src + (uint64_t)row * row_bytes + (uint64_t)k * 16u;
  if (pos < a.n_first) return (char *)a.head + ((uint64_t)g * a.n_first + pos) * row_bytes + k * 16u;
  if (pos >= tail_from) {
    const uint32_t q = fastdiv(pos, a.div_nlast);
    return (char *)a.tail + ((uint64_t)g * a.n_last + (pos - q * a.n_last)) * row_bytes + k * 16u;
  }
  return nullptr;
}

__global__ __launch_bounds__(kThreads) void admit_kernel(AdmitArgs a, uint32_t row_bytes) {
  uint32_t t_old = a.t_old;
  if (a.len_dev) {  // device-resident length: skip an append that does not fit
    t_old = (uint32_t)*a.len_dev;
    if (t_old + a.t_new > a.total) return;
  }
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t c = blockIdx.x * kThreads + threadIdx.x; c < a.nchunks; c += stride) {
    const char *src;
    char *dst = admit_dst(a, row_bytes, t_old, c, src);
    if (dst) *(uint4 *)dst = *(const uint4 *)src;
  }
}

// The device-resident length after an append: t_old + t_new when that fits the
// cache (the append kernels ran), else unchanged (they skipped). One lane.
__global__ void advance_length_kernel(int64_t *len, uint32_t t_new, uint32_t total) {
  if (threadIdx.x == 0) {
    const int64_t t = *len;
    if (t + (int64_t)t_new <= (int64_t)total) *len = t + (int64_t)t_new;
  }
}

// A KV append small enough for one workgroup, in one launch (a decode step's
// append would otherwise be two or three launches of a few lanes each). The
// device-resident length (len, the same as c.len_dev and q.map.len_dev; null
// for a host-held one) is read once, and the admit's sources, which do not
// depend on it, are loaded at once; so is each lane's block leaving the recent
// window (at most one: nblocks <= kThreads), before the tables are built, so
// its latency overlaps theirs. After the tables' barrier every lane has its
// copy of the length, so it is advanced there; the leaving blocks are coded
// (bf16 with offsets [-2, 6]: the certified search, else the exact one); a
// barrier (the admit overwrites ring slots the coding reads); the new
// full-precision tokens are stored. The tensor scale is the caller's.
template <bool BF16>
__device__ __forceinline__ void kv_append_small(const QuantArgs &q, const AdmitArgs &c,
                                                uint32_t row_bytes, int64_t *len,
                                                f32x2 *tbl, CertEntry *ctbl) {
  constexpr uint32_t kPer = kSmallAppendChunks / kThreads;
  const uint32_t t_old = len ? (uint32_t)*len : c.t_old;
  const bool fits = !len || (uint64_t)t_old + c.t_new <= c.total;
  uint4 v[kPer];
#pragma unroll
  for (uint32_t i = 0; i < kPer; ++i) {
    const uint32_t ch = threadIdx.x + i * kThreads;
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (ch < c.nchunks) {
      const uint32_t row = fastdiv(ch, c.div_cpr);
      v[i] = *(const uint4 *)((const char *)c.src + (uint64_t)row * row_bytes +
                              (uint64_t)(ch - row * c.chunks_per_row) * 16u);
    }
  }
  const float sg = *q.gscale;
  BlockIO io{nullptr, 0, false};
  uint4 r[4] = {};  // the block's bytes: 32 (bf16) or 64 (FP32)
  if (threadIdx.x < q.map.nblocks) {
    io = block_io(q.x, q.map, threadIdx.x, BF16 ? 2u : 4u, t_old);
    if (io.valid) {
#pragma unroll
      for (int k = 0; k < (BF16 ? 2 : 4); ++k) r[k] = ((const uint4 *)io.src)[k];
    }
  }
  const bool sg_ok = (sg > 0.0f) && (sg < INFINITY);
  const bool cert = BF16 && q.f_lo == -2 && q.f_hi == 6;
  build_scale_table(tbl, sg);
  if (cert) {
    build_cert_table(tbl, ctbl);
    __syncthreads();
  }
  if (len && fits && threadIdx.x == 0) *len = (int64_t)t_old + c.t_new;
  if (io.valid) {
    uint32_t best_p, bc0, bc1;
    if (cert) {
      const float c6 = (float)(1.0 / (6.0 * (double)sg));
      const bool c6_ok = sg_ok && sg >= 0x1p-100f && sg <= 0x1p100f;
      certified_block_bf16<-2, 6, true>(r[0], r[1], sg, sg_ok, c6, c6_ok, tbl, ctbl, -2, 6,
                                        best_p, bc0, bc1);
    } else {
      float x[16];
      if (BF16) {
        const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          x[2 * k] = __uint_as_float(w[k] << 16);
          x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[4 * k] = __uint_as_float(r[k].x);
          x[4 * k + 1] = __uint_as_float(r[k].y);
          x[4 * k + 2] = __uint_as_float(r[k].z);
          x[4 * k + 3] = __uint_as_float(r[k].w);
        }
      }
      search_block(x, sg, sg_ok, tbl, q.f_lo, q.f_hi, best_p, bc0, bc1);
    }
    *(uint2 *)(q.codes + io.dst * 8u) = make_uint2(bc0, bc1);
    q.scales[io.dst] = (uint8_t)best_p;
  }
  __syncthreads();
  if (!fits) return;
#pragma unroll
  for (uint32_t i = 0; i < kPer; ++i) {
    const uint32_t ch = threadIdx.x + i * kThreads;
    if (ch < c.nchunks) {
      const char *src;
      char *dst = admit_dst(c, row_bytes, t_old, ch, src);
      if (dst) *(uint4 *)dst = v[i];
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void kv_append_small_kernel(QuantArgs q, AdmitArgs c,
                                                                   uint32_t row_bytes,
                                                                   int64_t *len) {
  __shared__ f32x2 tbl[128];
  __shared__ CertEntry ctbl[BF16 ? kCertRows : 1];
  kv_append_small<BF16>(q, c, row_bytes, len, tbl, ctbl);
}

// Two small appends in one launch, one workgroup each (the K and V caches of a
// decode step: distinct caches with their own lengths, so the workgroups share
// nothing).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void kv_append_small_pair_kernel(KvAppendPair p) {
  __shared__ f32x2 tbl[128];
  __shared__ CertEntry ctbl[BF16 ? kCertRows : 1];
  if (blockIdx.x == 0)
    kv_append_small<BF16>(p.q[0], p.c[0], p.row_bytes, p.len[0], tbl, ctbl);
  else
    kv_append_small<BF16>(p.q[1], p.c[1], p.row_bytes, p.len[1], tbl, ctbl);
}

// y[BH][T][D] from the sink tokens and the dequantized middle, one 16-element
// block a lane.
template <bool SINK_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequantize_kv_kernel(DequantKvArgs a) {
  const float sg = *a.gscale;
  const uint32_t ns = a.n_first + a.n_last;
  const uint32_t tm = a.T - ns;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t ob = blockIdx.x * kThreads + threadIdx.x; ob < a.nblocks; ob += stride) {
    const uint32_t row = fastdiv(ob, a.div_bpr);
    const uint32_t j = ob - row * a.bpr;
    const uint32_t g = fastdiv(row, a.div_T);
    const uint32_t t = row - g * a.T;
    float o[16];
    if (t < a.n_first || t >= a.T - a.n_last) {
      const uint32_t s = t < a.n_first ? t : a.n_first + (t - (a.T - a.n_last));
      const uint64_t off = ((uint64_t)g * ns + s) * (a.bpr * 16u) + (uint64_t)j * 16u;
      load_block<SINK_BF16>(a.sink, off, o);
    } else {
      const uint32_t mb = (g * tm + (t - a.n_first)) * a.bpr + j;
      const uint2 c = *(const uint2 *)(a.codes + (uint64_t)mb * 8u);
      decode_block(c, block_decode_scale(a.scales[mb], sg), o);
    }
    store_block<OUT_BF16>(a.y, (uint64_t)ob * 16u, o);
  }
}

// ---------------------------------------------------------------------------
// MXFP4 contrast format (power-of-two block scaling, set against NVFP4 on
// "NVIDIAのFP4推論が50倍の効率を実現", 超低精度推論を支えるアーキテクチャ). Read as
// the OCP Microscaling format: 32 elements share one E8M0 byte b = X + 127
// (2^X, 255 = NaN); X0 = floor(log2 amax) - 2, at least -127 (-127 for an
// all-zero block); elements are E2M1 of x * 2^-X, nearest-even, saturating.
// With a non-trivial offset range the ScaleSearch rule runs over exponents:
// X0 + f, f = 0 first, least left-to-right FP32 squared error, first strictly
// smaller wins. One lane per block; 2^X and 2^-X are exact (2^-127 is
// subnormal) and so is every reconstruction V * 2^X.
// ---------------------------------------------------------------------------

// 2^k for k in -127..127, exact.
__device__ __forceinline__ float pow2_exact(int k) {
  return k >= -126 ? __uint_as_float((uint32_t)(k + 127) << 23) : __uint_as_float(0x00400000u);
}

// Codes of the 32 signed elements at scale 2^X; returns the squared error
// when SSE (sum of fl(fl(|x| - |x^|)^2), left to right).
template <bool SSE>
__device__ __forceinline__ float mx_candidate(const float (&x)[32], int X, uint32_t (&cw)[4]) {
  const float r = pow2_exact(-X), d = pow2_exact(X);
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 8 * q + 2 * j;
      w = fp4_encode_pair(w, x[i] * r, x[i + 1] * r, j);
      if (SSE) {
        const f32x2 v = fp4_decode_pair(w, j);
        const float e0 = fabsf(x[i]) - fabsf(v.x * d);
        const float e1 = fabsf(x[i + 1]) - fabsf(v.y * d);
        const float q0 = e0 * e0;
        s = s + q0;
        const float q1 = e1 * e1;
        s = s + q1;
      }
    }
    cw[q] = w;
  }
  return s;
}

template <bool BF16, bool SEARCH>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(MxArgs a) {
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < a.nblocks; b += stride) {
    float x[32];
    uint32_t amb = 0u;
    if (BF16) {
      const uint4 *p = (const uint4 *)((const uint16_t *)a.x + (uint64_t)b * 32u);
      uint4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = load_stream(p + q);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[8 * q + 2 * k] = __uint_as_float(w[k] << 16);
          x[8 * q + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
          amb = max(amb, (w[k] << 16) & 0x7FFFFFFFu);
          amb = max(amb, w[k] & 0x7FFF0000u);
        }
      }
    } else {
      const uint4 *p = (const uint4 *)((const float *)a.x + (uint64_t)b * 32u);
      uint4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = load_stream(p + q);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[4 * q + k] = __uint_as_float(w[k]);
          amb = max(amb, w[k] & 0x7FFFFFFFu);
        }
      }
    }
    uint32_t cw[4];
    uint32_t byte;
    if (amb >= 0x7F800000u) {  // NaN or Inf in the block
      cw[0] = cw[1] = cw[2] = cw[3] = 0u;
      byte = 255u;
    } else {
      int X0 = -127;
      if (amb != 0u) {
        const int e = amb >= 0x00800000u ? (int)(amb >> 23) - 127 : (31 - (int)__clz(amb)) - 149;
        X0 = max(e - 2, -127);
      }
      int bestX = X0;
      if (SEARCH) {
        float best = mx_candidate<true>(x, X0, cw);
        for (int f = a.f_lo; f <= a.f_hi; ++f) {
          const int X = X0 + f;
          if (f == 0 || X < -127 || X > 127) continue;
          uint32_t c[4];
          const float e = mx_candidate<true>(x, X, c);
          if (e < best) {
            best = e;
            bestX = X;
            cw[0] = c[0];
            cw[1] = c[1];
            cw[2] = c[2];
            cw[3] = c[3];
          }
        }
      } else {
        mx_candidate<false>(x, X0, cw);
      }
      byte = (uint32_t)(bestX + 127);
    }
    store_stream(a.codes + (uint64_t)b * 16u, cw[0], cw[1], cw[2], cw[3]);
    a.scales[b] = (uint8_t)byte;
  }
}

// The OCP rule alone (offsets [0, 0]) with four lanes per 32-element block:
// each lane loads 8 consecutive elements (16 B of bf16 or 32 B of FP32, so a
// wave's loads are contiguous), the block amax is the maximum over the lane
// quad (DPP quad permutes; a block's four lanes are always active together),
// and each lane codes its 8 elements into one 32-bit word with the same
// arithmetic as the one-lane kernel.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void mx_rule_kernel(MxArgs a) {
  const uint32_t nunits = a.nblocks * 4u;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < nunits; u += stride) {
    float x[8];
    uint32_t amb = 0u;
    if (BF16) {
      const uint4 v = load_stream((const uint4 *)((const uint16_t *)a.x + (uint64_t)u * 8u));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        amb = max(amb, (w[k] << 16) & 0x7FFFFFFFu);
        amb = max(amb, w[k] & 0x7FFF0000u);
      }
    } else {
      const uint4 *p = (const uint4 *)((const float *)a.x + (uint64_t)u * 8u);
      const uint4 v0 = load_stream(p), v1 = load_stream(p + 1);
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[k] = __uint_as_float(w[k]);
        amb = max(amb, w[k] & 0x7FFFFFFFu);
      }
    }
    amb = max(amb, (uint32_t)__builtin_amdgcn_update_dpp((int)amb, (int)amb, 0xB1, 0xF, 0xF, false));
    amb = max(amb, (uint32_t)__builtin_amdgcn_update_dpp((int)amb, (int)amb, 0x4E, 0xF, 0xF, false));
    uint32_t w = 0u, byte = 255u;
    if (amb < 0x7F800000u) {
      int X = -127;
      if (amb != 0u) {
        const int e = amb >= 0x00800000u ? (int)(amb >> 23) - 127 : (31 - (int)__clz(amb)) - 149;
        X = max(e - 2, -127);
      }
      const float r = pow2_exact(-X);
#pragma unroll
      for (int j = 0; j < 4; ++j) w = fp4_encode_pair(w, x[2 * j] * r, x[2 * j + 1] * r, j);
      byte = (uint32_t)(X + 127);
    }
    *(uint32_t *)(a.codes + (uint64_t)u * 4u) = w;
    if ((u & 3u) == 0u) a.scales[u >> 2] = (uint8_t)byte;
  }
}

// One lane per 16-byte output chunk (8 bf16 or 4 FP32), as the NVFP4 inverse.
template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void mx_dequantize_kernel(MxDequantArgs a) {
  constexpr uint32_t EPU = OUT_BF16 ? 8u : 4u;
  constexpr uint32_t SHIFT = OUT_BF16 ? 2u : 3u;  // log2(chunks per 32-element block)
  constexpr int UNROLL = 4;
  const uint32_t nunits = a.nblocks << SHIFT;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t u0 = blockIdx.x * kThreads + threadIdx.x; u0 < nunits; u0 += UNROLL * stride) {
    uint32_t cw[UNROLL];
    uint32_t sb[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const uint32_t u = u0 + k * stride;
      cw[k] = 0u;
      sb[k] = 0u;
      if (u < nunits) {
        const uint32_t b = u >> SHIFT, part = u & ((1u << SHIFT) - 1u);
        if (OUT_BF16)
          cw[k] = *(const uint32_t *)(a.codes + (uint64_t)b * 16u + part * 4u);
        else
          cw[k] = *(const uint16_t *)(a.codes + (uint64_t)b * 16u + part * 2u);
        sb[k] = a.scales[b];
      }
    }
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const uint32_t u = u0 + k * stride;
      if (u < nunits) {
        const float d = sb[k] == 255u ? __uint_as_float(0x7FC00000u) : pow2_exact((int)sb[k] - 127);
        float o[EPU];
#pragma unroll
        for (int j = 0; j < (int)EPU / 2; ++j) {
          const f32x2 v = fp4_decode_pair(cw[k], j);
          o[2 * j] = v.x * d;
          o[2 * j + 1] = v.y * d;
        }
        if (OUT_BF16) {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            w[j] = __builtin_bit_cast(uint32_t,
                                      __builtin_convertvector((f32x2{o[2 * j], o[2 * j + 1]}), bf16x2));
          store_stream((uint16_t *)a.y + (uint64_t)u * EPU, w[0], w[1], w[2], w[3]);
        } else {
          store_stream((float *)a.y + (uint64_t)u * EPU, __float_as_uint(o[0]), __float_as_uint(o[1]),
                       __float_as_uint(o[2]), __float_as_uint(o[3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
// Balancing pair calibration (ScaleSearch summary page, ScaleSearchAttention,
// 非干渉処理（IP）と絶対値低減: an additional pair Q' = Q R^-T, K' = K R that keeps
// the scores and lowers the mean-square magnitude). R = diag(2^e); channel j's
// share of ||Q'||^2 + ||K'||^2 is a^2 4^-e + b^2 4^e with a^2, b^2 its sums of
// squares in Q and K; e_j is the least e in [-16, 16] with a^2 <= b^2 4^(2e+1)
// (16 if none), 0 when a or b is 0.
// ---------------------------------------------------------------------------

// Workgroup g sums rows [g R / G, (g + 1) R / G): a lane owns 8 consecutive
// columns (one 16- or 32-byte load per row), cols / 8 lanes cover a row, the
// workgroup's lanes take kThreads / (cols / 8) rows at a time; double sums,
// then the lanes of one column group add their sums in a fixed order.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void colsumsq_kernel(ColSumArgs a) {
  __shared__ double red[kThreads][8];
  const uint32_t tpr = a.cols / 8u;
  const uint32_t rpi = kThreads / tpr;
  const uint32_t cg = threadIdx.x % tpr, rsub = threadIdx.x / tpr;
  const uint32_t r0 = (uint32_t)((uint64_t)a.rows * blockIdx.x / gridDim.x);
  const uint32_t r1 = (uint32_t)((uint64_t)a.rows * (blockIdx.x + 1) / gridDim.x);
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (rsub < rpi) {
    for (uint32_t r = r0 + rsub; r < r1; r += rpi) {
      float v[8];
      if (BF16) {
        const uint4 c = load_stream((const char *)a.x + ((uint64_t)r * a.cols + 8u * cg) * 2u);
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[2 * k] = __uint_as_float(w[k] << 16);
          v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      } else {
        const char *p = (const char *)a.x + ((uint64_t)r * a.cols + 8u * cg) * 4u;
        const uint4 c0 = load_stream(p), c1 = load_stream(p + 16);
        const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(w[k]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) s[k] += (double)v[k] * (double)v[k];
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[threadIdx.x][k] = s[k];
  __syncthreads();
  if (threadIdx.x < tpr) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      double t = 0.0;
      for (uint32_t i = 0; i < rpi; ++i) t += red[i * tpr + threadIdx.x][k];
      a.part[(uint64_t)blockIdx.x * a.cols + 8u * threadIdx.x + k] = t;
    }
  }
}

__device__ __forceinline__ int balance_exponent(double a2, double b2) {
  if (!(a2 > 0.0) || !(b2 > 0.0)) return 0;
  for (int e = -16; e <= 15; ++e)
    if (a2 <= ldexp(b2, 2 * (2 * e + 1))) return e;
  return 16;
}

// One workgroup: each channel's partial sums in workgroup order, then its exponent.
__global__ __launch_bounds__(kThreads) void balance_exponents_kernel(const double *qpart,
                                                                     const double *kpart,
                                                                     uint32_t cols, int8_t *e) {
  for (uint32_t j = threadIdx.x; j < cols; j += kThreads) {
    double a2 = 0.0, b2 = 0.0;
    for (int g = 0; g < kColSumGroups; ++g) {
      a2 += qpart[(uint64_t)g * cols + j];
      b2 += kpart[(uint64_t)g * cols + j];
    }
    e[j] = (int8_t)balance_exponent(a2, b2);
  }
}

// ---------------------------------------------------------------------------

static int grid_for(uint64_t items, int cap) {
  uint64_t g = (items + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  return (int)(g > (uint64_t)cap ? cap : g);
}

hipError_t launch_amax(const AmaxArgs &a, bool bf16, int groups, hipStream_t s) {
  const bool bal = a.bal.e != nullptr;
  if (bf16 && bal)
    hipLaunchKernelGGL((amax_kernel<true, true>), dim3(groups), dim3(kThreads), 0, s, a);
  else if (bf16)
    hipLaunchKernelGGL((amax_kernel<true, false>), dim3(groups), dim3(kThreads), 0, s, a);
  else if (bal)
    hipLaunchKernelGGL((amax_kernel<false, true>), dim3(groups), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((amax_kernel<false, false>), dim3(groups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const uint32_t *partials, int n, float *gscale, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kThreads), 0, s, partials, n, gscale);
  return hipGetLastError();
}

// The balancing pair's plain quantize: the exact search on the scaled binary32
// values (the certified search needs bf16 values).
static hipError_t launch_quantize_balanced(const QuantArgs &a, bool bf16, int g, hipStream_t s) {
  const int range = (a.f_lo == -2 && a.f_hi == 6) ? 1 : (a.f_lo == -8 && a.f_hi == 8) ? 2 : 0;
  if (bf16) {
    if (range == 1)
      hipLaunchKernelGGL((quantize_kernel<true, -2, 6, true, true>), dim3(g), dim3(kThreads), 0, s, a);
    else if (range == 2)
      hipLaunchKernelGGL((quantize_kernel<true, -8, 8, true, true>), dim3(g), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((quantize_kernel<true, 0, 0, false, true>), dim3(g), dim3(kThreads), 0, s, a);
  } else {
    if (range == 1)
      hipLaunchKernelGGL((quantize_kernel<false, -2, 6, true, true>), dim3(g), dim3(kThreads), 0, s, a);
    else if (range == 2)
      hipLaunchKernelGGL((quantize_kernel<false, -8, 8, true, true>), dim3(g), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((quantize_kernel<false, 0, 0, false, true>), dim3(g), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

// Grid cap of the max-scaling rule kernels (NVFP4 and MXFP4): on the 8192 x 28672
// bf16 tensor 2048 workgroups beat 8192 by 4% (106.1 -> 102.1 us; MXFP4 102.1 -> 98.1 us),
// while 1024 and 512 lose (121.6 and 195.7 us).
constexpr int kRuleGroups = 2048;

hipError_t launch_quantize(const QuantArgs &a, bool bf16, hipStream_t s) {
  const int g = grid_for(a.map.nblocks, kMaxQuantGroups);
  const int gc = grid_for(a.map.nblocks, kMaxCertGroups);
  if (a.bal.e) return launch_quantize_balanced(a, bf16, g, s);
  if (a.f_lo == 0 && a.f_hi == 0) {
    const int gr = grid_for((uint64_t)a.map.nblocks * 2u, kRuleGroups);
    if (bf16)
      hipLaunchKernelGGL(quantize_rule_kernel<true>, dim3(gr), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(quantize_rule_kernel<false>, dim3(gr), dim3(kThreads), 0, s, a);
  } else if (bf16 && a.f_lo == -2 && a.f_hi == 6)
    hipLaunchKernelGGL((quantize_certified_kernel<-2, 6, true>), dim3(gc), dim3(kThreads), 0, s, a);
  else if (bf16 && a.f_lo == -8 && a.f_hi == 8)
    hipLaunchKernelGGL((quantize_certified_kernel<-8, 8, true>), dim3(gc), dim3(kThreads), 0, s, a);
  else if (bf16 && a.f_lo >= -8 && a.f_hi <= 8)
    hipLaunchKernelGGL((quantize_certified_kernel<-8, 8, false>), dim3(gc), dim3(kThreads), 0, s, a);
  else if (bf16)
    hipLaunchKernelGGL((quantize_kernel<true, 0, 0, false>), dim3(g), dim3(kThreads), 0, s, a);
  else if (a.f_lo == -2 && a.f_hi == 6)
    hipLaunchKernelGGL((quantize_kernel<false, -2, 6, true>), dim3(g), dim3(kThreads), 0, s, a);
  else if (a.f_lo == -8 && a.f_hi == 8)
    hipLaunchKernelGGL((quantize_kernel<false, -8, 8, true>), dim3(g), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<false, 0, 0, false>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

static int hadamard_groups(uint32_t nvec, int cap) {
  const uint64_t tiles = (nvec + 31u) / 32u;
  uint64_t g = (tiles + (kThreads / 64) - 1) / (kThreads / 64);
  if (g < 1) g = 1;
  return (int)(g > (uint64_t)cap ? cap : g);
}

int amax_hadamard_groups(uint32_t nblocks) { return hadamard_groups(nblocks / 8u, kMaxAmaxGroups); }

hipError_t launch_amax_hadamard(const AmaxArgs &a, int groups, hipStream_t s) {
  const bool bal = a.bal.e != nullptr;
  if (a.hs.on && bal)
    hipLaunchKernelGGL((amax_hadamard_kernel<true, true>), dim3(groups), dim3(kThreads), 0, s, a);
  else if (a.hs.on)
    hipLaunchKernelGGL((amax_hadamard_kernel<true, false>), dim3(groups), dim3(kThreads), 0, s, a);
  else if (bal)
    hipLaunchKernelGGL((amax_hadamard_kernel<false, true>), dim3(groups), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((amax_hadamard_kernel<false, false>), dim3(groups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// The balancing pair before the transform (the exponents ride in the A operand).
template <bool SIGNS>
static void launch_quantize_hadamard_bal(const QuantArgs &a, int g, int range, hipStream_t s) {
  if (range == 1)
    hipLaunchKernelGGL((quantize_hadamard_kernel<SIGNS, -2, 6, true, true>), dim3(g), dim3(kThreads), 0, s, a);
  else if (range == 2)
    hipLaunchKernelGGL((quantize_hadamard_kernel<SIGNS, -8, 8, true, true>), dim3(g), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_hadamard_kernel<SIGNS, 0, 0, false, true>), dim3(g), dim3(kThreads), 0, s, a);
}

hipError_t launch_quantize_hadamard(const QuantArgs &a, hipStream_t s) {
  const int g = hadamard_groups(a.map.nblocks / 8u, kMaxQuantGroups);
  const int range = (a.f_lo == -2 && a.f_hi == 6) ? 1 : (a.f_lo == -8 && a.f_hi == 8) ? 2 : 0;
  if (a.bal.e) {
    if (a.hs.on)
      launch_quantize_hadamard_bal<true>(a, g, range, s);
    else
      launch_quantize_hadamard_bal<false>(a, g, range, s);
    return hipGetLastError();
  }
  if (a.hs.on) {
    if (range == 1)
      hipLaunchKernelGGL((quantize_hadamard_kernel<true, -2, 6, true>), dim3(g), dim3(kThreads), 0, s, a);
    else if (range == 2)
      hipLaunchKernelGGL((quantize_hadamard_kernel<true, -8, 8, true>), dim3(g), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((quantize_hadamard_kernel<true, 0, 0, false>), dim3(g), dim3(kThreads), 0, s, a);
  } else {
    if (range == 1)
      hipLaunchKernelGGL((quantize_hadamard_kernel<false, -2, 6, true>), dim3(g), dim3(kThreads), 0, s, a);
    else if (range == 2)
      hipLaunchKernelGGL((quantize_hadamard_kernel<false, -8, 8, true>), dim3(g), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((quantize_hadamard_kernel<false, 0, 0, false>), dim3(g), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_hadamard(const uint16_t *x, float *y, uint32_t nvec, const HadamardSigns &hs,
                           const Balance &bal, hipStream_t s) {
  const int g = hadamard_groups(nvec, kMaxQuantGroups);
  if (hs.on && bal.e)
    hipLaunchKernelGGL((hadamard_kernel<true, true>), dim3(g), dim3(kThreads), 0, s, x, y, nvec, hs, bal);
  else if (hs.on)
    hipLaunchKernelGGL((hadamard_kernel<true, false>), dim3(g), dim3(kThreads), 0, s, x, y, nvec, hs, bal);
  else if (bal.e)
    hipLaunchKernelGGL((hadamard_kernel<false, true>), dim3(g), dim3(kThreads), 0, s, x, y, nvec, hs, bal);
  else
    hipLaunchKernelGGL((hadamard_kernel<false, false>), dim3(g), dim3(kThreads), 0, s, x, y, nvec, hs, bal);
  return hipGetLastError();
}

hipError_t launch_colsumsq(const ColSumArgs &a, bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(colsumsq_kernel<true>, dim3(kColSumGroups), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(colsumsq_kernel<false>, dim3(kColSumGroups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_balance_exponents(const double *qpart, const double *kpart, uint32_t cols,
                                    int8_t *e, hipStream_t s) {
  hipLaunchKernelGGL(balance_exponents_kernel, dim3(1), dim3(kThreads), 0, s, qpart, kpart, cols, e);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const MxArgs &a, bool bf16, hipStream_t s) {
  const int g = grid_for(a.nblocks, kMaxQuantGroups);
  const bool search = a.f_lo != 0 || a.f_hi != 0;
  if (!search) {
    const int gr = grid_for((uint64_t)a.nblocks * 4u, kRuleGroups);
    if (bf16)
      hipLaunchKernelGGL(mx_rule_kernel<true>, dim3(gr), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(mx_rule_kernel<false>, dim3(gr), dim3(kThreads), 0, s, a);
  } else if (bf16) {
    hipLaunchKernelGGL((mx_quantize_kernel<true, true>), dim3(g), dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((mx_quantize_kernel<false, true>), dim3(g), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const MxDequantArgs &a, bool out_bf16, hipStream_t s) {
  const uint64_t units = (uint64_t)a.nblocks << (out_bf16 ? 2 : 3);
  const int g = grid_for(units / 4u, kMaxStreamGroups);  // four chunks in flight per lane
  if (out_bf16)
    hipLaunchKernelGGL(mx_dequantize_kernel<true>, dim3(g), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(mx_dequantize_kernel<false>, dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, bool out_bf16, hipStream_t s) {
  const int g = grid_for((uint64_t)a.nblocks * (out_bf16 ? 2u : 4u) / 4u, kMaxStreamGroups);
  if (out_bf16)
    hipLaunchKernelGGL(dequantize_kernel<true>, dim3(g), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(dequantize_kernel<false>, dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sink_copy(const SinkArgs &a, bool bf16, hipStream_t s) {
  const int g = grid_for(a.nchunks, kMaxQuantGroups);
  hipLaunchKernelGGL(sink_copy_kernel, dim3(g), dim3(kThreads), 0, s, a, bf16 ? 2u : 4u);
  return hipGetLastError();
}

hipError_t launch_advance_length(int64_t *len, uint32_t t_new, uint32_t total, hipStream_t s) {
  hipLaunchKernelGGL(advance_length_kernel, dim3(1), dim3(64), 0, s, len, t_new, total);
  return hipGetLastError();
}

hipError_t launch_kv_append_small(const QuantArgs &q, const AdmitArgs &c, int64_t *len,
                                  bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((kv_append_small_kernel<true>), dim3(1), dim3(kThreads), 0, s, q, c,
                       c.chunks_per_row * 16u, len);
  else
    hipLaunchKernelGGL((kv_append_small_kernel<false>), dim3(1), dim3(kThreads), 0, s, q, c,
                       c.chunks_per_row * 16u, len);
  return hipGetLastError();
}

hipError_t launch_kv_append_small_pair(const KvAppendPair &p, bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((kv_append_small_pair_kernel<true>), dim3(2), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((kv_append_small_pair_kernel<false>), dim3(2), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_admit(const AdmitArgs &a, bool bf16, hipStream_t s) {
  const int g = grid_for(a.nchunks, kMaxQuantGroups);
  hipLaunchKernelGGL(admit_kernel, dim3(g), dim3(kThreads), 0, s, a, a.chunks_per_row * 16u);
  return hipGetLastError();
}

// Grid cap of the sink-mode dequantize: on the bf16 K cache [1, 8, 32768, 128] (128 + 128
// kept) 2048 workgroups take 15.4 us against 16.3 us at 8192 (512: 16.2, 4096: 15.7).
constexpr int kKvDequantGroups = 2048;

hipError_t launch_dequantize_kv(const DequantKvArgs &a, bool sink_bf16, bool out_bf16,
                                hipStream_t s) {
  const int g = grid_for(a.nblocks, kKvDequantGroups);
  if (sink_bf16 && out_bf16)
    hipLaunchKernelGGL((dequantize_kv_kernel<true, true>), dim3(g), dim3(kThreads), 0, s, a);
  else if (sink_bf16)
    hipLaunchKernelGGL((dequantize_kv_kernel<true, false>), dim3(g), dim3(kThreads), 0, s, a);
  else if (out_bf16)
    hipLaunchKernelGGL((dequantize_kv_kernel<false, true>), dim3(g), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((dequantize_kv_kernel<false, false>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace nvfp4
