// nvfp4_attention.hip -- attention whose QK^T and PV products take NVFP4
// operands (ScaleSearch summary page, ScaleSearchAttention: both products on
// NVFP4 data with FP32 accumulation; Q and K prepared by incoherence
// processing, K and V from the sink-aware cache).
//
// gfx950's scaled MFMAs take power-of-two (E8M0) block scales only, so the
// E4M3 block scales cannot ride inside the matrix instruction. Instead every
// operand element V[code] * s_block is formed exactly in fp16 (a 2-bit by
// 4-bit significand product between 2^-10 and 2688: always a normal fp16),
// two at a time by the hardware FP4 -> fp16 convert and a packed fp16
// multiply; the products run on v_mfma_f32_32x32x16_f16 with FP32
// accumulation, and the tensor scales multiply the FP32 results.
//
// Per workgroup: 128 queries of one head (4 waves x 32), looping over chunks
// of 64 keys, each decoded once into LDS (K row-major, V transposed with its
// key columns swizzled against bank conflicts) and consumed as two tiles of
// 32 keys. A wave
// computes S^T = K Q^T, so each lane holds 16 keys of one query (its lane-pair
// partner the other 16): the softmax statistics of a query live in one lane
// pair. Online softmax in base 2 (log2 e folded into the score scale); P is
// coded to NVFP4 per 16 keys by max scaling under the fixed tensor scale
// fl(1/2688) and decoded again to exact fp16 values, and O^T += V^T P^T keeps
// each query's 128 outputs in its lane pair, so the rescale by
// exp(m - m') is a per-lane multiply. The K index of both PV operands runs
// over the keys in the order the S^T accumulator holds them.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kAttnD = 128;
constexpr uint32_t kKeyTile = 32;                // softmax / P-coding tile
constexpr uint32_t kChunk = 2 * kKeyTile;        // keys decoded into LDS per barrier
constexpr uint32_t kAttnWaves = 4;
constexpr uint32_t kQueriesPerGroup = 32 * kAttnWaves;
constexpr uint32_t kKsStride = kAttnD + 8;     // fp16 per K row in LDS (16-byte pad)
constexpr uint32_t kVtStride = kChunk + 4;     // fp16 per V^T row in LDS (34 dwords)

// UE4M3 scale byte -> value, NaN for bytes 127..255. Below 127 the byte is also
// an OCP E4M3 bit pattern with the sign clear, and that format gives it the same
// value, 2^(e-7)(1 + m/8), or m 2^-9 at e = 0: gfx950's FP8 convert returns it
// (nvfp4_hw_self_check compares every such byte on the device).
__device__ __forceinline__ float scale_value(uint32_t p) {
  return p >= 127u ? NAN : __builtin_amdgcn_cvt_f32_fp8((int)p, 0);
}

// P's scale tables under S_P = fl(1/2688), evaluated by the compiler in IEEE
// binary32 (round to nearest even: the rounding of the device's own float
// multiply and correctly rounded divide), so a workgroup copies them instead
// of deriving them. For pattern k: s[k] its value, r[k] = fl(1/fl(s * S_P))
// (0 where that is not finite: everything codes as 0), and thr[k] the least
// binary32 a with E4M3(fl(fl(a / 6) / S_P)) >= k. That pattern is
// non-decreasing in a, so thr is found by bisection over the bit patterns of
// a in [0, 1] (p <= 1 puts every block amax there); thr[0] = 0, thr[127] = inf.
struct PTables {
  float s[128], r[128], thr[128];
};

constexpr float ce_e4m3_value(uint32_t p) {
  const uint32_t e = p >> 3, m = p & 7u;
  return e == 0 ? (float)m * 0x1p-9f : __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
}

// e4m3_rne_sat for the compiler: the same steps, with the subnormal rounding
// (t * 2^9 < 8, exact) done by hand.
constexpr uint32_t ce_e4m3_rne_sat(float t) {
  if (t >= 448.0f) return 126u;
  if (t < 0x1p-6f) {
    const float x = t * 512.0f;
    const uint32_t i = (uint32_t)x;
    const float f = x - (float)i;
    return f > 0.5f || (f == 0.5f && (i & 1u)) ? i + 1u : i;
  }
  const uint32_t b = __builtin_bit_cast(uint32_t, t);
  return ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - 960u;
}

constexpr PTables make_ptables() {
  PTables t{};
  const float SP = 1.0f / 2688.0f;
  for (uint32_t k = 0; k < 128; ++k) {
    t.s[k] = k < 127u ? ce_e4m3_value(k) : 0.0f;
    t.r[k] = t.s[k] > 0.0f ? 1.0f / (t.s[k] * SP) : 0.0f;
    if (k == 0u) {
      t.thr[k] = 0.0f;
    } else if (k == 127u) {
      t.thr[k] = __builtin_inff();
    } else {
      uint32_t lo = 0u, hi = 0x3F800000u;
      while (lo < hi) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if (ce_e4m3_rne_sat((__builtin_bit_cast(float, mid) / 6.0f) / SP) >= k)
          hi = mid;
        else
          lo = mid + 1u;
      }
      t.thr[k] = __builtin_bit_cast(float, lo);
    }
  }
  return t;
}

__constant__ PTables kPTables = make_ptables();

// UE4M3 scale byte -> its value in fp16 bits (exact: at most 4 significant bits
// between 2^-9 and 448), NaN for bytes 127..255, evaluated by the compiler. The
// decode kernel looks its block scales up here instead of forming them.
struct ScaleF16Table {
  uint16_t v[256];
};

constexpr ScaleF16Table make_scale_f16_table() {
  ScaleF16Table t{};
  for (uint32_t p = 0; p < 256u; ++p)
    t.v[p] = p < 127u ? __builtin_bit_cast(uint16_t, (_Float16)ce_e4m3_value(p)) : (uint16_t)0x7E00u;
  return t;
}

__constant__ ScaleF16Table kScaleF16 = make_scale_f16_table();

// Two codes of byte sel of w as fp16 (the byte selector must be a constant).
__device__ __forceinline__ f16x2 fp4_pair_f16(uint32_t w, int sel) {
  switch (sel & 3) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// Eight codes of one 32-bit word (element 2j in the low nibble of byte j)
// times the block scale s, as fp16 (exact: at most 6 significant bits).
__device__ __forceinline__ f16x8 decode8(uint32_t w, float s) {
  const _Float16 sh = (_Float16)s;  // E4M3 values are exact in fp16
  const f16x2 s2 = {sh, sh};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 v = fp4_pair_f16(w, j) * s2;
    r[2 * j] = v.x;
    r[2 * j + 1] = v.y;
  }
  return r;
}

// decode8 with the scale given as fp16 bits.
__device__ __forceinline__ f16x8 decode8_h(uint32_t w, uint16_t sbits) {
  const _Float16 sh = __builtin_bit_cast(_Float16, sbits);
  const f16x2 s2 = {sh, sh};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 v = fp4_pair_f16(w, j) * s2;
    r[2 * j] = v.x;
    r[2 * j + 1] = v.y;
  }
  return r;
}

// One chunk's raw K and V codes and scales as this thread loads them from
// memory: key tid >> 2 of the chunk, elements 32 c .. 32 c + 31, c = tid & 3.
struct TileRegs {
  uint4 kw, vw;
  uint32_t ksb, vsb;  // two scale bytes each
};

__device__ __forceinline__ TileRegs load_chunk(const AttnArgs &a, uint64_t row_base,
                                               uint32_t row_off, uint32_t c0, uint32_t hi,
                                               uint32_t tid) {
  TileRegs r{make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u), 0u, 0u};
  const uint32_t key = tid >> 2, c = tid & 3u, j = c0 + key;
  if (j < hi) {
    const uint64_t row = row_base + (j - row_off);
    r.kw = *(const uint4 *)(a.kc + row * 64u + 16u * c);
    r.vw = *(const uint4 *)(a.vc + row * 64u + 16u * c);
    r.ksb = *(const uint16_t *)(a.ks + row * 8u + 2u * c);
    r.vsb = *(const uint16_t *)(a.vs + row * 8u + 2u * c);
  }
  return r;
}

// Decode a loaded chunk into LDS: K row-major [key][d]; V transposed [d][key]
// with the key column XOR-ed with 16 (d >> 5), which spreads the four lanes
// that share a key over different banks and keeps 4-key groups contiguous.
// Keys past the segment end were loaded as zero codes and scale bytes, so
// they decode to zeros.
__device__ __forceinline__ void store_chunk(const TileRegs &r, uint32_t tid, _Float16 *Ks,
                                            _Float16 *Vt) {
  const uint32_t key = tid >> 2, c = tid & 3u;
  const float k0 = scale_value(r.ksb & 0xFFu);
  const float k1 = scale_value((r.ksb >> 8) & 0xFFu);
  _Float16 *kd = &Ks[key * kKsStride + 32u * c];
  *(f16x8 *)(kd) = decode8(r.kw.x, k0);
  *(f16x8 *)(kd + 8) = decode8(r.kw.y, k0);
  *(f16x8 *)(kd + 16) = decode8(r.kw.z, k1);
  *(f16x8 *)(kd + 24) = decode8(r.kw.w, k1);
  const float v0 = scale_value(r.vsb & 0xFFu);
  const float v1 = scale_value((r.vsb >> 8) & 0xFFu);
  const f16x8 x[4] = {decode8(r.vw.x, v0), decode8(r.vw.y, v0), decode8(r.vw.z, v1),
                      decode8(r.vw.w, v1)};
  const uint32_t pk = key ^ (16u * c);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) Vt[(32u * c + 8u * i + e) * kVtStride + pk] = x[i][e];
}

// A chunk of sink keys (bf16 rows of the cache head, or of the tail ring at
// slot t mod n_last) copied into LDS as bf16 bits in the same layouts; keys
// past the segment end are zeros. Loaded directly: sink chunks are few.
__device__ __forceinline__ void store_sink_chunk(const AttnArgs &a, uint32_t kvh, bool head,
                                                 uint32_t c0, uint32_t hi, uint32_t tid,
                                                 _Float16 *Ks, _Float16 *Vt) {
  const uint32_t key = tid >> 2, c = tid & 3u, j = c0 + key;
  uint4 kq[4], vq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kq[i] = vq[i] = make_uint4(0u, 0u, 0u, 0u);
  if (j < hi) {
    const uint64_t row = head ? (uint64_t)kvh * a.nf + j : (uint64_t)kvh * a.nl + j % a.nl;
    const uint4 *kr = (const uint4 *)((head ? a.kh : a.kt) + row * kAttnD + 32u * c);
    const uint4 *vr = (const uint4 *)((head ? a.vh : a.vt) + row * kAttnD + 32u * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kq[i] = kr[i];
      vq[i] = vr[i];
    }
  }
  uint4 *kd = (uint4 *)&Ks[key * kKsStride + 32u * c];
#pragma unroll
  for (int i = 0; i < 4; ++i) kd[i] = kq[i];
  const uint32_t pk = key ^ (16u * c);
  uint16_t *vt = (uint16_t *)Vt;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {vq[i].x, vq[i].y, vq[i].z, vq[i].w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vt[(32u * c + 8u * i + e) * kVtStride + pk] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
}

// fp16 values that are exact in bf16 too (at most 8 significant bits) as bf16.
__device__ __forceinline__ bf16x8 to_bf16x8(f16x8 h) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x2 b =
        __builtin_convertvector((f32x2{(float)h[2 * j], (float)h[2 * j + 1]}), bf16x2);
    r[2 * j] = b.x;
    r[2 * j + 1] = b.y;
  }
  return r;
}

// Reductions over the lanes l, l ^ 32 (and l ^ 16) with the gfx950 permlane
// swaps, which exchange rows of lanes in the VALU (a lane shuffle would take an
// LDS round trip): after a swap of v with itself the two results hold the value
// of each lane and of its partner, the same pair on both lanes.
__device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The one-multiply estimate E4M3(fl(a * 448)) of a P block's pattern (a <= 1):
// gfx950's FP32 -> FP8 (E4M3) convert rounds to nearest even exactly as the
// UE4M3 rounding does on [0, 448] (nvfp4_hw_self_check compares every binary32
// of that range on the device), in one instruction.
__device__ __forceinline__ uint32_t p_pattern_estimate(float am) {
  return min((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(am * 448.0f, 0.0f, 0, false) & 0xFFu, 126u);
}

// Online softmax of one 32-key tile held as an Sᵀ accumulator (sacc[v] = key
// 8 (v >> 2) + 4 g + (v & 3) of the tile; this lane's query; base-2 scores
// s = acc * c2, c2 > 0, so the max is taken on acc), then P to NVFP4 per 16
// keys (keys 16 blk .. +15: 8 in this lane, 8 in its partner lane ^ 32), max
// scaling under S_P = fl(1/2688), and back to exact fp16 values V[code] * s.
// Branch-free, so matrix instructions issued around it can run while it
// executes. Updates the running max m and sum l; returns the factor exp2(m_old
// - m_new) the accumulator must be rescaled by. pthr2 / ptbl: the PTables
// thresholds as pairs (thr[k], thr[k + 1]) and (r, s) per pattern, in LDS.
__device__ __forceinline__ float softmax_code_tile(const f32x16 &sacc, float c2, float &m,
                                                   float &l, const f32x2 *pthr2,
                                                   const f32x2 *ptbl, f16x8 (&pb)[2]) {
  float mt = -INFINITY;
#pragma unroll
  for (int v = 0; v < 16; ++v) mt = fmaxf(mt, sacc[v]);
  mt = pair_max32(mt) * c2;
  const float mn = fmaxf(m, mt);
  // with every score -inf so far, the exponent base 0 gives p = 0 and
  // alpha = 0 on an accumulator and sum that are still 0
  const float mb = mn == -INFINITY ? 0.0f : mn;
  const float alpha = __builtin_amdgcn_exp2f(m - mb);
  float p[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], c2, -mb));
  float ps = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) ps += p[v];
  l = l * alpha + ps;
  m = mn;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, p[8 * blk + e]);
    am = pair_max32(am);
    // a one-multiply estimate of the pattern E4M3(fl(fl(am / 6) / S_P)), never
    // more than one pattern off, corrected against the thresholds
    uint32_t pat = p_pattern_estimate(am);
    const f32x2 th = pthr2[pat];
    pat = am >= th.y ? pat + 1u : (am < th.x ? pat - 1u : pat);
    const f32x2 rs = ptbl[pat];
    uint32_t cw = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      cw = fp4_encode_pair(cw, p[8 * blk + 2 * j] * rs.x, p[8 * blk + 2 * j + 1] * rs.x, j);
    pb[blk] = decode8(cw, rs.y);
  }
  return alpha;
}

// CACHE: keys from the sink cache's three segments (else one coded segment).
// The query heads that share a KV head are adjacent rows of Q, so in cache
// mode (never causal) a workgroup takes 128 consecutive rows of those G * Nq
// and the cache is read once per KV head, not once per query head.
template <bool OUT_BF16, bool CACHE>
__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs a) {
  // two buffers: tile i is decoded into buffer i & 1 while the codes of tile
  // i + 1 are in flight, so one barrier per tile suffices
  __shared__ __attribute__((aligned(16))) _Float16 Ks[2][kChunk * kKsStride];
  __shared__ __attribute__((aligned(16))) _Float16 Vt[2][kAttnD * kVtStride];
  __shared__ f32x2 ptbl[128];
  __shared__ float pthr[128];
  __shared__ f32x2 pthr2[127];  // (pthr[k], pthr[k + 1]): both bounds in one read

  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6, g = lane >> 5;
  const uint32_t col = lane & 31u;
  // rows of Q this grid row covers: one head's Nq queries, or in cache mode the
  // G * Nq queries of the G heads of KV head blockIdx.y
  const uint32_t bh = blockIdx.y;
  const uint32_t rows = CACHE ? a.Nq * (a.Hq / a.Hkv) : a.Nq;
  const uint32_t kvh = CACHE ? bh : (bh / a.Hq) * a.Hkv + (bh % a.Hq) / (a.Hq / a.Hkv);
  // causal: the last query blocks see the most keys; dispatch them first
  const uint32_t qb = a.causal ? gridDim.x - 1u - blockIdx.x : blockIdx.x;
  const uint32_t q0 = qb * kQueriesPerGroup;
  const uint32_t qi = q0 + wave * 32u + col;
  const bool qvalid = qi < rows;
  // a wave without a valid query only helps load and decode the chunks
  const bool wave_live = q0 + wave * 32u < rows;

  // P's tables (see PTables); in the loop a one-multiply estimate
  // E4M3(fl(a * 448)) of the block pattern is never more than one pattern off
  // (checked over every binary32 in [0, 1]) and one comparison each way against
  // the thresholds corrects it.
  const float SP = 1.0f / 2688.0f;
  if (tid < 128u) {
    ptbl[tid] = f32x2{kPTables.r[tid], kPTables.s[tid]};
    pthr[tid] = kPTables.thr[tid];
  }

  const float qg = *a.qg;
  const float c2_coded = (qg * *a.kg) * a.tau_log2e;  // score scale, base 2
  const float c2_sink = qg * a.tau_log2e;
  const float vg = *a.vg;

  // keys: a.Nk, or in cache mode with a device-resident length, that length
  // (at most the cache's n_first + cap + n_last tokens)
  const uint32_t Nk = (CACHE && a.nk_dev) ? (uint32_t)min<int64_t>(*a.nk_dev, (int64_t)a.nf + a.cap + a.nl)
                                          : a.Nk;
  uint32_t kend = Nk;
  if (a.causal) {
    const int64_t qlast = (int64_t)min(q0 + kQueriesPerGroup, a.Nq) - 1;
    const int64_t last = qlast + (int64_t)Nk - (int64_t)a.Nq;
    kend = last < 0 ? 0u : (uint32_t)min<int64_t>(last + 1, Nk);
  }
  const int64_t lim = a.causal ? (int64_t)qi + (int64_t)Nk - (int64_t)a.Nq : (int64_t)Nk - 1;
  // the smallest lim of the wave (its first query), for the unmasked fast path
  const int64_t lim_wave =
      a.causal ? (int64_t)(q0 + wave * 32u) + (int64_t)Nk - (int64_t)a.Nq : (int64_t)Nk - 1;

  const uint64_t coded_base = CACHE ? (uint64_t)kvh * a.cap : (uint64_t)kvh * Nk;
  const uint32_t coded_off = CACHE ? a.nf : 0u;

  // This lane's B operand of S^T: query qi, elements 16 ks + 8 g .. +7.
  f16x8 qf[8];
  {
    const uint64_t row = (uint64_t)bh * rows + (qvalid ? qi : 0u);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint32_t w = 0u;
      float s = 0.0f;
      if (qvalid) {
        w = *(const uint32_t *)(a.qc + row * 64u + 8u * ks + 4u * g);
        s = scale_value(a.qs[row * 8u + ks]);
      }
      qf[ks] = decode8(w, s);
    }
  }
  __syncthreads();  // the P tables
  // published by the barrier that ends the first segment's prologue, before any use
  if (tid < 127u) pthr2[tid] = f32x2{pthr[tid], pthr[tid + 1u]};

  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = f32x16{};
  float m = -INFINITY, l = 0.0f;
  float unit = vg;  // the factor (tensor scale of V) the accumulator o is counted in
  uint32_t buf = 0;

  // S^T = K Q^T for one tile of 32 keys: sacc[v] = key 8 (v >> 2) + 4 g + (v & 3)
  // of the tile, query qi.
  auto s_tile = [&](auto sink_tag, const _Float16 *K) {
    constexpr bool SINK = decltype(sink_tag)::value;
    f32x16 sacc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (!SINK) {
        const f16x8 ka = *(const f16x8 *)&K[col * kKsStride + 16u * ks + 8u * g];
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[ks], sacc, 0, 0, 0);
      } else {
        const bf16x8 ka = *(const bf16x8 *)&K[col * kKsStride + 16u * ks + 8u * g];
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, to_bf16x8(qf[ks]), sacc, 0, 0, 0);
      }
    }
    return sacc;
  };

  // Keys that are absent (past hi) or not visible to this lane's query score
  // -inf. Full tiles (every key present and visible to every query of the
  // wave) are left as they are.
  auto mask_tile = [&](f32x16 &sacc, uint32_t t0, uint32_t hi) {
    const bool full = t0 + kKeyTile <= hi && (int64_t)(t0 + kKeyTile - 1u) <= lim_wave;
    if (!full) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t key = t0 + 8u * (v >> 2) + 4u * g + (v & 3);
        const bool vis = key < hi && (int64_t)key <= lim;
        sacc[v] = vis ? sacc[v] : -INFINITY;
      }
    }
  };

  auto softmax_code = [&](const f32x16 &sacc, float c2, f16x8 (&pb)[2]) {
    return softmax_code_tile(sacc, c2, m, l, pthr2, ptbl, pb);
  };

  // O^T = alpha O^T: multiplying by alpha = 1 changes nothing, so the wave
  // skips it when no lane needs it.
  auto rescale = [&](float alpha) {
    if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[t][v] *= alpha;
    }
  };

  // O^T += V^T P^T for the tile at key offset kb of the chunk; o[t][v] =
  // output d = 32 t + 8 (v >> 2) + 4 g + (v & 3). Row d = 32 t + col of V^T;
  // its key columns are XOR-ed with 16 t.
  auto pv_tile = [&](auto sink_tag, const _Float16 *V, uint32_t kb, const f16x8 (&pb)[2]) {
    constexpr bool SINK = decltype(sink_tag)::value;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const _Float16 *vrow = &V[(32u * t + col) * kVtStride];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const uint2 x0 = *(const uint2 *)(vrow + ((kb + 16u * blk + 4u * g) ^ (16u * t)));
        const uint2 x1 = *(const uint2 *)(vrow + ((kb + 16u * blk + 8u + 4u * g) ^ (16u * t)));
        const uint4 vv = make_uint4(x0.x, x0.y, x1.x, x1.y);
        if (!SINK)
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv), pb[blk],
                                                        o[t], 0, 0, 0);
        else
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                         to_bf16x8(pb[blk]), o[t], 0, 0, 0);
      }
    }
  };

  // Keys [lo, hi) of one segment, coded (SINK false) or bf16 sink rows of the
  // cache head or tail ring, in chunks of 64 keys that stay inside the segment.
  // Software-pipelined per chunk: tile 1's scores are issued to the matrix
  // units before tile 0's softmax, tile 0's P V^T before tile 1's softmax, and
  // tile 1's P V^T before the next chunk is decoded into the other LDS buffer;
  // one barrier per chunk publishes that buffer and retires the reads of this
  // one. A chunk's second tile past hi is all masked and adds nothing.
  auto run_segment = [&](auto sink_tag, uint32_t lo, uint32_t hi, bool head) {
    constexpr bool SINK = decltype(sink_tag)::value;
    if (lo >= hi) return;
    const float c2 = SINK ? c2_sink : c2_coded;
    const float cunit = SINK ? 1.0f : vg;
    if (cunit != unit) {  // at most twice per launch, uniform
      const float ratio = unit / cunit;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[t][v] *= ratio;
      unit = cunit;
    }
    TileRegs nxt{make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u), 0u, 0u};
    if (SINK) {
      store_sink_chunk(a, kvh, head, lo, hi, tid, Ks[buf], Vt[buf]);
    } else {
      nxt = load_chunk(a, coded_base, coded_off, lo, hi, tid);
      store_chunk(nxt, tid, Ks[buf], Vt[buf]);
      if (lo + kChunk < hi) nxt = load_chunk(a, coded_base, coded_off, lo + kChunk, hi, tid);
    }
    __syncthreads();
    for (uint32_t c0 = lo; c0 < hi; c0 += kChunk, buf ^= 1u) {
      const _Float16 *K = Ks[buf];
      const _Float16 *V = Vt[buf];
      if (wave_live) {
        f32x16 sa0 = s_tile(sink_tag, K);
        mask_tile(sa0, c0, hi);
        f32x16 sa1 = s_tile(sink_tag, K + kKeyTile * kKsStride);
        f16x8 pb0[2], pb1[2];
        const float a0 = softmax_code(sa0, c2, pb0);
        rescale(a0);
        mask_tile(sa1, c0 + kKeyTile, hi);
        pv_tile(sink_tag, V, 0u, pb0);
        const float a1 = softmax_code(sa1, c2, pb1);
        rescale(a1);
        pv_tile(sink_tag, V, kKeyTile, pb1);
      }
      const uint32_t c1 = c0 + kChunk;
      if (c1 < hi) {
        if (SINK) {
          store_sink_chunk(a, kvh, head, c1, hi, tid, Ks[buf ^ 1u], Vt[buf ^ 1u]);
        } else {
          store_chunk(nxt, tid, Ks[buf ^ 1u], Vt[buf ^ 1u]);
          if (c1 + kChunk < hi) nxt = load_chunk(a, coded_base, coded_off, c1 + kChunk, hi, tid);
        }
      }
      __syncthreads();
    }
  };

  if (CACHE) {
    // head sinks, coded middle, tail ring: tiles never straddle two segments
    const uint32_t mid_hi = max(Nk > a.nl ? Nk - a.nl : 0u, a.nf);
    run_segment(std::true_type{}, 0u, min(a.nf, Nk), true);
    run_segment(std::false_type{}, a.nf, mid_hi, false);
    run_segment(std::true_type{}, max(mid_hi, a.nf), Nk, false);
  } else {
    run_segment(std::false_type{}, 0u, kend, false);
  }

  l = pair_sum32(l);
  if (!qvalid) return;
  const uint64_t row = (uint64_t)bh * rows + qi;
  const float f = l > 0.0f ? (SP * unit) / l : 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t d0 = 32u * t + 8u * q4 + 4u * g;
      const float y0 = o[t][4 * q4] * f, y1 = o[t][4 * q4 + 1] * f;
      const float y2 = o[t][4 * q4 + 2] * f, y3 = o[t][4 * q4 + 3] * f;
      if (OUT_BF16) {
        const bf16x2 lo = __builtin_convertvector((f32x2{y0, y1}), bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2{y2, y3}), bf16x2);
        *(uint2 *)((uint16_t *)a.o + row * kAttnD + d0) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      } else {
        *(float4 *)((float *)a.o + row * kAttnD + d0) = make_float4(y0, y1, y2, y3);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split keys for decode steps: one wave per workgroup takes 16 query rows and
// one unit of keys (blockIdx.z: 0 the head, 1 the tail, 2 + k the k-th piece
// of `split` middle tokens), in chunks of 32 keys, one softmax tile each. With
// few valid rows (one query per head) the 4-wave kernel above keeps one wave in
// four busy; here each workgroup is one wave. Its K operands go from registers
// to the matrix instructions (each lane loads and decodes the code words of its
// own operand slices), so only V, transposed, passes through LDS: 12 KB a
// workgroup. A single wave needs no barrier: its LDS accesses run in order, so
// the next chunk's V is stored into the same buffer once this one's reads are
// issued, while the chunk after is in flight in registers (codes, or for the
// head and tail units the bf16 K and V rows, whose loads would otherwise sit in
// the dependent chain of every chunk). Two waves share each SIMD (the sink
// prefetch takes 64 registers), so up to 2,048 units' waves run at once.
// Writes the unit's state for attention_merge_kernel.
// ---------------------------------------------------------------------------
constexpr uint32_t kDecKeys = 32;                // keys per chunk = one softmax tile
constexpr uint32_t kDecVtStride = kDecKeys + 4;  // fp16 per V^T row (18 dwords)

// This lane's share of one coded chunk. K, as its A operands of Sᵀ: key
// 16 h + (t & 15) of the chunk (h = 0, 1), elements 32 (t >> 4) .. +31 (one
// 16-byte code word, slice s = 0..3 of it feeding the s-th product, since the
// sum over d may run in any order as long as Q's slices follow the same one)
// and their two block scales. V, to be transposed into LDS: key t >> 1,
// elements 64 (t & 1) .. +63 (two 16-byte code words, four scale bytes). Keys
// past the unit's end stay zero.
struct DecRegs {
  uint4 kw[2];
  uint32_t ks[2];
  uint4 v0, v1;
  uint32_t vs;
};

__device__ __forceinline__ DecRegs dec_load(const AttnArgs &a, uint64_t row_base, uint32_t c0,
                                            uint32_t hi, uint32_t t) {
  DecRegs r{};
  const uint32_t g = t >> 4, qc = t & 15u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t j = c0 + 16u * h + qc;
    if (j < hi) {
      const uint64_t row = row_base + (j - a.nf);
      r.kw[h] = *(const uint4 *)(a.kc + row * 64u + 16u * g);
      r.ks[h] = *(const uint16_t *)(a.ks + row * 8u + 2u * g);
    }
  }
  const uint32_t jv = c0 + (t >> 1), hv = t & 1u;
  if (jv < hi) {
    const uint64_t row = row_base + (jv - a.nf);
    const uint8_t *vc = a.vc + row * 64u + 32u * hv;
    r.v0 = *(const uint4 *)vc;
    r.v1 = *(const uint4 *)(vc + 16);
    r.vs = *(const uint32_t *)(a.vs + row * 8u + 4u * hv);
  }
  return r;
}

// V^T [d][key] in LDS: row d, the key column XOR-ed with 16 (d >> 6), so the
// two lanes of a key (d below and above 64) write different banks; 4-key
// groups stay contiguous for the products' reads.
__device__ __forceinline__ uint32_t dec_vt_index(uint32_t d, uint32_t key) {
  return d * kDecVtStride + (key ^ (16u * (d >> 6)));
}

// V of a loaded coded chunk decoded (block scales from the fp16 table) and
// transposed into LDS.
__device__ __forceinline__ void dec_store_v(const DecRegs &r, uint32_t t, const uint16_t *sf16,
                                            _Float16 *Vt) {
  const uint32_t key = t >> 1, d0 = 64u * (t & 1u);
  const uint32_t vw[8] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w};
  uint16_t vsf[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) vsf[b] = sf16[(r.vs >> (8 * b)) & 0xFFu];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f16x8 x = decode8_h(vw[i], vsf[i >> 1]);
#pragma unroll
    for (int e = 0; e < 8; ++e) Vt[dec_vt_index(d0 + 8u * i + e, key)] = x[e];
  }
}

// The K operand slice s of half h from loaded codes: elements 32 (t >> 4) + 8 s
// .. +7, in block 2 (t >> 4) + s / 2 of the key.
__device__ __forceinline__ f16x8 dec_k_operand(const DecRegs &r, int h, int s4,
                                               const uint16_t *sf16) {
  const uint32_t w[4] = {r.kw[h].x, r.kw[h].y, r.kw[h].z, r.kw[h].w};
  return decode8_h(w[s4], sf16[(r.ks[h] >> (8 * (s4 >> 1))) & 0xFFu]);
}

// Row of sink key j (bf16): the head, or the tail ring at slot j mod n_last.
__device__ __forceinline__ uint64_t sink_row(const AttnArgs &a, uint32_t kvh, bool head,
                                             uint32_t j) {
  return head ? (uint64_t)kvh * a.nf + j : (uint64_t)kvh * a.nl + j % a.nl;
}

// One chunk of sink keys as this lane loads them, one chunk ahead of its use
// (as the coded chunks): K rows of keys c0 + 16 h + (t & 15), elements
// 32 (t >> 4) .. +31 (the A operands of Sᵀ), and the V row of key c0 + (t >> 1),
// elements 64 (t & 1) .. +63 (for the transpose into LDS). Keys past hi stay zero.
struct SinkRegs {
  uint4 k[2][4];
  uint4 v[8];
};

__device__ __forceinline__ SinkRegs sink_load(const AttnArgs &a, uint32_t kvh, bool head,
                                              uint32_t c0, uint32_t hi, uint32_t t) {
  SinkRegs r;
  const uint32_t g = t >> 4, qc = t & 15u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t j = c0 + 16u * h + qc;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) r.k[h][s4] = make_uint4(0u, 0u, 0u, 0u);
    if (j < hi) {
      const uint4 *kr = (const uint4 *)((head ? a.kh : a.kt) + sink_row(a, kvh, head, j) * kAttnD +
                                        32u * g);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) r.k[h][s4] = kr[s4];
    }
  }
  const uint32_t jv = c0 + (t >> 1), d0 = 64u * (t & 1u);
#pragma unroll
  for (int i = 0; i < 8; ++i) r.v[i] = make_uint4(0u, 0u, 0u, 0u);
  if (jv < hi) {
    const uint4 *vr =
        (const uint4 *)((head ? a.vh : a.vt) + sink_row(a, kvh, head, jv) * kAttnD + d0);
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = vr[i];
  }
  return r;
}

// V of a loaded sink chunk transposed into LDS as bf16 bits.
__device__ __forceinline__ void sink_store_v(const SinkRegs &r, uint32_t t, _Float16 *Vt) {
  const uint32_t key = t >> 1, d0 = 64u * (t & 1u);
  uint16_t *vt = (uint16_t *)Vt;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vt[dec_vt_index(d0 + 8u * i + e, key)] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
}

// Online softmax and P coding of one 32-key tile in the 16 x 16 layout of the
// decode kernel: lane l holds, for query l & 15, the scores of keys 4 g + v
// (s0[v]) and 16 + 4 g + v (s1[v]), g = l >> 4, so each 16-key block of P is
// spread over the four lanes l, l ^ 16, l ^ 32, l ^ 48. The arithmetic is that
// of softmax_code_tile: base-2 scores s = acc * c2, running max m and sum l
// (this lane's share), P per 16 keys by max scaling under S_P = fl(1/2688),
// back to exact fp16 values; returns the accumulator's rescale factor. pb
// holds the lane's P values in the order of its scores (s0, then s1).
__device__ __forceinline__ float softmax_code_tile16(const f32x4 &s0, const f32x4 &s1, float c2,
                                                     float &m, float &l, const f32x2 *pthr2,
                                                     const f32x2 *ptbl, f16x8 &pb) {
  float mt = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                   fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
  mt = pair_max32(pair_max16(mt)) * c2;
  const float mn = fmaxf(m, mt);
  const float mb = mn == -INFINITY ? 0.0f : mn;  // every score -inf so far: p = 0
  const float alpha = __builtin_amdgcn_exp2f(m - mb);
  float p[8];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[v], c2, -mb));
    p[4 + v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[v], c2, -mb));
  }
  float ps = 0.0f;
#pragma unroll
  for (int v = 0; v < 8; ++v) ps += p[v];
  l = l * alpha + ps;
  m = mn;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float am = pair_max32(pair_max16(
        fmaxf(fmaxf(p[4 * blk], p[4 * blk + 1]), fmaxf(p[4 * blk + 2], p[4 * blk + 3]))));
    uint32_t pat = p_pattern_estimate(am);
    const f32x2 th = pthr2[pat];
    pat = am >= th.y ? pat + 1u : (am < th.x ? pat - 1u : pat);
    const f32x2 rs = ptbl[pat];
    uint32_t cw = fp4_encode_pair(0u, p[4 * blk] * rs.x, p[4 * blk + 1] * rs.x, 0);
    cw = fp4_encode_pair(cw, p[4 * blk + 2] * rs.x, p[4 * blk + 3] * rs.x, 1);
    const _Float16 sh = (_Float16)rs.y;
    const f16x2 s2 = {sh, sh};
    const f16x2 lo = fp4_pair_f16(cw, 0) * s2, hi = fp4_pair_f16(cw, 1) * s2;
    pb[4 * blk] = lo.x;
    pb[4 * blk + 1] = lo.y;
    pb[4 * blk + 2] = hi.x;
    pb[4 * blk + 3] = hi.y;
  }
  return alpha;
}

// 16 query rows per wave in the 16 x 16 x 32 matrix layout: with one query
// per head only a few rows are valid, and the narrower layout halves both the
// softmax work per lane and the accumulator registers against 32 x 32.
// Sᵀ = K Qᵀ per 16-key half h, in four products s: A = key 16 h + (l & 15),
// d = 32 g + 8 s .. +7; B = query l & 15, the same d; the result holds keys
// 16 h + 4 g + v.
// Oᵀ += Vᵀ Pᵀ per 16-row slice of d: the K index 8 g + e runs over keys
// 4 g + e (e < 4) and 16 + 4 g + e - 4, the order the lane holds its P in.
__global__ __launch_bounds__(64, 2) void attention_decode_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 Vt[kAttnD * kDecVtStride];
  __shared__ f32x2 ptbl[128];
  __shared__ f32x2 pthr2[127];
  __shared__ uint16_t sf16[256];

  const uint32_t t = threadIdx.x, g = t >> 4, qc = t & 15u;
  const uint32_t kvh = blockIdx.y;
  const uint32_t rows = a.Nq * (a.Hq / a.Hkv);
  const uint32_t qi = blockIdx.x * 16u + qc;
  const bool qvalid = qi < rows;
  const uint64_t row = (uint64_t)kvh * rows + (qvalid ? qi : 0u);

  const uint32_t z = blockIdx.z;
  const bool sink = z < 2u;
  // A middle unit's piece of the cache's capacity (rows nf .. nf + cap): its first
  // chunk is loaded from it before the token count is known (every row in
  // bounds), and the keys at or past the count are dropped once it is.
  const uint64_t coded_base = (uint64_t)kvh * a.cap;
  const uint64_t l64 = (uint64_t)a.nf + (uint64_t)(sink ? 0u : z - 2u) * a.split;
  const uint32_t slo = (uint32_t)min<uint64_t>(l64, (uint64_t)a.nf + a.cap);
  const uint32_t shi = (uint32_t)min<uint64_t>(l64 + a.split, (uint64_t)a.nf + a.cap);
  DecRegs cur{}, nxt{};
  if (!sink && slo < shi) cur = dec_load(a, coded_base, slo, shi, t);
  // The device-resident token count, if there is one, read by a vector load (the
  // pointer is hidden from the uniformity analysis): scalar loads may complete in
  // any order, so a wait for a later scalar would wait for this one too and hold
  // the set-up loads below back by a round trip. The three tensor scales (every
  // call passes all three) go out with it.
  int64_t nk_raw = a.Nk;
  if (a.nk_dev) {
    uint64_t pv = (uint64_t)a.nk_dev;
    asm volatile("" : "+v"(pv));
    nk_raw = *(const __attribute__((address_space(1))) int64_t *)pv;
  }
  const float qg = *a.qg, kg = *a.kg, vg = *a.vg;

  // Set-up loads in the order they are needed, so that each wait leaves the
  // later ones in flight (a coded unit's first chunk went first): the tables,
  // then this lane's Q codes, stored and decoded while the codes arrive.
  f32x2 tb_r[2], tb_t[2];
  uint16_t tb_s[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t k = t + 64u * i;
    tb_r[i] = f32x2{kPTables.r[k], kPTables.s[k]};
    tb_t[i] = f32x2{kPTables.thr[k], k < 127u ? kPTables.thr[k + 1u] : 0.0f};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) tb_s[i] = kScaleF16.v[t + 64u * i];
  uint4 qw = make_uint4(0u, 0u, 0u, 0u);
  uint32_t qsb = 0u;
  if (qvalid) {
    qw = *(const uint4 *)(a.qc + row * 64u + 16u * g);
    qsb = *(const uint16_t *)(a.qs + row * 8u + 2u * g);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t k = t + 64u * i;
    ptbl[k] = tb_r[i];
    if (k < 127u) pthr2[k] = tb_t[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sf16[t + 64u * i] = tb_s[i];

  // this lane's B operands of Sᵀ: query qi, elements 32 g + 8 s .. +7 (block 2 g + s / 2)
  f16x8 qf[4];
  {
    const uint32_t w[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      qf[s4] = decode8(w[s4], qvalid ? scale_value((qsb >> (8 * (s4 >> 1))) & 0xFFu) : 0.0f);
  }
  // a sink unit multiplies bf16 keys: its Q values (exact in bf16 too) are
  // converted once, in place, and read back as bf16 bits
  if (sink) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qf[s4] = __builtin_bit_cast(f16x8, to_bf16x8(qf[s4]));
  }

  const float c2 = sink ? qg * a.tau_log2e : (qg * kg) * a.tau_log2e;
  const float unit = sink ? 1.0f : vg;  // the factor the accumulator is counted in
  f32x4 o[8];  // o[i][v]: output d = 16 i + 4 g + v of query qi
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{};
  float m = -INFINITY, l = 0.0f;

  // keys present and this unit's range; a middle unit's [lo, hi) lies in
  // [slo, shi), with lo = slo when it is not empty (the middle ends at nf + cap)
  const uint32_t Nk = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)min<int64_t>(nk_raw, (int64_t)a.nf + a.cap + a.nl));
  const uint32_t mid_hi = max(Nk > a.nl ? Nk - a.nl : 0u, a.nf);
  uint32_t lo, hi;
  if (z == 0u) {
    lo = 0u;
    hi = min(a.nf, Nk);
  } else if (z == 1u) {
    lo = max(mid_hi, a.nf);
    hi = Nk;
  } else {
    lo = (uint32_t)min<uint64_t>(l64, mid_hi);
    hi = (uint32_t)min<uint64_t>(l64 + a.split, mid_hi);
  }
  // the first chunk's keys past hi (loaded before hi was known) score -inf in the
  // chunk loop; their V, which may hold any bits, is zeroed here
  if (slo + (t >> 1) >= hi) {
    cur.v0 = make_uint4(0u, 0u, 0u, 0u);
    cur.v1 = make_uint4(0u, 0u, 0u, 0u);
    cur.vs = 0u;
  }

  // Scores Sᵀ of the chunk at c0: coded keys from loaded codes r, sink keys read
  // here (rows past hi read as zeros).
  struct Scores {
    f32x4 h[2];
  };
  auto scores = [&](const auto &r) {
    constexpr bool SINK = std::is_same<std::decay_t<decltype(r)>, SinkRegs>::value;
    Scores sc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc.h[h] = f32x4{};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        if constexpr (!SINK)
          sc.h[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dec_k_operand(r, h, s4, sf16), qf[s4],
                                                           sc.h[h], 0, 0, 0);
        else
          sc.h[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, r.k[h][s4]), __builtin_bit_cast(bf16x8, qf[s4]), sc.h[h],
              0, 0, 0);
      }
    }
    return sc;
  };

  // The chunk loop, compiled once for sink units (bf16 keys) and once for coded
  // ones, so that no branch separates its loads from the matrix instructions.
  // Software-pipelined by one chunk: the next chunk's scores depend only on its
  // keys and Q, so their products are issued before this chunk's softmax, P
  // coding and PV products, which hold the dependent chain.
  // Keys of the chunk at c0 past the unit's end score -inf.
  auto mask_tail = [&](Scores &sc, uint32_t c0) {
    if (c0 + kDecKeys > hi) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sc.h[h][v] = c0 + 16u * h + 4u * g + v < hi ? sc.h[h][v] : -INFINITY;
    }
  };
  // The chunk's online softmax, P coding and O^T += V^T P^T (V^T in LDS).
  auto consume = [&](auto sink_tag, Scores &sc, uint32_t c0) {
    constexpr bool SINK = decltype(sink_tag)::value;
    mask_tail(sc, c0);
    f16x8 pb;
    const float alpha = softmax_code_tile16(sc.h[0], sc.h[1], c2, m, l, pthr2, ptbl, pb);
    if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t d = 16u * i + qc;
      const uint2 x0 = *(const uint2 *)&Vt[dec_vt_index(d, 4u * g)];
      const uint2 x1 = *(const uint2 *)&Vt[dec_vt_index(d, 16u + 4u * g)];
      const uint4 vv = make_uint4(x0.x, x0.y, x1.x, x1.y);
      if (!SINK)
        o[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, vv), pb, o[i], 0,
                                                      0, 0);
      else
        o[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv),
                                                       to_bf16x8(pb), o[i], 0, 0, 0);
    }
  };

  // Sink units: the first two chunks' bf16 rows loaded at once, then the chunk
  // loop pipelined by one chunk (the next chunk's score products, which need
  // only its keys and Q, issued before this chunk's softmax, P coding and PV
  // products, which hold the dependent chain; the next chunk's V stored into the
  // same buffer once this one's reads are issued, as LDS runs one wave's
  // accesses in order; the rows of the chunk after in flight).
  auto run_sink = [&]() {
    const bool head = z == 0u;
    if (lo >= hi) return;
    SinkRegs snxt;
    Scores sc;
    {
      const SinkRegs scur = sink_load(a, kvh, head, lo, hi, t);
      if (lo + kDecKeys < hi) snxt = sink_load(a, kvh, head, lo + kDecKeys, hi, t);
      sink_store_v(scur, t, Vt);
      sc = scores(scur);
    }
    for (uint32_t c0 = lo; c0 < hi; c0 += kDecKeys) {
      const uint32_t c1 = c0 + kDecKeys;
      Scores sn;
      if (c1 < hi) sn = scores(snxt);
      consume(std::true_type{}, sc, c0);
      if (c1 < hi) {
        sink_store_v(snxt, t, Vt);
        if (c1 + kDecKeys < hi) snxt = sink_load(a, kvh, head, c1 + kDecKeys, hi, t);
        sc = sn;
      }
    }
  };

  // Coded units: only the first chunk's codes are loaded in the set-up, so that
  // the first chunks of all units, which every wave requests at once, arrive
  // first; each wave asks for its second chunk once its first is in. The next
  // chunk's V store and score products follow this chunk's PV products (they
  // are needed only at the next chunk's softmax), the codes of the chunk after
  // in flight meanwhile.
  auto run_coded = [&]() {
    if (lo >= hi) return;
    dec_store_v(cur, t, sf16, Vt);
    Scores sc = scores(cur);
    if (lo + kDecKeys < hi) nxt = dec_load(a, coded_base, lo + kDecKeys, hi, t);
    for (uint32_t c0 = lo; c0 < hi; c0 += kDecKeys) {
      const uint32_t c1 = c0 + kDecKeys;
      consume(std::false_type{}, sc, c0);
      if (c1 < hi) {
        dec_store_v(nxt, t, sf16, Vt);
        sc = scores(nxt);
        if (c1 + kDecKeys < hi) nxt = dec_load(a, coded_base, c1 + kDecKeys, hi, t);
      }
    }
  };
  if (sink)
    run_sink();
  else
    run_coded();

  l = pair_sum32(pair_sum16(l));
  if (!qvalid) return;
  const uint64_t urow = row * a.ustride + z;
  float *dst = a.part + urow * kAttnD;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *(float4 *)(dst + 16u * i + 4u * g) =
        make_float4(o[i][0] * unit, o[i][1] * unit, o[i][2] * unit, o[i][3] * unit);
  if (g == 0u) a.ml[urow] = make_float2(m, l);
}

// The units' states of one output row merged: with M the largest base-2 max,
// w_u = 2^(m_u - M), O = S_P sum_u w_u acc_u / sum_u w_u l_u (0 with no key).
// One wave per (row, slice of 16 outputs): 16 groups of four lanes take the
// units u = j mod 16 (four outputs per lane). A lane loads the states and
// accumulator slices of its first kMergePre units together, so one memory round
// trip serves both the maximum and the sums, then the groups' maxima and sums
// are combined inside the wave (row rotations, then the permlane swaps between
// rows): no LDS and no barrier. The combination order is fixed, so the sums do
// not depend on timing, and a grid that covers more units (all empty: weight 0,
// zero terms) gives the same sums. Every slice forms the same sum of weights. A
// unit that saw no key holds m_u = -inf, l_u = 0 and a zero accumulator: its
// weight and terms are 0.
constexpr uint32_t kMergeSlices = kAttnD / 16;
constexpr uint32_t kMergeGroups = 16;
constexpr uint32_t kMergePre = 16;

// v combined with the lanes 4, 8 and 12 further round its row of 16 (row
// rotations: every lane of the row gets the combination of its four groups).
__device__ __forceinline__ float row_groups_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF,
                                                           false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF,
                                                             0xF, false)));
}
__device__ __forceinline__ float row_groups_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF,
                                                        false));
}

template <bool OUT_BF16>
__global__ __launch_bounds__(64) void attention_merge_kernel(AttnArgs a, uint32_t units) {
  const uint32_t row = blockIdx.x, slice = blockIdx.y, lane = threadIdx.x;
  const float2 *ml = a.ml + (uint64_t)row * a.ustride;
  const float *part = a.part + (uint64_t)row * a.ustride * kAttnD;
  const uint32_t grp = lane >> 2, q = lane & 3u;
  const uint32_t d0 = 16u * slice + 4u * q;
  float2 st[kMergePre];
  float4 pv[kMergePre];
#pragma unroll
  for (uint32_t k = 0; k < kMergePre; ++k) {
    const uint32_t u = grp + kMergeGroups * k;
    st[k] = make_float2(-INFINITY, 0.0f);
    pv[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (u < units) {
      st[k] = ml[u];
      pv[k] = *(const float4 *)(part + (uint64_t)u * kAttnD + d0);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (uint32_t k = 0; k < kMergePre; ++k) mx = fmaxf(mx, st[k].x);
  for (uint32_t u = grp + kMergeGroups * kMergePre; u < units; u += kMergeGroups)
    mx = fmaxf(mx, ml[u].x);
  const float M = pair_max32(pair_max16(row_groups_max(mx)));
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float L = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (uint32_t k = 0; k < kMergePre; ++k) {
      const float w = __builtin_amdgcn_exp2f(st[k].x - M);
      acc.x += w * pv[k].x;
      acc.y += w * pv[k].y;
      acc.z += w * pv[k].z;
      acc.w += w * pv[k].w;
      L += w * st[k].y;
    }
    for (uint32_t u = grp + kMergeGroups * kMergePre; u < units; u += kMergeGroups) {
      const float2 s2 = ml[u];
      const float4 p = *(const float4 *)(part + (uint64_t)u * kAttnD + d0);
      const float w = __builtin_amdgcn_exp2f(s2.x - M);
      acc.x += w * p.x;
      acc.y += w * p.y;
      acc.z += w * p.z;
      acc.w += w * p.w;
      L += w * s2.y;
    }
  }
  acc.x = pair_sum32(pair_sum16(row_groups_sum(acc.x)));
  acc.y = pair_sum32(pair_sum16(row_groups_sum(acc.y)));
  acc.z = pair_sum32(pair_sum16(row_groups_sum(acc.z)));
  acc.w = pair_sum32(pair_sum16(row_groups_sum(acc.w)));
  L = pair_sum32(pair_sum16(row_groups_sum(L)));
  if (grp != 0u) return;
  const float f = L > 0.0f ? (1.0f / 2688.0f) / L : 0.0f;
  const float y0 = acc.x * f, y1 = acc.y * f, y2 = acc.z * f, y3 = acc.w * f;
  if (OUT_BF16) {
    const bf16x2 lo = __builtin_convertvector((f32x2{y0, y1}), bf16x2);
    const bf16x2 hi = __builtin_convertvector((f32x2{y2, y3}), bf16x2);
    *(uint2 *)((uint16_t *)a.o + (uint64_t)row * kAttnD + d0) =
        make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  } else {
    *(float4 *)((float *)a.o + (uint64_t)row * kAttnD + d0) = make_float4(y0, y1, y2, y3);
  }
}

hipError_t launch_attention(const AttnArgs &a, bool out_bf16, hipStream_t s) {
  if (a.cache) {
    // rows of one KV head's query heads per grid row
    const uint32_t rows = a.Nq * (a.Hq / a.Hkv);
    const uint32_t cap_mid = a.nk_dev ? a.cap : (a.Nk > a.nf + a.nl ? a.Nk - a.nf - a.nl : 0u);
    if (a.split) {  // units: head, tail, middle pieces
      const uint32_t units = 2u + (cap_mid + a.split - 1u) / a.split;
      const dim3 dgrid((rows + 15u) / 16u, a.B * a.Hkv, units);
      hipLaunchKernelGGL(attention_decode_kernel, dgrid, dim3(64), 0, s, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_attention_merge(a, units, out_bf16, s);
    }
    const dim3 grid((rows + kQueriesPerGroup - 1) / kQueriesPerGroup, a.B * a.Hkv);
    if (out_bf16)
      hipLaunchKernelGGL((attention_kernel<true, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attention_kernel<false, true>), grid, dim3(256), 0, s, a);
  } else {
    const dim3 grid((a.Nq + kQueriesPerGroup - 1) / kQueriesPerGroup, a.B * a.Hq);
    if (out_bf16)
      hipLaunchKernelGGL((attention_kernel<true, false>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attention_kernel<false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attention_merge(const AttnArgs &a, uint32_t units, bool out_bf16,
                                  hipStream_t s) {
  const dim3 grid(a.B * a.Hq * a.Nq, kMergeSlices);
  if (out_bf16)
    hipLaunchKernelGGL((attention_merge_kernel<true>), grid, dim3(64), 0, s, a, units);
  else
    hipLaunchKernelGGL((attention_merge_kernel<false>), grid, dim3(64), 0, s, a, units);
  return hipGetLastError();
}

}  // namespace nvfp4
