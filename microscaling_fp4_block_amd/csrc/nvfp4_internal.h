// nvfp4_internal.h -- launch descriptors shared by the host API and the kernels
// of the gfx950 NVFP4 library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kThreads = 256;          // 4 wave64 per workgroup
constexpr int kMaxAmaxGroups = 512;    // partial maxima kept in the workspace
// Grid cap of the streaming dequantize: fewer concurrent streams write HBM faster
// here. On the 8192 x 28672 tensor a sweep of 256-4096 workgroups put 352 first (bf16
// out 97.0 -> 83.4 us, FP32 out 210 -> 149 us against 1024; 256, 288 and 384-512 slower).
constexpr int kMaxStreamGroups = 352;
constexpr int kMaxQuantGroups = 8192;  // grid cap of the block-parallel kernels
// Grid cap of the certified search: up to four blocks per lane, so the last
// round of workgroups is short (measured 253 us against 256 us at 8192 groups
// on an 8192 x 28672 bf16 tensor, the same as at 28672 groups, which repeat
// the per-workgroup set-up twice as often; a persistent grid of 1792 took 282 us).
constexpr int kMaxCertGroups = 14336;

// Division by a runtime constant with one high multiply (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994,
// the round-up variant): q = (umulhi(n, m) + n) >> s for every 32-bit n,
// for divisors 1 <= d <= 2^31.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

// Where block b of the quantized region lives in the input, and where its
// codes go. Plain tensors are one contiguous region (segments == 0, output
// block b). The attention-sink mode quantizes the middle tokens of every
// (batch, head) segment: row r of the region is token n_first + (r mod tm) of
// segment r / tm, a segment spans seg_tokens input rows; output block b.
// Append mode (append != 0) quantizes the tokens that leave the recent window
// of a KV cache: row r of the region is token pos = lo + (r mod tm) of segment
// g = r / tm; a token below t_old comes from the ring [segments][n_last][cols]
// (slot pos mod n_last), a later one from x [segments][t_new][cols] (row
// pos - t_old); its codes go to row g * cap + pos - n_first of the cache.
// With len_dev set, t_old is read from that device word when the kernel runs,
// tm is t_new (an upper bound on the positions that leave the window), lo and
// the end of the window follow from t_old, rows past the end are skipped, and
// an append that would not fit (t_old + t_new > total) skips every row.
struct RegionMap {
  uint32_t nblocks;     // 16-element blocks in the region
  uint32_t bpr;         // blocks per row (cols / 16)
  FastDiv div_bpr;
  uint32_t segments;    // 0: plain contiguous region
  uint32_t tm;          // region rows per segment
  FastDiv div_tm;
  uint32_t seg_tokens;  // input rows per segment (T)
  uint32_t n_first;     // first region row inside a segment
  uint32_t cols;        // elements per row
  uint32_t append;      // append mode
  uint32_t lo, t_old, n_last, t_new, cap;
  FastDiv div_nlast;
  const void *ring;
  const int64_t *len_dev;  // device-resident t_old (append mode), or null
  uint32_t total;          // n_first + cap + n_last: tokens the cache holds
};

// Random sign flips of the randomized Hadamard transform: bit k of w[k / 32]
// set negates input feature k of every 128-vector before H is applied.
struct HadamardSigns {
  uint32_t on;    // 0: plain transform (w ignored)
  uint32_t w[4];
};

// The balancing pair Q' = Q diag(2^-e), K' = K diag(2^e): channel exponents
// e[cols] (device, int8, 16-byte aligned; clamped to [-32, 32]) applied with
// the sign `side` (+1 or -1) to every row before anything else (before the
// Hadamard transform, whose kernels then need cols == 128).
struct Balance {
  const int8_t *e;  // null: no balancing
  int32_t side;
};

struct QuantArgs {
  const void *x;
  uint8_t *codes;
  uint8_t *scales;
  float *gscale;              // read when npartials == 0, else written by workgroup 0
  const uint32_t *partials;   // per-workgroup maxima of the amax pass
  int npartials;              // 0: the tensor scale is given
  RegionMap map;
  int f_lo, f_hi;
  HadamardSigns hs;           // Hadamard kernels only
  Balance bal;
};

struct AmaxArgs {
  const void *x;
  uint32_t *partials;
  RegionMap map;
  HadamardSigns hs;           // Hadamard kernels only
  Balance bal;
};

// Column sums of squares of the balancing pair's calibration (double): the
// partial sums of workgroup g over its rows go to part[g][cols].
struct ColSumArgs {
  const void *x;
  uint32_t rows, cols;
  double *part;
};

struct DequantArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  const float *gscale;
  void *y;
  uint32_t nblocks;
};

// Append: copy new tokens kv_new[BH][t_new][D] at positions t_old.. into the
// cache head [BH][n_first][D] (positions < n_first) or tail ring
// [BH][n_last][D] (positions >= t_old + t_new - n_last, slot pos mod n_last).
struct AdmitArgs {
  const void *src;
  void *head, *tail;
  uint32_t t_old, t_new, n_first, n_last;
  uint32_t chunks_per_row, nchunks;
  FastDiv div_cpr, div_tnew, div_nlast;
  const int64_t *len_dev;  // device-resident t_old, or null
  uint32_t total;          // tokens the cache holds (with len_dev)
};

// Sink copy / reassembly: BH segments of T tokens of D elements; tokens
// [0, n_first) and [T - n_last, T) live in sink[BH][n_first + n_last][D].
struct SinkArgs {
  const void *src;
  void *dst;
  uint32_t bh, T, D, n_first, n_last;
  uint32_t nchunks;      // 16-byte chunks to move
  uint32_t chunks_per_row;
  FastDiv div_cpr;
  FastDiv div_ns;        // n_first + n_last
};

struct DequantKvArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  const float *gscale;
  const void *sink;
  void *y;
  uint32_t nblocks;      // output blocks: BH * T * D / 16
  uint32_t bpr;          // D / 16
  FastDiv div_bpr;
  FastDiv div_T;
  uint32_t T, n_first, n_last;
};

// Launchers (nvfp4_kernels.hip). Return hipSuccess or the launch error.
hipError_t launch_amax(const AmaxArgs &a, bool bf16, int groups, hipStream_t s);
hipError_t launch_finalize(const uint32_t *partials, int n, float *gscale, hipStream_t s);
hipError_t launch_quantize(const QuantArgs &a, bool bf16, hipStream_t s);
int amax_hadamard_groups(uint32_t nblocks);
hipError_t launch_amax_hadamard(const AmaxArgs &a, int groups, hipStream_t s);
hipError_t launch_quantize_hadamard(const QuantArgs &a, hipStream_t s);
// MXFP4 contrast format: 32-element blocks, E8M0 scale bytes.
struct MxArgs {
  const void *x;
  uint8_t *codes;
  uint8_t *scales;
  uint32_t nblocks;
  int f_lo, f_hi;
};

struct MxDequantArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  void *y;
  uint32_t nblocks;
};

// Attention on NVFP4 operands (head dimension 128).
struct AttnArgs {
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;  // codes [rows][64], scales [rows][8]
  const float *qg, *kg, *vg;                   // device tensor scales
  void *o;                                     // [B][Hq][Nq][128] FP32 or bf16
  uint32_t B, Hq, Hkv, Nq, Nk;                 // Nk: keys (tokens in the cache)
  uint32_t causal;
  float tau_log2e;                             // log2(e) / sqrt(128)
  // sink-cache mode: bf16 head [BHkv][nf][128] and tail ring [BHkv][nl][128];
  // coded middle rows [BHkv][cap] (token t at row t - nf)
  uint32_t cache;
  const uint16_t *kh, *kt, *vh, *vt;
  uint32_t nf, nl, cap;
  const int64_t *nk_dev;  // cache mode: device-resident token count (replaces Nk), or null
  // cache mode with split keys (split > 0 tokens per middle piece): unit z of the grid
  // (0 head, 1 tail, 2 + k middle piece k) writes its softmax state to part
  // [rows][ustride][128] (accumulator times the unit's value factor) and
  // ml [rows][ustride] (running max in base 2, sum); attention_merge combines them
  uint32_t split, ustride;
  float *part;
  float2 *ml;
};

hipError_t launch_attention_merge(const AttnArgs &a, uint32_t units, bool out_bf16,
                                  hipStream_t s);

hipError_t launch_attention(const AttnArgs &a, bool out_bf16, hipStream_t s);

hipError_t launch_mx_quantize(const MxArgs &a, bool bf16, hipStream_t s);
hipError_t launch_mx_dequantize(const MxDequantArgs &a, bool out_bf16, hipStream_t s);

hipError_t launch_hadamard(const uint16_t *x, float *y, uint32_t nvec, const HadamardSigns &hs,
                           const Balance &bal, hipStream_t s);
// Balancing pair calibration: per-workgroup column sums of squares of x (cols
// % 8 == 0, cols <= 2048) into part[kColSumGroups][cols], then the channel
// exponents from Q's and K's sums.
constexpr int kColSumGroups = 256;
hipError_t launch_colsumsq(const ColSumArgs &a, bool bf16, hipStream_t s);
hipError_t launch_balance_exponents(const double *qpart, const double *kpart, uint32_t cols,
                                    int8_t *e, hipStream_t s);
hipError_t launch_dequantize(const DequantArgs &a, bool out_bf16, hipStream_t s);
hipError_t launch_sink_copy(const SinkArgs &a, bool bf16, hipStream_t s);
hipError_t launch_admit(const AdmitArgs &a, bool bf16, hipStream_t s);
hipError_t launch_advance_length(int64_t *len, uint32_t t_new, uint32_t total, hipStream_t s);
// The coding, admit and (with len, the device-resident length, else null) length
// advance of one append in a single workgroup: for appends of at most
// kSmallAppendBlocks coded blocks and kSmallAppendChunks admitted 16-byte chunks,
// without the Hadamard transform.
constexpr uint32_t kSmallAppendBlocks = 256, kSmallAppendChunks = 1024;
hipError_t launch_kv_append_small(const QuantArgs &q, const AdmitArgs &c, int64_t *len,
                                  bool bf16, hipStream_t s);
// The K and V appends of a decode step: two small appends, one workgroup each.
struct KvAppendPair {
  QuantArgs q[2];
  AdmitArgs c[2];
  int64_t *len[2];
  uint32_t row_bytes;
};
hipError_t launch_kv_append_small_pair(const KvAppendPair &p, bool bf16, hipStream_t s);
hipError_t launch_dequantize_kv(const DequantKvArgs &a, bool sink_bf16, bool out_bf16,
                                hipStream_t s);

}  // namespace nvfp4
