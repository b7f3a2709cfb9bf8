/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 block quantizer with ScaleSearch.
 *
 * What is computed (web pages, cited by title and section):
 *  - "NVIDIAのFP4推論が50倍の効率を実現", 超低精度推論を支えるアーキテクチャ: NVFP4
 *    codes each value as E2M1 (1 sign, 2 exponent, 1 mantissa bit), with one
 *    E4M3 scale per 16-value micro-block and a second FP32 per-tensor scale.
 *  - "技術サマリー：ブロック浮動小数点スケールを検索せよ！" (ScaleSearch summary),
 *    手法 > ScaleSearch: the default block scale is round(amax / 6); ScaleSearch
 *    instead adds integer offsets f to the default scale's UE4M3 bit pattern
 *    (メカニズム) and keeps, over a small range such as f in [-2, 6], the scale
 *    with the least block MSE (検索戦略).
 *  - same page, ScaleSearchAttention: a Hadamard transform of Q and K before
 *    coding (非干渉処理（IP）と絶対値低減), and a KV cache whose first and last
 *    blocks stay at full precision (アテンション・シンク対応混合精度キャッシング).
 *
 * Numerics (identical to the CPU oracle, bit for bit):
 *  A     = max |x| over the quantized region; NaN/Inf anywhere -> S_g = NaN.
 *  S_g   = fl(A / 2688) (2688 = 6 * 448), or 1 if that is 0. Decode scale.
 *  block : a_b = max |x_i| over 16 consecutive elements of the last dimension;
 *          p0 = UE4M3 round-to-nearest-even-saturating of fl(fl(a_b / 6) / S_g).
 *  candidates p = p0 + f, f = 0 first, then f_lo..f_hi; p outside 0..126 is
 *          skipped. d = fl(s_p * S_g), r = fl(1 / d); if r is not finite the
 *          candidate codes everything as 0. Each element: y = fl(|x| * r),
 *          c = E2M1 nearest-even-saturating(y), xhat = fl(V[c] * d),
 *          e = fl(|x| - xhat); SSE = sum of fl(e * e) strictly left to right
 *          in FP32 (no fused multiply-add). The first candidate with strictly
 *          smaller SSE wins (ties keep f = 0, then the lowest f).
 *  codes : nibble = sign(x) << 3 | c (sign copied even for c = 0); byte j of a
 *          row holds elements 2j (low nibble) and 2j + 1 (high nibble).
 *  scales: the winning pattern p (0..126), one byte per block; 0x7F (NaN) marks
 *          a block coded under the non-finite contract (all code bytes 0).
 *  dequantize: xhat = (-1)^sign * fl(V[c] * fl(s_p * S_g)); bf16 output is the
 *          nearest-even bf16 of that FP32 value. A scale byte >= 127 gives NaN.
 *
 * Conventions for every entry point:
 *  - Every tensor pointer is a device pointer (HIP global memory) owned by the
 *    caller; the library allocates nothing and keeps no state between calls.
 *  - Tensors are dense and row-major; blocks of 16 run along the last
 *    dimension. Input tensors must be 16-byte aligned; codes 8-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream). All device work is
 *    enqueued on it and the call returns without waiting. The returned status
 *    reports argument checks (made on the host before anything is enqueued)
 *    and launch errors; data-dependent cases follow the non-finite contract
 *    above instead of an error.
 *  - Calls that use the same workspace must not overlap in time.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

/* Exported symbols (the library is built with hidden default visibility). */
#if defined(__GNUC__) || defined(__clang__)
#define NVFP4_API __attribute__((visibility("default")))
#else
#define NVFP4_API
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_EINVAL = 1,     /* null pointer, unknown dtype/flag, block != 16, bad offsets */
    NVFP4_ESHAPE = 2,     /* a size is negative, not a multiple of 16 (128 with the
                             Hadamard), too large, or sink sizes exceed T */
    NVFP4_EALIGN = 3,     /* input not 16-byte aligned or codes not 8-byte aligned */
    NVFP4_EWORKSPACE = 4, /* workspace missing or smaller than nvfp4_workspace_bytes() */
    NVFP4_EHIP = 5        /* a HIP launch failed */
} nvfp4_status;

typedef enum {
    NVFP4_F32 = 0,  /* IEEE binary32 */
    NVFP4_BF16 = 1  /* bfloat16 */
} nvfp4_dtype;

/* Flags for the quantize calls. */
#define NVFP4_HADAMARD128 1u  /* transform each 128-vector by H/sqrt(128) first (bf16 input) */
#define NVFP4_GSCALE_GIVEN 2u /* *global_scale is an input: skip the global amax pass */
#define NVFP4_PAIR_Q 4u       /* balancing pair: this tensor is the Q side (2^-e), else K (2^e) */

/* Text for a status code (static storage). */
NVFP4_API const char *nvfp4_status_str(nvfp4_status s);

/* NVFP4_ABI_VERSION of the built library. */
NVFP4_API int nvfp4_abi_version(void);

/* Checks, on the current device, two properties of gfx950's converters that the
 * attention kernels rely on; blocking (runs on the null stream, allocates 16 bytes
 * of device memory for the call). counts (host int64[2]) receives: [0] the
 * binary32 values t in [0, 448] whose hardware FP32 -> FP8 (E4M3) convert differs
 * from the nearest-even UE4M3 rounding (their P block-pattern estimate); [1] the
 * bytes 0..126 whose hardware FP8 -> FP32 convert differs from their UE4M3 value
 * (their block-scale decode; the pages' block scales are UE4M3, which for these
 * bytes coincides with OCP E4M3). Both are 0 on a conforming device.
 * NVFP4_EINVAL for a null counts, NVFP4_EHIP for a runtime error. */
NVFP4_API nvfp4_status nvfp4_hw_self_check(int64_t *counts);

/* Bytes of device workspace the quantize calls need for a rows x cols region
 * (it holds the per-workgroup partial maxima of the global amax pass). */
NVFP4_API size_t nvfp4_workspace_bytes(int64_t rows, int64_t cols, uint32_t flags);

/* Quantize x[rows][cols] (xdt) to NVFP4 with ScaleSearch over offsets
 * [f_lo, f_hi] (f_lo <= 0 <= f_hi, |f| <= 126; the pages' example range is
 * [-2, 6]; [0, 0] is plain max scaling). block must be 16; cols % 16 == 0
 * (cols % 128 == 0 and xdt == NVFP4_BF16 with NVFP4_HADAMARD128).
 * Outputs: codes[rows][cols/2], scales[rows][cols/16], global_scale[1]
 * (written, or read when NVFP4_GSCALE_GIVEN: then it must be positive and
 * finite, and only blocks holding a NaN/Inf get the non-finite contract).
 * With NVFP4_HADAMARD128 the codes are those of y = x H / sqrt(128) (FP32);
 * dequantize then returns y-domain values (H/sqrt(128) is its own inverse). */
NVFP4_API nvfp4_status nvfp4_quantize(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                            int block, int f_lo, int f_hi, uint32_t flags, uint8_t *codes,
                            uint8_t *scales, float *global_scale, void *workspace,
                            size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory or pass a workspace (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * exactly nvfp4_quantize (same arguments, checks, outputs and bytes), with the
 * partial maxima of the global amax pass kept in a library-owned device array of
 * nvfp4_noalloc_scratch_bytes() bytes (2 KiB; every tensor size fits, the amax
 * pass never keeps more than 512 partials) instead of a workspace. Each GPU the
 * library runs on holds its own copy until the process ends; its address is
 * looked up on the first call on that GPU (the device of `stream`, or the
 * current device for the null stream). All calls on one GPU share that array:
 * calls that overlap in time on one GPU race and must be ordered by the caller
 * (one stream, or events). The call allocates nothing (no hipMalloc, no
 * library allocation) and enqueues only kernel launches. NVFP4_EHIP if the
 * array's address cannot be found. */
NVFP4_API nvfp4_status nvfp4_quantize_noalloc(const void *x, nvfp4_dtype xdt, int64_t rows,
                                    int64_t cols, int block, int f_lo, int f_hi,
                                    uint32_t flags, uint8_t *codes, uint8_t *scales,
                                    float *global_scale, void *stream);

/* Size in bytes of the device array nvfp4_quantize_noalloc uses on each GPU. */
NVFP4_API size_t nvfp4_noalloc_scratch_bytes(void);

/* Only the global scale: S_g of x[rows][cols] (after the Hadamard transform
 * with NVFP4_HADAMARD128) into global_scale[1]. The first half of
 * nvfp4_quantize; feed the result back with NVFP4_GSCALE_GIVEN. */
NVFP4_API nvfp4_status nvfp4_global_scale(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                                uint32_t flags, float *global_scale, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Inverse: y[rows][cols] (ydt: FP32 or bf16) from codes, scales and the
 * device-resident global_scale[1]. */
NVFP4_API nvfp4_status nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales,
                              const float *global_scale, int64_t rows, int64_t cols, int block,
                              void *y, nvfp4_dtype ydt, void *stream);

/* Attention-sink KV mode. kv[B][H][T][D] (dt). For every (b, h) the first
 * n_first and last n_last tokens are copied verbatim to
 * sink[B][H][n_first + n_last][D] (dt; first, then last), and the middle
 * Tm = T - n_first - n_last tokens are quantized as one region (its global
 * amax excludes the sink tokens): codes[B][H][Tm][D/2],
 * scales[B][H][Tm][D/16]. Requires n_first + n_last <= T and D % 16 == 0. */
NVFP4_API nvfp4_status nvfp4_quantize_kv_sink(const void *kv, nvfp4_dtype dt, int64_t B, int64_t H,
                                    int64_t T, int64_t D, int64_t n_first, int64_t n_last,
                                    int block, int f_lo, int f_hi, uint32_t flags,
                                    uint8_t *codes, uint8_t *scales, float *global_scale,
                                    void *sink, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Inverse of the sink mode: y[B][H][T][D] (ydt) with the sink tokens copied
 * exactly (bf16 -> FP32 widening is exact; FP32 -> bf16 rounds to nearest
 * even) and the middle tokens dequantized. */
NVFP4_API nvfp4_status nvfp4_dequantize_kv_sink(const uint8_t *codes, const uint8_t *scales,
                                      const float *global_scale, const void *sink,
                                      nvfp4_dtype sink_dt, int64_t B, int64_t H, int64_t T,
                                      int64_t D, int64_t n_first, int64_t n_last, int block,
                                      void *y, nvfp4_dtype ydt, void *stream);

/* KV-cache append with attention sinks (decode-time streaming of the sink mode).
 * The cache, per (b, h): head[B][H][n_first][D] (dt) holds the first n_first
 * tokens verbatim; tail[B][H][n_last][D] (dt) is a ring of the n_last most recent
 * tokens, token t at slot t mod n_last; codes[B][H][cap][D/2] and
 * scales[B][H][cap][D/16] hold middle token t (n_first <= t < T - n_last) at row
 * t - n_first. T is the number of tokens already in the cache. The call appends
 * kv_new[B][H][t_new][D] as tokens T .. T + t_new - 1: tokens that leave the recent
 * window are coded with the tensor scale *global_scale (a device float the caller
 * holds fixed: the pages do not say how the tensor scale evolves as tokens arrive;
 * one taken from the prefill's middle tokens with nvfp4_global_scale fits, larger
 * values saturate), and the new tokens that stay in full precision go to the head
 * or the ring. After the call the cache holds exactly what nvfp4_quantize_kv_sink
 * with NVFP4_GSCALE_GIVEN and the same scale gives for tokens 0 .. T + t_new - 1
 * (ring order aside). Requires the middle rows to fit: max(n_first, T + t_new -
 * n_last) - n_first <= cap. flags: NVFP4_HADAMARD128 allowed (bf16, D % 128 == 0);
 * the scale is always read. Calls on one cache must not overlap in time. */
NVFP4_API nvfp4_status nvfp4_kv_append(const void *kv_new, nvfp4_dtype dt, int64_t B, int64_t H,
                                       int64_t T, int64_t t_new, int64_t D, int64_t n_first,
                                       int64_t n_last, int64_t cap, int block, int f_lo, int f_hi,
                                       uint32_t flags, const float *global_scale, void *head,
                                       void *tail, uint8_t *codes, uint8_t *scales, void *stream);

/* nvfp4_kv_append with the token count T held in device memory, so a decode
 * step can be captured once in a HIP graph and replayed token after token (the
 * caller refills kv_new in place between replays). length: device int64[1],
 * 8-byte aligned; the kernels read T = *length when they run and the call ends
 * by setting *length = T + t_new, all in stream order. An append that does not
 * fit the cache (T + t_new > n_first + cap + n_last) changes neither the cache
 * nor *length (check the length to detect it: nothing is reported at call time,
 * T being on the device). signs: NULL, or four uint32 words for the randomized
 * Hadamard transform as in nvfp4_kv_append_rht (read during the call only).
 * Everything else, including the result, is as nvfp4_kv_append with T = *length. */
NVFP4_API nvfp4_status nvfp4_kv_append_dev(const void *kv_new, nvfp4_dtype dt, int64_t B,
                                           int64_t H, int64_t t_new, int64_t D, int64_t n_first,
                                           int64_t n_last, int64_t cap, int block, int f_lo,
                                           int f_hi, uint32_t flags, const uint32_t *signs,
                                           const float *global_scale, void *head, void *tail,
                                           uint8_t *codes, uint8_t *scales, int64_t *length,
                                           void *stream);

/* One KV cache of nvfp4_kv_append2_dev: the new tokens and the cache arrays
 * with their meaning in nvfp4_kv_append_dev (flags and signs likewise, per
 * cache, so that K may take the randomized Hadamard transform and V not). */
typedef struct {
  const void *kv_new;
  uint32_t flags;
  const uint32_t *signs;
  const float *global_scale;
  void *head;
  void *tail;
  uint8_t *codes;
  uint8_t *scales;
  int64_t *length;
} nvfp4_kv_cache_ref;

/* The K and the V append of one decode step (ScaleSearch summary page,
 * ScaleSearchAttention: the mixed-precision KV cache, extended token by token)
 * in one call: exactly nvfp4_kv_append_dev on *k, then on *v, with the shared
 * shape and offset arguments. k and v: host pointers to the two caches' refs,
 * read during the call only. The two caches must not overlap and must keep
 * their own length words (k->length == v->length is NVFP4_EINVAL). Both are
 * checked before anything is enqueued. When both appends are small (at most 256
 * coded blocks and 1024 admitted 16-byte chunks each, no Hadamard: a decode
 * step's) they run as one launch of two workgroups; otherwise as the two calls. */
NVFP4_API nvfp4_status nvfp4_kv_append2_dev(const nvfp4_kv_cache_ref *k,
                                            const nvfp4_kv_cache_ref *v, nvfp4_dtype dt,
                                            int64_t B, int64_t H, int64_t t_new, int64_t D,
                                            int64_t n_first, int64_t n_last, int64_t cap,
                                            int block, int f_lo, int f_hi, void *stream);

/* The FP32 Hadamard pre-transform alone: y[rows][128] = x[rows][128] H/sqrt(128)
 * (x bf16), as the quantizer computes it on the fly. For inspection and split
 * parity checks; the quantize path never writes it to memory. */
NVFP4_API nvfp4_status nvfp4_hadamard128(const void *x, nvfp4_dtype xdt, int64_t rows, float *y,
                               void *stream);

/* Attention on NVFP4 operands (ScaleSearch summary page, ScaleSearchAttention:
 * QK^T and PV with NVFP4 operands and FP32 accumulation). q: codes
 * [B][Hq][Nq][64], scales [B][Hq][Nq][8], tensor scale q_gscale[1]; k and v the
 * same with Hkv heads and Nk keys (Hq % Hkv == 0: query head h reads K/V head
 * h / (Hq / Hkv)), as nvfp4_quantize writes them for rows of 128 elements (the
 * head dimension must be 128). Computes, per query row i,
 *   s_j = (q_i . k_j) * Sq * Sk / sqrt(128) with q, k the values V[code] * s_block,
 * an online softmax over tiles of 32 keys (p_j = exp(s_j - m), m the running max),
 * P coded to NVFP4 per 16 keys of a tile by max scaling under the fixed tensor
 * scale fl(1/2688), and O_i = (sum_j P^_j v_j) * fl(1/2688) * Sv / l_i, l_i the
 * sum of the unrounded p_j. causal != 0 masks keys j > i + Nk - Nq (a query with
 * no visible key gets 0). out: [B][Hq][Nq][128] FP32 or bf16. Products are
 * exact; sums are FP32 in the matrix units' order, so results agree with an
 * exact evaluation to FP32 accumulation error plus P codes that round the other
 * way near a midpoint. All arrays device memory; codes and out 16-byte aligned,
 * scales 8-byte aligned (NVFP4_EALIGN otherwise). */
NVFP4_API nvfp4_status nvfp4_attention(const uint8_t *q_codes, const uint8_t *q_scales,
                                       const float *q_gscale, const uint8_t *k_codes,
                                       const uint8_t *k_scales, const float *k_gscale,
                                       const uint8_t *v_codes, const uint8_t *v_scales,
                                       const float *v_gscale, int64_t B, int64_t Hq, int64_t Hkv,
                                       int64_t Nq, int64_t Nk, int64_t D, int causal, void *out,
                                       nvfp4_dtype out_dt, void *stream);

/* Attention over the attention-sink KV cache that nvfp4_kv_append maintains
 * (ScaleSearch summary page, ScaleSearchAttention: mixed-precision KV cache with
 * the first and last tokens in full precision). q as for nvfp4_attention. The K
 * and V caches each hold T tokens: token t < n_first in head[b][h][t] (bf16),
 * token t >= max(n_first, T - n_last) in the ring tail[b][h][t mod n_last]
 * (bf16), every other token coded at row t - n_first of codes[b][h][cap][64] /
 * scales[b][h][cap][8] under the tensor scale k_gscale / v_gscale. cache_dt must
 * be NVFP4_BF16; T - n_first - n_last <= cap. Every token is visible (no causal
 * mask). Keys are visited segment by segment (head, middle, tail, each in token
 * order) in tiles of 32 keys that never straddle two segments; otherwise as
 * nvfp4_attention: sink keys enter the products as their exact bf16 values, coded
 * keys as V[code] * s_block times the tensor scale. out: [B][Hq][Nq][128].
 * Codes, head, tail and out 16-byte aligned, scales 8-byte aligned. */
NVFP4_API nvfp4_status nvfp4_attention_kv_cache(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, nvfp4_dtype cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    int64_t T, int64_t D, int64_t n_first, int64_t n_last, int64_t cap, void *out,
    nvfp4_dtype out_dt, void *stream);

/* nvfp4_attention_kv_cache with the token count read from device memory
 * (length: device int64[1], 8-byte aligned, as nvfp4_kv_append_dev keeps it)
 * when the kernel runs, clamped to n_first + cap + n_last; for a decode step
 * captured in a HIP graph. The host checks that need T use the capacity
 * instead (head, tail, codes and scales must cover n_first + cap + n_last). */
NVFP4_API nvfp4_status nvfp4_attention_kv_cache_dev(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, nvfp4_dtype cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    const int64_t *length, int64_t D, int64_t n_first, int64_t n_last, int64_t cap, void *out,
    nvfp4_dtype out_dt, void *stream);

/* Cache attention with the keys split over workgroups, for decode steps with few
 * queries (ScaleSearch summary page, ScaleSearchAttention: the online softmax of
 * the attention on NVFP4 operands; the split is a reading of this library, as the
 * pages do not say how one query's keys are spread over parallel workers). The
 * keys fall into units: the head, the tail, and the middle cut into pieces of
 * `split` tokens from n_first (the last may be short). Each unit runs the online
 * softmax and the P coding of nvfp4_attention_kv_cache over its own keys, from its
 * own running max (P codes therefore differ from the unsplit call's); a second
 * kernel merges the unit states exactly: with M the largest running max and
 * w_u = exp(m_u - M), O = fl(1/2688) * sum w_u acc_u / sum w_u l_u. split > 0 and a
 * multiple of 32; at most 65535 units. workspace: device memory of at least
 * nvfp4_attention_split_workspace_bytes(B, Hq, Nq, cap, split) bytes, 16-byte
 * aligned, owned by the caller, overwritten by the call (calls sharing a workspace
 * must not overlap). Other arguments and errors as nvfp4_attention_kv_cache;
 * NVFP4_EWORKSPACE for a missing or short workspace. */
NVFP4_API nvfp4_status nvfp4_attention_kv_cache_split(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, nvfp4_dtype cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    int64_t T, int64_t D, int64_t n_first, int64_t n_last, int64_t cap, int64_t split,
    void *workspace, size_t workspace_bytes, void *out, nvfp4_dtype out_dt, void *stream);

/* nvfp4_attention_kv_cache_split with the token count read from device memory,
 * as nvfp4_attention_kv_cache_dev: the grid covers every unit of a full cache and
 * units past the tokens present contribute nothing, so one captured launch serves
 * every length. */
NVFP4_API nvfp4_status nvfp4_attention_kv_cache_split_dev(
    const uint8_t *q_codes, const uint8_t *q_scales, const float *q_gscale, const void *k_head,
    const void *k_tail, const uint8_t *k_codes, const uint8_t *k_scales, const float *k_gscale,
    const void *v_head, const void *v_tail, const uint8_t *v_codes, const uint8_t *v_scales,
    const float *v_gscale, nvfp4_dtype cache_dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
    const int64_t *length, int64_t D, int64_t n_first, int64_t n_last, int64_t cap, int64_t split,
    void *workspace, size_t workspace_bytes, void *out, nvfp4_dtype out_dt, void *stream);

/* Workspace bytes of the split cache attention for a cache of `cap` middle rows:
 * (2 + ceil(cap / split)) units x B * Hq * Nq rows x (128 + 2) FP32 values. 0 for
 * arguments the split calls reject (split not a positive multiple of 32, too many
 * units, sizes out of range). */
NVFP4_API size_t nvfp4_attention_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq,
                                                       int64_t cap, int64_t split);

/* Randomized Hadamard transform (QuIP#-style incoherence processing, ScaleSearch
 * summary page, ScaleSearchAttention section: a transform pair Q' = Q R^-T,
 * K' = K R that keeps Q K^T while lowering the mean-square absolute value).
 * Reading: R = diag(s) H / sqrt(128) per 128-vector with random signs s; R is
 * orthogonal, so R^-T = R and Q and K take the same transform (the same signs):
 * (Q R)(K R)^T = Q K^T. signs: host pointer to four uint32 words (read during
 * the call only); bit k % 32 of signs[k / 32] set negates feature k of every
 * 128-vector before H. The caller draws the signs (once per model or layer) and
 * must use the same words for Q and K. Each *_rht call is its namesake with
 * NVFP4_HADAMARD128 implied (other flags as there, bf16 input, cols % 128 == 0)
 * and x replaced by x o s; signs == NULL is NVFP4_EINVAL. All-zero signs give
 * exactly the plain-transform results. */
NVFP4_API nvfp4_status nvfp4_quantize_rht(const void *x, nvfp4_dtype xdt, int64_t rows,
                                          int64_t cols, int block, int f_lo, int f_hi,
                                          uint32_t flags, const uint32_t *signs, uint8_t *codes,
                                          uint8_t *scales, float *global_scale, void *workspace,
                                          size_t workspace_bytes, void *stream);
NVFP4_API nvfp4_status nvfp4_global_scale_rht(const void *x, nvfp4_dtype xdt, int64_t rows,
                                              int64_t cols, uint32_t flags, const uint32_t *signs,
                                              float *global_scale, void *workspace,
                                              size_t workspace_bytes, void *stream);
NVFP4_API nvfp4_status nvfp4_quantize_kv_sink_rht(const void *kv, nvfp4_dtype dt, int64_t B,
                                                  int64_t H, int64_t T, int64_t D,
                                                  int64_t n_first, int64_t n_last, int block,
                                                  int f_lo, int f_hi, uint32_t flags,
                                                  const uint32_t *signs, uint8_t *codes,
                                                  uint8_t *scales, float *global_scale,
                                                  void *sink, void *workspace,
                                                  size_t workspace_bytes, void *stream);
NVFP4_API nvfp4_status nvfp4_kv_append_rht(const void *kv_new, nvfp4_dtype dt, int64_t B,
                                           int64_t H, int64_t T, int64_t t_new, int64_t D,
                                           int64_t n_first, int64_t n_last, int64_t cap,
                                           int block, int f_lo, int f_hi, uint32_t flags,
                                           const uint32_t *signs, const float *global_scale,
                                           void *head, void *tail, uint8_t *codes,
                                           uint8_t *scales, void *stream);
NVFP4_API nvfp4_status nvfp4_hadamard128_rht(const void *x, nvfp4_dtype xdt, int64_t rows,
                                             const uint32_t *signs, float *y, void *stream);

/* ------------------------------------------------------------------------
 * The balancing pair of incoherence processing (ScaleSearch summary page,
 * ScaleSearchAttention, 非干渉処理（IP）と絶対値低減: besides the Hadamard
 * transform, an additional linear pair Q' = Q R^-T, K' = K R that keeps every
 * attention score and lowers the mean-square magnitude of the projected
 * tensors). The pages fix neither R nor how it is found. Reading taken:
 * R = diag(2^e) over the channels (columns), so Q'_tj = Q_tj 2^-e_j and
 * K'_tj = K_tj 2^e_j: each score term q_j k_j is kept exactly, and bf16 values
 * stay bf16 values. With the Hadamard transform the pair acts first:
 * Q' = Q diag(2^-e) H_s, K' = K diag(2^e) H_s (H_s orthogonal), so
 * Q' K'^T = Q K^T.
 * ------------------------------------------------------------------------ */

/* Workspace bytes of nvfp4_balance_exponents for `cols` channels (0 if cols
 * is outside 1..2048). */
NVFP4_API size_t nvfp4_balance_workspace_bytes(int64_t cols);

/* Calibration: channel exponents chan_exp[cols] (device int8) from a Q tensor
 * q[rows_q][cols] and a K tensor k[rows_k][cols] (device, dt, 16-byte
 * aligned; cols % 16 == 0, cols <= 2048). With a_j^2 and b_j^2 the channel's
 * sums of squares over Q's and K's rows (double), channel j's share of
 * ||Q'||^2 + ||K'||^2 is a^2 4^-e + b^2 4^e; e_j is the least e in [-16, 16]
 * with a^2 <= b^2 4^(2e+1) (the minimiser, ties to the smaller e; 16 if none),
 * 0 when a or b is 0. The sums are taken in a fixed order, so the result is
 * deterministic; a channel whose a^2 / b^2 lies within double rounding of a
 * decision boundary may differ from another summation order's choice (either
 * is a minimiser). Workspace: nvfp4_balance_workspace_bytes(cols), 8-byte
 * aligned, caller-owned. NVFP4_ESHAPE for a size outside those limits. */
NVFP4_API nvfp4_status nvfp4_balance_exponents(const void *q, const void *k, nvfp4_dtype dt,
                                               int64_t rows_q, int64_t rows_k, int64_t cols,
                                               int8_t *chan_exp, void *workspace,
                                               size_t workspace_bytes, void *stream);

/* nvfp4_quantize of one side of the pair: x' = x 2^(side e_col) with side -1
 * under NVFP4_PAIR_Q (the Q side) and +1 otherwise (K), chan_exp[cols] device
 * int8, 16-byte aligned, each clamped to [-32, 32]. Without
 * NVFP4_HADAMARD128, x' is formed in binary32 (exact unless it leaves the
 * normal range) and quantized as FP32 values (the exact search: slower than
 * the bf16 certified search). With NVFP4_HADAMARD128 (bf16 input, cols ==
 * 128) the transform is applied to x' (its products stay exact: the factors
 * 2^e ride in the transform's matrix operand), with the random signs when
 * `signs` (host uint32[4], as in nvfp4_quantize_rht) is not NULL; `signs`
 * without the transform flag is NVFP4_EINVAL. Outputs, tensor scale and
 * workspace as nvfp4_quantize; the codes are those of x' (dequantize returns
 * x'-domain values, whose products with the other side's keep the scores). */
NVFP4_API nvfp4_status nvfp4_quantize_balanced(const void *x, nvfp4_dtype xdt, int64_t rows,
                                               int64_t cols, int block, int f_lo, int f_hi,
                                               uint32_t flags, const int8_t *chan_exp,
                                               const uint32_t *signs, uint8_t *codes,
                                               uint8_t *scales, float *global_scale,
                                               void *workspace, size_t workspace_bytes,
                                               void *stream);

/* The transform alone on one side of the pair: y[rows][128] (FP32) =
 * (x diag(2^(side e)) o s) H / sqrt(128) for bf16 x[rows][128] (side as in
 * nvfp4_quantize_balanced from NVFP4_PAIR_Q in flags; signs optional). */
NVFP4_API nvfp4_status nvfp4_hadamard128_balanced(const void *x, nvfp4_dtype xdt, int64_t rows,
                                                  const int8_t *chan_exp, uint32_t flags,
                                                  const uint32_t *signs, float *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
