/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for NVFP4 block quantization with
 * ScaleSearch.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. The product path (the HIP
 * library and its Python binding) never calls, links or imports it, and this
 * file shares no code, header, table or helper with the product.
 *
 * Sources (web pages; cited by title and section):
 *  [SS]  "技術サマリー：ブロック浮動小数点スケールを検索せよ！" (gist.science summary
 *        of the ScaleSearch paper), section 手法 > ScaleSearch: the max-scaling
 *        default s = round(amax/6), the offset rule s(f) = reinterpret(
 *        reinterpret(s, int8) + f, UE4M3) (メカニズム), the exhaustive search of
 *        a small offset range for the least block MSE (検索戦略), and the
 *        bimodal optimum (根拠).
 *  [SSA] same page, ScaleSearchAttention: Hadamard incoherence processing
 *        (非干渉処理（IP）と絶対値低減) and the attention-sink cache that keeps the
 *        first and last KV blocks at full precision (アテンション・シンク対応混合精度
 *        キャッシング).
 *  [NV]  "NVIDIAのFP4推論が50倍の効率を実現", section 超低精度推論を支えるアーキテクチャ:
 *        E2M1 elements, one E4M3 scale per 16-value micro-block, and a second
 *        FP32 per-tensor scale.
 *  [BEV] "自動運転モデル BEVFormer の NVIDIA Blackwell B200 FP8/FP4 CUDAカーネル・
 *        チューニング", sections 7 and 1-A/1-B: e4m3 = 1 sign/4 exponent/3 mantissa
 *        bits, e2m1 = 1/2/1 bits, FP8 range max/448 and FP4 range max/6, two FP4
 *        values packed per byte.
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 *
 * Arithmetic: every float operation below is one IEEE-754 binary32 operation
 * rounded to nearest-even (x86-64 SSE, FLT_EVAL_METHOD == 0). The file must be
 * built with -ffp-contract=off and without -ffast-math, so that no product and
 * sum are fused. Subnormals are kept.
 *
 * Parity status: every function here is pinned by the CPU tests (closed forms,
 * a hand-derived worked example, invariants, an independent NumPy brute force
 * and published statistics of the offset optimum). The Hadamard transform is
 * pinned against closed forms and a library Hadamard matrix.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* dtype tags used by the oracle's own entry points */
#define ORACLE_F32 0
#define ORACLE_BF16 1

/* ------------------------------------------------------------------------ */
/* Element format: E2M1 ([BEV] 1-A/1-B, [NV]).                              */
/* 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit. The non-negative   */
/* values, by magnitude code 0..7, are 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, */
/* 6; 6 is the largest, as the default scale amax/6 of [SS] implies.       */
/* ------------------------------------------------------------------------ */
static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* Magnitude code of y >= 0: the nearest grid value; a value exactly halfway
 * between two grid values takes the even code (round-to-nearest-even of the
 * format, whose mantissa LSB is the code LSB); anything above 6, +Inf
 * included, saturates to code 7. Returns -1 for NaN or negative input. */
int oracle_e2m1_code(float y)
{
    if (!(y >= 0.0f))
        return -1;
    int c = 0;
    for (int k = 0; k < 7; ++k) {
        /* midpoint of two neighbouring grid values: exact in double */
        double mid = 0.5 * ((double)E2M1_MAG[k] + (double)E2M1_MAG[k + 1]);
        double yy = (double)y;
        int up = (yy > mid) || (yy == mid && ((k + 1) % 2 == 0));
        if (!up)
            break;
        c = k + 1;
    }
    return c;
}

float oracle_e2m1_value(int code)
{
    float m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* ------------------------------------------------------------------------ */
/* Block-scale format: unsigned E4M3 ([BEV] 1-A: 4 exponent bits, 3        */
/* mantissa bits, bias 7; [BEV] sec. 7: largest value 448). The sign bit is */
/* unused (the scale is non-negative), so a scale is a pattern p in 0..127; */
/* 127 (exponent and mantissa all ones) is NaN and never a scale.           */
/* ------------------------------------------------------------------------ */
float oracle_e4m3_value(int p)
{
    if (p < 0 || p >= 127)
        return NAN;
    int e = p >> 3, m = p & 7;
    if (e == 0)
        return (float)ldexp((double)m, -9); /* subnormal: m * 2^-9 */
    return (float)ldexp(1.0 + m / 8.0, e - 7);
}

/* Round t >= 0 to the nearest E4M3 value (ties to the even pattern, i.e.
 * even mantissa), saturating at 448 (pattern 126). Reading: the pages write
 * "round" in s = round(amax/6); round-to-nearest-even with saturation is the
 * plain meaning for a float format with no infinity. -1 for NaN/negative. */
int oracle_e4m3_encode(float t)
{
    if (!(t >= 0.0f))
        return -1;
    if (t >= 448.0f)
        return 126;
    /* values grow with the pattern, so binary search the largest p with
     * value(p) <= t */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if ((double)oracle_e4m3_value(mid) <= (double)t)
            lo = mid;
        else
            hi = mid - 1;
    }
    int p = lo; /* p <= 125 because t < 448 */
    double below = oracle_e4m3_value(p), above = oracle_e4m3_value(p + 1);
    double mid = 0.5 * (below + above); /* exact in double */
    if ((double)t > mid)
        return p + 1;
    if ((double)t < mid)
        return p;
    return (p % 2 == 0) ? p : p + 1;
}

/* ------------------------------------------------------------------------ */
/* Input access.                                                            */
/* ------------------------------------------------------------------------ */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float load_elem(const void *x, int dtype, int64_t i)
{
    if (dtype == ORACLE_BF16)
        return bf16_bits_to_float(((const uint16_t *)x)[i]);
    return ((const float *)x)[i];
}

static uint32_t float_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* ------------------------------------------------------------------------ */
/* Global scale. [NV]: a second, FP32 per-tensor scale sets the global      */
/* range. Reading (the [SS] formula has no tensor scale): the tensor scale  */
/* is a decode scale S_g = A / (6 * 448), A = max |x| over the quantized    */
/* region, so that the block scale t = (amax_b / 6) / S_g of the largest    */
/* block lands on the largest E4M3 value 448; reconstruction is             */
/* x ~ V[code] * s_block * S_g. S_g = 0 (all-zero region or underflow)      */
/* becomes 1.                                                               */
/* ------------------------------------------------------------------------ */
static float global_scale_from_amax(float A)
{
    float sg = A / 2688.0f; /* 2688 = 6 * 448 */
    if (sg == 0.0f)
        sg = 1.0f;
    return sg;
}

/* ------------------------------------------------------------------------ */
/* One 16-element block ([NV]: 16-value micro-block; [SS]: ScaleSearch).    */
/* ------------------------------------------------------------------------ */

/* Squared error of coding the 16 magnitudes ax[] with block-scale pattern p
 * under tensor scale sg, as the sum of squared differences between each
 * element and its reconstruction, added strictly left to right in FP32
 * (the search ranks candidates by MSE = this / 16, [SS] 検索戦略).
 * Reading: the quantizer multiplies by the encode scale r = 1/d of the
 * candidate's decode scale d = s_p * S_g; a candidate whose r is not finite
 * (p = 0, or d so small that 1/d overflows) codes every element as 0. */
static float block_sse(const float ax[16], int p, float sg, uint8_t mag_codes[16])
{
    float s = oracle_e4m3_value(p);
    float d = s * sg;
    float r = 1.0f / d;
    int zero = !isfinite(r);
    float sse = 0.0f;
    for (int i = 0; i < 16; ++i) {
        int c;
        float xhat;
        if (zero) {
            c = 0;
            xhat = 0.0f;
        } else {
            float y = ax[i] * r;
            c = oracle_e2m1_code(y);
            xhat = E2M1_MAG[c] * d;
        }
        float e = ax[i] - xhat;
        float q = e * e;
        sse = (i == 0) ? q : sse + q;
        if (mag_codes)
            mag_codes[i] = (uint8_t)c;
    }
    return sse;
}

float oracle_block_sse(const float x[16], float sg, int p)
{
    float ax[16];
    for (int i = 0; i < 16; ++i)
        ax[i] = fabsf(x[i]);
    if (p < 0 || p > 126)
        return NAN;
    return block_sse(ax, p, sg, NULL);
}

/* Default pattern of a block ([SS] メカニズム: s = round(amax / 6)), in units
 * of the tensor scale: t = (a_b / 6) / S_g, each division rounded once. */
static int default_pattern(float amax_b, float sg)
{
    float t = (amax_b / 6.0f) / sg;
    return oracle_e4m3_encode(t);
}

/* ScaleSearch on one block. x[16] is the block (signed), sg a positive
 * finite tensor scale. Writes 8 code bytes and returns the scale pattern.
 * The candidates are the E4M3 patterns p0 + f for integer f in [f_lo, f_hi]
 * ([SS] メカニズム: the offset is added to the scale's bit pattern, so p0 + f
 * is the f-th neighbouring representable scale). f = 0 is visited first,
 * then f_lo, f_lo+1, ..., f_hi; a pattern outside 0..126 is skipped (the
 * int8 reinterpretation would flip the sign or give NaN); the first visited
 * candidate with strictly smaller squared error wins, so ties keep f = 0 and
 * then the lowest f. */
static int search_block(const float x[16], float sg, int f_lo, int f_hi,
                        uint8_t codes[8], int *chosen_f)
{
    float ax[16];
    float amax_b = 0.0f;
    for (int i = 0; i < 16; ++i) {
        ax[i] = fabsf(x[i]);
        if (ax[i] > amax_b)
            amax_b = ax[i];
    }
    int p0 = default_pattern(amax_b, sg);

    int best_p = p0, best_f = 0;
    uint8_t best_mag[16];
    float best_sse = block_sse(ax, p0, sg, best_mag);
    for (int f = f_lo; f <= f_hi; ++f) {
        if (f == 0)
            continue;
        int p = p0 + f;
        if (p < 0 || p > 126)
            continue;
        uint8_t mag[16];
        float sse = block_sse(ax, p, sg, mag);
        if (sse < best_sse) {
            best_sse = sse;
            best_p = p;
            best_f = f;
            memcpy(best_mag, mag, 16);
        }
    }
    /* Codes: a nibble is sign << 3 | magnitude code (E2M1 sign-magnitude),
     * the sign copied from the input even for a zero code. Reading: two
     * nibbles per byte with the even element in the low nibble. */
    for (int j = 0; j < 8; ++j) {
        uint8_t n0 = (uint8_t)((signbit(x[2 * j]) ? 8 : 0) | best_mag[2 * j]);
        uint8_t n1 = (uint8_t)((signbit(x[2 * j + 1]) ? 8 : 0) | best_mag[2 * j + 1]);
        codes[j] = (uint8_t)(n0 | (n1 << 4));
    }
    if (chosen_f)
        *chosen_f = best_f;
    return best_p;
}

/* ------------------------------------------------------------------------ */
/* Threads: a static partition of block rows; every block is computed the   */
/* same way whatever the thread count, so results do not depend on it.      */
/* ------------------------------------------------------------------------ */
typedef struct {
    const void *x;
    int dtype;
    int64_t rows, cols, r0, r1;
    int f_lo, f_hi;
    float sg;
    int sg_ok;
    uint8_t *codes, *scales;
    int8_t *chosen_f;
} qjob_t;

static void quantize_rows(const qjob_t *J)
{
    int64_t nb = J->cols / 16;
    for (int64_t r = J->r0; r < J->r1; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            float x[16];
            int finite = 1;
            for (int i = 0; i < 16; ++i) {
                x[i] = load_elem(J->x, J->dtype, r * J->cols + b * 16 + i);
                if (!isfinite(x[i]))
                    finite = 0;
            }
            uint8_t *cb = J->codes + r * (J->cols / 2) + b * 8;
            uint8_t *sb = J->scales + r * nb + b;
            int fsel = 0;
            if (!J->sg_ok || !finite) {
                /* non-finite contract: scale NaN pattern, codes zero */
                memset(cb, 0, 8);
                *sb = 0x7F;
            } else {
                *sb = (uint8_t)search_block(x, J->sg, J->f_lo, J->f_hi, cb, &fsel);
            }
            if (J->chosen_f)
                J->chosen_f[r * nb + b] = (int8_t)fsel;
        }
    }
}

static void *quantize_thread(void *arg)
{
    quantize_rows((const qjob_t *)arg);
    return NULL;
}

static int run_quantize_rows(qjob_t base, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads == 1 || base.rows < 2) {
        base.r0 = 0;
        base.r1 = base.rows;
        quantize_rows(&base);
        return ORACLE_OK;
    }
    pthread_t th[256];
    int running[256];
    qjob_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].r0 = base.rows * t / nthreads;
        jobs[t].r1 = base.rows * (t + 1) / nthreads;
        running[t] = pthread_create(&th[t], NULL, quantize_thread, &jobs[t]) == 0;
        if (!running[t])
            quantize_rows(&jobs[t]); /* could not start a thread: do it here */
    }
    for (int t = 0; t < nthreads; ++t)
        if (running[t])
            pthread_join(th[t], NULL);
    return ORACLE_OK;
}

/* Global amax A = max |x| over the region, as the largest absolute-value
 * bit pattern (exact and order-free). Returns 0 if a NaN/Inf was seen. */
static int region_amax(const void *x, int dtype, int64_t n, float *A)
{
    uint32_t best = 0;
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = float_bits(load_elem(x, dtype, i)) & 0x7FFFFFFFu;
        if (u > best)
            best = u;
    }
    float a;
    memcpy(&a, &best, 4);
    *A = a;
    return best < 0x7F800000u;
}

/* ------------------------------------------------------------------------ */
/* Hadamard pre-transform ([SSA] 非干渉処理: a Hadamard transform as in      */
/* QuIP#). Reading: per contiguous 128-vector, y = x * H / sqrt(128) with H */
/* the 128 x 128 Sylvester matrix in natural order (H[j][k] = (-1)^popcount */
/* (j & k)), no random signs. The sum is taken in double in natural order   */
/* (exact while the 128 inputs span less than about 2^38 in magnitude),     */
/* multiplied by the double nearest 1/sqrt(128), then rounded to binary32.   */
/* ------------------------------------------------------------------------ */
static int popcount_parity(unsigned v)
{
    int p = 0;
    while (v) {
        p ^= 1;
        v &= v - 1;
    }
    return p;
}

typedef struct {
    const void *x;
    int dtype;
    int64_t v0, v1;
    float *y;
    const uint32_t *signs; /* NULL, or 128 bits: bit k set negates input feature k */
    const int8_t *bal;     /* NULL, or the channel exponents of the balancing pair */
    int bal_sign;          /* +1 or -1: the side of the pair */
    int64_t cols;          /* row length (channels), with bal */
} hjob_t;

/* The Sylvester matrix, entry by entry from its definition; filled before any
 * worker thread starts, read-only afterwards. */
static double H[128][128];

static void fill_hadamard(void)
{
    for (int j = 0; j < 128; ++j)
        for (int k = 0; k < 128; ++k)
            H[j][k] = popcount_parity((unsigned)(j & k)) ? -1.0 : 1.0;
}

static void hadamard_vectors(const hjob_t *J)
{
    const double c = sqrt(1.0 / 128.0); /* correctly rounded 2^-3.5 */
    for (int64_t v = J->v0; v < J->v1; ++v) {
        double in[128];
        for (int k = 0; k < 128; ++k) {
            in[k] = (double)load_elem(J->x, J->dtype, v * 128 + k);
            if (J->bal) /* exact: a power of two times a binary32 value, in double */
                in[k] = ldexp(in[k], J->bal_sign * J->bal[(v * 128 + k) % J->cols]);
            if (J->signs && ((J->signs[k >> 5] >> (k & 31)) & 1u))
                in[k] = -in[k];
        }
        for (int j = 0; j < 128; ++j) {
            double s = 0.0;
            for (int k = 0; k < 128; ++k)
                s += H[j][k] * in[k];
            J->y[v * 128 + j] = (float)(s * c);
        }
    }
}

static void *hadamard_thread(void *arg)
{
    hadamard_vectors((const hjob_t *)arg);
    return NULL;
}

static int hadamard_threads_bal(const void *x, int dtype, int64_t nvec, float *y, int nthreads,
                                const uint32_t *signs, const int8_t *bal, int bal_sign,
                                int64_t cols);

static int hadamard_threads(const void *x, int dtype, int64_t nvec, float *y, int nthreads,
                            const uint32_t *signs)
{
    return hadamard_threads_bal(x, dtype, nvec, y, nthreads, signs, NULL, 1, 128);
}

static int hadamard_threads_bal(const void *x, int dtype, int64_t nvec, float *y, int nthreads,
                                const uint32_t *signs, const int8_t *bal, int bal_sign,
                                int64_t cols)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    int running[256];
    hjob_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].x = x;
        jobs[t].dtype = dtype;
        jobs[t].y = y;
        jobs[t].v0 = nvec * t / nthreads;
        jobs[t].v1 = nvec * (t + 1) / nthreads;
        jobs[t].signs = signs;
        jobs[t].bal = bal;
        jobs[t].bal_sign = bal_sign;
        jobs[t].cols = cols;
    }
    fill_hadamard();
    for (int t = 0; t < nthreads; ++t) {
        running[t] = pthread_create(&th[t], NULL, hadamard_thread, &jobs[t]) == 0;
        if (!running[t])
            hadamard_vectors(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (running[t])
            pthread_join(th[t], NULL);
    return ORACLE_OK;
}

int oracle_hadamard128(const void *x, int dtype, int64_t nvec, float *y, int nthreads)
{
    if (!x || !y || nvec < 0 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    return hadamard_threads(x, dtype, nvec, y, nthreads, NULL);
}

/* Randomized Hadamard transform (QuIP#-style incoherence processing): each
 * 128-vector has the features whose bit is set in signs[4] negated, then is
 * transformed as above: y = (x o s) H / sqrt(128). The random signs are an
 * input (the caller draws them). */
int oracle_hadamard128_rht(const void *x, int dtype, int64_t nvec, const uint32_t *signs, float *y,
                           int nthreads)
{
    if (!x || !y || !signs || nvec < 0 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    return hadamard_threads(x, dtype, nvec, y, nthreads, signs);
}

/* ------------------------------------------------------------------------ */
/* Entry points.                                                            */
/* ------------------------------------------------------------------------ */

/* Quantize a contiguous rows x cols tensor (blocks of 16 along the last
 * dimension). If gscale_given, *gscale is read as the tensor scale (it must be
 * positive and finite, else every block gets the non-finite contract);
 * otherwise it is computed from the global amax and written. A NaN/Inf in the
 * region (computed mode) gives S_g = NaN and every block scale 0x7F with zero
 * codes; in given mode only the blocks holding a NaN/Inf get that. hadamard:
 * transform each 128-vector first (cols % 128 == 0) and quantize the FP32
 * result. chosen_f (nullable) receives the winning offset per block. */
int oracle_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int f_lo,
                    int f_hi, int hadamard, int gscale_given, float *gscale,
                    uint8_t *codes, uint8_t *scales, int8_t *chosen_f, int nthreads)
{
    if (!x || !gscale || !codes || !scales || rows < 0 || cols <= 0 || cols % 16 ||
        f_lo > 0 || f_hi < 0 || f_lo < -126 || f_hi > 126 ||
        (dtype != ORACLE_F32 && dtype != ORACLE_BF16) || (hadamard && cols % 128))
        return ORACLE_EINVAL;
    const void *src = x;
    int sdt = dtype;
    float *ybuf = NULL;
    int64_t n = rows * cols;
    if (hadamard) {
        ybuf = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
        if (!ybuf)
            return ORACLE_ENOMEM;
        hadamard_threads(x, dtype, n / 128, ybuf, nthreads, NULL);
        src = ybuf;
        sdt = ORACLE_F32;
    }
    float sg;
    int sg_ok;
    if (gscale_given) {
        sg = *gscale;
        sg_ok = (sg > 0.0f) && isfinite(sg);
    } else {
        float A;
        int finite = region_amax(src, sdt, n, &A);
        if (finite) {
            sg = global_scale_from_amax(A);
            sg_ok = 1;
        } else {
            sg = NAN;
            sg_ok = 0;
        }
        *gscale = sg;
    }
    qjob_t J;
    memset(&J, 0, sizeof J);
    J.x = src;
    J.dtype = sdt;
    J.rows = rows;
    J.cols = cols;
    J.f_lo = f_lo;
    J.f_hi = f_hi;
    J.sg = sg;
    J.sg_ok = sg_ok;
    J.codes = codes;
    J.scales = scales;
    J.chosen_f = chosen_f;
    int rc = run_quantize_rows(J, nthreads);
    free(ybuf);
    return rc;
}

/* Quantize after the randomized Hadamard transform with the given signs. */
int oracle_quantize_rht(const void *x, int dtype, int64_t rows, int64_t cols, const uint32_t *signs,
                        int f_lo, int f_hi, int gscale_given, float *gscale, uint8_t *codes,
                        uint8_t *scales, int nthreads)
{
    if (!x || !signs || rows < 0 || cols <= 0 || cols % 128 ||
        (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    int64_t n = rows * cols;
    float *ybuf = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!ybuf)
        return ORACLE_ENOMEM;
    hadamard_threads(x, dtype, n / 128, ybuf, nthreads, signs);
    int rc = oracle_quantize(ybuf, ORACLE_F32, rows, cols, f_lo, f_hi, 0, gscale_given, gscale,
                             codes, scales, NULL, nthreads);
    free(ybuf);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* The additional transform pair of [SSA] 非干渉処理（IP）と絶対値低減: a pair  */
/* Q' = Q R^-T, K' = K R keeps every score of QK^T and lowers the mean-     */
/* square magnitude of the projected tensors. The pages fix neither R nor   */
/* how it is found. Reading: R is diagonal over the channels (the columns)  */
/* with power-of-two entries, R = diag(2^e_j): then Q'_tj = Q_tj 2^-e_j and */
/* K'_tj = K_tj 2^e_j, each score term is unchanged exactly, even in binary  */
/* floating point, and a bf16 operand stays a bf16 value. With the Hadamard */
/* transform the pair acts first, R_total = diag(2^e) H_s, so that           */
/* (Q D^-1 H_s)(K D H_s)^T = Q K^T for the orthogonal H_s.                   */
/* Calibration from a Q and a K tensor: a_j^2 = sum_t Q_tj^2 and b_j^2 =     */
/* sum_t K_tj^2 (double, rows in order); channel j's share of ||Q'||^2 +     */
/* ||K'||^2 is f(e) = a^2 4^-e + b^2 4^e, convex in e, and f(e) <= f(e + 1)  */
/* exactly when a^2 <= b^2 4^(2e+1); e_j is the least e in [-16, 16] with    */
/* that property (16 if none), so ties go to the smaller e; a channel with   */
/* a or b zero keeps e_j = 0.                                                */
/* ------------------------------------------------------------------------ */
static void column_sumsq(const void *x, int dtype, int64_t rows, int64_t cols, double *out)
{
    for (int64_t j = 0; j < cols; ++j)
        out[j] = 0.0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) {
            double v = (double)load_elem(x, dtype, r * cols + j);
            out[j] += v * v;
        }
}

int oracle_balance_exponent(double a2, double b2)
{
    if (!(a2 > 0.0) || !(b2 > 0.0))
        return 0;
    for (int e = -16; e <= 15; ++e)
        if (a2 <= ldexp(b2, 2 * (2 * e + 1)))
            return e;
    return 16;
}

int oracle_balance_exponents(const void *q, const void *k, int dtype, int64_t rows_q,
                             int64_t rows_k, int64_t cols, int8_t *e_out)
{
    if (!q || !k || !e_out || rows_q < 0 || rows_k < 0 || cols <= 0 ||
        (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    double *a2 = malloc(sizeof(double) * (size_t)cols), *b2 = malloc(sizeof(double) * (size_t)cols);
    if (!a2 || !b2) {
        free(a2);
        free(b2);
        return ORACLE_ENOMEM;
    }
    column_sumsq(q, dtype, rows_q, cols, a2);
    column_sumsq(k, dtype, rows_k, cols, b2);
    for (int64_t j = 0; j < cols; ++j)
        e_out[j] = (int8_t)oracle_balance_exponent(a2[j], b2[j]);
    free(a2);
    free(b2);
    return ORACLE_OK;
}

/* Quantize one side of the pair: x'_tj = x_tj 2^(side e_j) (side = -1 for Q,
 * +1 for K; e_j clamped to [-32, 32]), then the quantizer. Without the Hadamard transform x' is formed
 * in binary32 (exact unless it leaves the normal range) and quantized as FP32
 * values; with it (hadamard, signs optional for the randomized transform),
 * the scaled values enter the transform's double sum exactly. */
int oracle_quantize_balanced(const void *x, int dtype, int64_t rows, int64_t cols,
                             const int8_t *e, int side, int hadamard, const uint32_t *signs,
                             int f_lo, int f_hi, int gscale_given, float *gscale,
                             uint8_t *codes, uint8_t *scales, int nthreads)
{
    if (!x || !e || (side != 1 && side != -1) || rows < 0 || cols <= 0 || cols % 16 ||
        (hadamard && cols % 128) || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    int8_t *ec = malloc((size_t)cols);
    if (!ec)
        return ORACLE_ENOMEM;
    for (int64_t j = 0; j < cols; ++j) /* the exponents are clamped to [-32, 32] */
        ec[j] = (int8_t)(e[j] < -32 ? -32 : (e[j] > 32 ? 32 : e[j]));
    e = ec;
    int64_t n = rows * cols;
    float *ybuf = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!ybuf) {
        free(ec);
        return ORACLE_ENOMEM;
    }
    if (hadamard) {
        hadamard_threads_bal(x, dtype, n / 128, ybuf, nthreads, signs, e, side, cols);
    } else {
        for (int64_t i = 0; i < n; ++i)
            ybuf[i] = ldexpf(load_elem(x, dtype, i), side * e[i % cols]);
    }
    int rc = oracle_quantize(ybuf, ORACLE_F32, rows, cols, f_lo, f_hi, 0, gscale_given, gscale,
                             codes, scales, NULL, nthreads);
    free(ybuf);
    free(ec);
    return rc;
}

/* The transform alone (inspection and split parity): y = (x D^side o s) H /
 * sqrt(128) per 128-vector, D = diag(2^e) over the row's cols channels. */
int oracle_hadamard128_balanced(const void *x, int dtype, int64_t rows, int64_t cols,
                                const int8_t *e, int side, const uint32_t *signs, float *y,
                                int nthreads)
{
    if (!x || !y || !e || (side != 1 && side != -1) || rows < 0 || cols <= 0 || cols % 128 ||
        (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    return hadamard_threads_bal(x, dtype, rows * cols / 128, y, nthreads, signs, e, side, cols);
}

/* Round binary32 to bfloat16, nearest-even (NaN -> quiet NaN, sign kept). */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u = float_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* Dequantize: x^ = (-1)^sign * (V[code] * (s_p * S_g)), the product of the
 * block's decode scale and the grid value rounded once each, the same value
 * the search scored. A scale byte >= 127 decodes as NaN. out_dtype 0: FP32,
 * 1: bf16 (nearest-even of the FP32 value). */
int oracle_dequantize(const uint8_t *codes, const uint8_t *scales, float gscale,
                      int64_t rows, int64_t cols, int out_dtype, void *y)
{
    if (!codes || !scales || !y || rows < 0 || cols <= 0 || cols % 16 ||
        (out_dtype != ORACLE_F32 && out_dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    int64_t nb = cols / 16;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            int p = scales[r * nb + b];
            float d = oracle_e4m3_value(p) * gscale;
            for (int i = 0; i < 16; ++i) {
                int64_t e = r * cols + b * 16 + i;
                uint8_t byte = codes[e / 2];
                int nib = (e % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                float v = E2M1_MAG[nib & 7] * d;
                if (nib & 8)
                    v = -v;
                if (out_dtype == ORACLE_F32)
                    ((float *)y)[e] = v;
                else
                    ((uint16_t *)y)[e] = float_to_bf16_rne(v);
            }
        }
    }
    return ORACLE_OK;
}

/* Attention-sink KV mode ([SSA] アテンション・シンク対応混合精度キャッシング).
 * kv is [B, H, T, D] contiguous (blocks of 16 along D). For each (b, h), the
 * first n_first and last n_last tokens are kept verbatim in sink[B, H,
 * n_first + n_last, D] (first, then last; same dtype as kv), and the middle
 * T - n_first - n_last tokens are quantized as one region: the global amax is
 * taken over the middle tokens only (reading: sink tokens are not coded, so
 * they do not set the range). codes[B, H, Tm, D/2], scales[B, H, Tm, D/16]. */
int oracle_quantize_kv_sink(const void *kv, int dtype, int64_t B, int64_t H, int64_t T,
                            int64_t D, int64_t n_first, int64_t n_last, int f_lo,
                            int f_hi, int hadamard, int gscale_given, float *gscale,
                            uint8_t *codes, uint8_t *scales, void *sink, int nthreads)
{
    if (!kv || !sink || B < 0 || H < 0 || T < 0 || D <= 0 || n_first < 0 || n_last < 0 ||
        n_first + n_last > T || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    size_t es = dtype == ORACLE_BF16 ? 2 : 4;
    int64_t Tm = T - n_first - n_last, NS = n_first + n_last;
    int64_t BH = B * H;
    unsigned char *mid = (unsigned char *)malloc((size_t)(BH * Tm * D > 0 ? BH * Tm * D : 1) * es);
    if (!mid)
        return ORACLE_ENOMEM;
    const unsigned char *src = (const unsigned char *)kv;
    unsigned char *snk = (unsigned char *)sink;
    for (int64_t g = 0; g < BH; ++g) {
        const unsigned char *base = src + (size_t)(g * T * D) * es;
        memcpy(snk + (size_t)(g * NS * D) * es, base, (size_t)(n_first * D) * es);
        memcpy(snk + (size_t)((g * NS + n_first) * D) * es,
               base + (size_t)((T - n_last) * D) * es, (size_t)(n_last * D) * es);
        memcpy(mid + (size_t)(g * Tm * D) * es, base + (size_t)(n_first * D) * es,
               (size_t)(Tm * D) * es);
    }
    int rc = oracle_quantize(mid, dtype, BH * Tm, D, f_lo, f_hi, hadamard, gscale_given,
                             gscale, codes, scales, NULL, nthreads);
    free(mid);
    return rc;
}

/* Inverse of the sink mode: y[B, H, T, D] with the sink tokens copied exactly
 * (converted to out_dtype; bf16 -> FP32 is exact) and the middle dequantized. */
int oracle_dequantize_kv_sink(const uint8_t *codes, const uint8_t *scales, float gscale,
                              const void *sink, int sink_dtype, int64_t B, int64_t H,
                              int64_t T, int64_t D, int64_t n_first, int64_t n_last,
                              int out_dtype, void *y)
{
    if (!codes || !scales || !sink || !y || n_first < 0 || n_last < 0 || n_first + n_last > T ||
        D <= 0 || D % 16)
        return ORACLE_EINVAL;
    int64_t Tm = T - n_first - n_last, NS = n_first + n_last, BH = B * H;
    size_t os = out_dtype == ORACLE_BF16 ? 2 : 4;
    void *mid = malloc((size_t)(BH * Tm * D > 0 ? BH * Tm * D : 1) * os);
    if (!mid)
        return ORACLE_ENOMEM;
    int rc = oracle_dequantize(codes, scales, gscale, BH * Tm, D, out_dtype, mid);
    if (rc) {
        free(mid);
        return rc;
    }
    for (int64_t g = 0; g < BH; ++g) {
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t k = 0; k < D; ++k) {
                float v;
                int from_mid = 0;
                int64_t mi = 0;
                if (t < n_first)
                    v = load_elem(sink, sink_dtype, (g * NS + t) * D + k);
                else if (t >= T - n_last)
                    v = load_elem(sink, sink_dtype, (g * NS + n_first + (t - (T - n_last))) * D + k);
                else {
                    from_mid = 1;
                    mi = (g * Tm + (t - n_first)) * D + k;
                    v = 0.0f;
                }
                int64_t o = (g * T + t) * D + k;
                if (from_mid) {
                    if (out_dtype == ORACLE_F32)
                        ((float *)y)[o] = ((float *)mid)[mi];
                    else
                        ((uint16_t *)y)[o] = ((uint16_t *)mid)[mi];
                } else {
                    if (out_dtype == ORACLE_F32)
                        ((float *)y)[o] = v;
                    else
                        ((uint16_t *)y)[o] = float_to_bf16_rne(v);
                }
            }
        }
    }
    free(mid);
    return rc;
}

int oracle_abi_version(void) { return 1; }

/* Batched codec helpers for the exhaustive codec tests. */
void oracle_e2m1_code_batch(const float *y, int64_t n, int8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (int8_t)oracle_e2m1_code(y[i]);
}

void oracle_e4m3_encode_batch(const float *t, int64_t n, int16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (int16_t)oracle_e4m3_encode(t[i]);
}

/* ======================================================================== */
/* MXFP4, the power-of-two contrast format ([NV]: NVFP4's E4M3 block scale   */
/* and FP32 tensor scale are set against MXFP4's plain power-of-two          */
/* scaling). The pages define MXFP4 no further; reading (the published OCP   */
/* Microscaling v1.0 format): blocks of 32 consecutive elements share one    */
/* E8M0 scale byte b = X + 127 standing for 2^X (X in -127..127; 255 is     */
/* NaN); elements are E2M1 codes as above; there is no tensor scale. The     */
/* spec's scale rule is X = floor(log2 amax) - 2 (2 = the exponent of E2M1's */
/* largest value, 6 = 1.5 * 2^2), clamped to -127; an all-zero block takes   */
/* X = -127. Elements are coded as y = |x| * 2^-X, nearest-even, saturating  */
/* at 6 (so a block amax in (6, 8) * 2^X clips). ScaleSearch carried over:   */
/* candidates X + f, f in [f_lo, f_hi] (an E8M0 pattern step doubles the     */
/* scale), ranked by the same left-to-right FP32 squared error over the 32   */
/* elements, f = 0 first, first strictly smaller wins; X + f outside         */
/* -127..127 is skipped. [0, 0] is the plain OCP conversion.                 */
/* ======================================================================== */

/* floor(log2 a) for finite a > 0: a = m * 2^e with m in [0.5, 1). */
static int floor_log2(float a)
{
    int e;
    frexpf(a, &e);
    return e - 1;
}

/* Squared error of coding the 32 magnitudes ax[] with scale 2^X. Both 2^X and
 * 2^-X are exact binary32 values for X in -127..127, and every reconstruction
 * V * 2^X (V an E2M1 value, at least 0.5 unless 0) is exact. */
static float mx_block_sse(const float ax[32], int X, uint8_t mag_codes[32])
{
    float d = ldexpf(1.0f, X);
    float r = ldexpf(1.0f, -X);
    float sse = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float y = ax[i] * r;
        int c = oracle_e2m1_code(y);
        float xhat = E2M1_MAG[c] * d;
        float e = ax[i] - xhat;
        float q = e * e;
        sse = (i == 0) ? q : sse + q;
        if (mag_codes)
            mag_codes[i] = (uint8_t)c;
    }
    return sse;
}

/* One block: 16 code bytes, returns the scale byte (255 for a non-finite block). */
static int mx_search_block(const float x[32], int f_lo, int f_hi, uint8_t out[16])
{
    float ax[32], amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        if (!isfinite(x[i])) {
            memset(out, 0, 16);
            return 255;
        }
        ax[i] = fabsf(x[i]);
        if (ax[i] > amax)
            amax = ax[i];
    }
    int X0 = amax > 0.0f ? floor_log2(amax) - 2 : -127;
    if (X0 < -127)
        X0 = -127;
    uint8_t best_codes[32];
    int best_X = X0;
    float best = mx_block_sse(ax, X0, best_codes);
    for (int f = f_lo; f <= f_hi; ++f) {
        int X = X0 + f;
        if (f == 0 || X < -127 || X > 127)
            continue;
        uint8_t c[32];
        float e = mx_block_sse(ax, X, c);
        if (e < best) {
            best = e;
            best_X = X;
            memcpy(best_codes, c, 32);
        }
    }
    for (int i = 0; i < 16; ++i) {
        int lo = best_codes[2 * i] | (signbit(x[2 * i]) ? 8 : 0);
        int hi = best_codes[2 * i + 1] | (signbit(x[2 * i + 1]) ? 8 : 0);
        out[i] = (uint8_t)(lo | (hi << 4));
    }
    return best_X + 127;
}

typedef struct {
    const void *x;
    int dtype;
    int64_t cols, r0, r1;
    int f_lo, f_hi;
    uint8_t *codes, *scales;
} mxjob_t;

static void *mx_rows(void *arg)
{
    const mxjob_t *J = (const mxjob_t *)arg;
    int64_t nb = J->cols / 32;
    for (int64_t r = J->r0; r < J->r1; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float x[32];
            for (int i = 0; i < 32; ++i)
                x[i] = load_elem(J->x, J->dtype, r * J->cols + b * 32 + i);
            J->scales[r * nb + b] =
                (uint8_t)mx_search_block(x, J->f_lo, J->f_hi, J->codes + r * (J->cols / 2) + b * 16);
        }
    return NULL;
}

/* MXFP4 quantize of x[rows][cols] (cols % 32 == 0): codes[rows][cols/2] (even
 * element in the low nibble), scales[rows][cols/32] (E8M0 bytes). */
int oracle_quantize_mxfp4(const void *x, int dtype, int64_t rows, int64_t cols, int f_lo, int f_hi,
                          uint8_t *codes, uint8_t *scales, int nthreads)
{
    if (rows < 0 || cols <= 0 || cols % 32 || f_lo > 0 || f_hi < 0 ||
        (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    if (rows == 0)
        return ORACLE_OK;
    if (!x || !codes || !scales)
        return ORACLE_EINVAL;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > rows)
        nthreads = (int)rows;
    pthread_t th[256];
    int running[256];
    mxjob_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (mxjob_t){x, dtype, cols, rows * t / nthreads, rows * (t + 1) / nthreads,
                            f_lo, f_hi, codes, scales};
        running[t] = nthreads > 1 && pthread_create(&th[t], NULL, mx_rows, &jobs[t]) == 0;
        if (!running[t])
            mx_rows(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (running[t])
            pthread_join(th[t], NULL);
    return ORACLE_OK;
}

/* Inverse: y = V * 2^(b - 127) in FP32 (exact), NaN for scale byte 255;
 * out_dtype BF16 rounds that value to nearest-even. */
int oracle_dequantize_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int64_t cols, int out_dtype, void *y)
{
    if (rows < 0 || cols <= 0 || cols % 32 || (out_dtype != ORACLE_F32 && out_dtype != ORACLE_BF16))
        return ORACLE_EINVAL;
    if (rows == 0)
        return ORACLE_OK;
    if (!codes || !scales || !y)
        return ORACLE_EINVAL;
    for (int64_t e = 0; e < rows * cols; ++e) {
        int nib = (codes[e / 2] >> ((e & 1) * 4)) & 0xF;
        int b = scales[e / 32];
        float v;
        if (b == 255)
            v = NAN;
        else {
            v = E2M1_MAG[nib & 7] * ldexpf(1.0f, b - 127);
            if (nib & 8)
                v = -v;
        }
        if (out_dtype == ORACLE_F32)
            ((float *)y)[e] = v;
        else
            ((uint16_t *)y)[e] = float_to_bf16_rne(v);
    }
    return ORACLE_OK;
}

/* Squared error of one 32-element block at scale 2^X (for the pins). */
float oracle_mx_block_sse(const float x[32], int X)
{
    float ax[32];
    for (int i = 0; i < 32; ++i)
        ax[i] = fabsf(x[i]);
    return mx_block_sse(ax, X, NULL);
}

/* ======================================================================== */
/* Attention on NVFP4 operands ([SSA] ネイティブ NVFP4 実行: ScaleSearchAttention */
/* computes QK^T and PV with NVFP4 operands and FP32 accumulation; the IP    */
/* transform and the sink cache are applied to the operands beforehand).     */
/*                                                                           */
/* Readings (the pages give no kernel): Q, K, V are NVFP4 tensors           */
/* [B][H][N][D] with 16-element blocks along D, each with its own tensor     */
/* scale; K and V heads may be shared by Hq / Hkv query heads. An operand   */
/* element is V[code] * s_block times its tensor scale. Scores              */
/* s_j = (q . k_j) / sqrt(D). The softmax runs online over the keys in      */
/* tiles of `tile` keys, in order: m' = max(m, max of the tile's s_j);      */
/* p_j = exp(s_j - m') rounded to binary32; l = e^(m - m') l + sum_j p_j.    */
/* P is coded to NVFP4 per 16 keys of a tile with max scaling (offset 0)    */
/* under the fixed tensor scale S_P = fl(1/2688) (p <= 1), exactly as the    */
/* quantizer codes a block, and acc = e^(m - m') acc + sum_j P^_j v_j with   */
/* P^_j = V[code] * s_block; O = acc * S_P / l. Because each tile's p is    */
/* taken against the running max, the tile size is part of the definition.  */
/* Keys past Nk are masked; with causal, query i sees keys j <= i + Nk - Nq. */
/* Everything is evaluated in double except p (binary32, as stated) and the */
/* coding of P (the quantizer's binary32 rule).                              */
/*                                                                           */
/* Besides O the oracle returns what a comparison with a binary32           */
/* implementation needs, per output element (in units of O):               */
/*   mag   sum_j |P^_j v_jd| * S_P / l: what FP32 sums of the products see; */
/*   rs    the sum over tiles of |acc_d| as each tile starts (after its      */
/*         rescale): the partial sums an in-order FP32 accumulation rounds;  */
/*   us    (split keys) sum over units |w_u acc_u,d|: the merge's terms;     */
/*   bound the largest change of sum_j P^_j |v_jd| from P codes that a       */
/*         binary32 score and exp could round the other way;                */
/* and per query row: the number of tiles whose max may move the running    */
/* max (each a rescale by a rounded exponential), the most tiles one softmax */
/* state visits, the largest relative error dl binary32 scores and exp can   */
/* put on a p, and the number of units merged.                              */
/* ======================================================================== */

static void decode_row(const uint8_t *codes, const uint8_t *scales, int64_t D, float *out)
{
    for (int64_t d = 0; d < D; ++d) {
        int nib = (codes[d / 2] >> ((d & 1) * 4)) & 0xF;
        float v = E2M1_MAG[nib & 7] * oracle_e4m3_value(scales[d / 16]);
        out[d] = (nib & 8) ? -v : v;
    }
}

/* Relative distance of y from the nearest E2M1 rounding midpoint, and the
 * gap between the two grid values on either side of it. */
static double e2m1_mid_distance(float y, float *gap)
{
    static const float MID[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    static const float GAP[7] = {0.5f, 0.5f, 0.5f, 0.5f, 1.0f, 1.0f, 2.0f};
    double best = INFINITY;
    for (int k = 0; k < 7; ++k) {
        double dd = fabs((double)y - MID[k]) / MID[k];
        if (dd < best) {
            best = dd;
            *gap = GAP[k];
        }
    }
    return best;
}

/* The flip allowance of one 16-key block of P. pf: the binary32 p values,
 * dl: each one's relative error allowance, p: the block's scale pattern,
 * ph: the coded values P^ (without S_P). flip[e] receives the largest
 * change of P^_e that a p within its allowance could cause:
 *  - the element's own code, when y = p * r lies within dl of an E2M1
 *    rounding midpoint: the grid gap there, times the block scale;
 *  - the block scale, when t = (amax / 6) / S_P lies within the allowance of
 *    an E4M3 midpoint: the neighbouring pattern p2 may be taken, and each
 *    element moves to its code under p2 (plus that code's own flip). */
static void p_block_allowance(const float pf[16], const double dl[16], int p, const float ph[16],
                              double flip[16])
{
    const float SP = 1.0f / 2688.0f;
    const float sp = oracle_e4m3_value(p);
    const float r = 1.0f / (sp * SP);
    float amax_b = 0.0f;
    double dmax = 0.0;
    for (int e = 0; e < 16; ++e) {
        if (pf[e] > amax_b)
            amax_b = pf[e];
        if (dl[e] > dmax)
            dmax = dl[e];
    }
    for (int e = 0; e < 16; ++e) {
        float gap = 0.0f;
        flip[e] = 0.0;
        if (pf[e] > 0.0f && e2m1_mid_distance(pf[e] * r, &gap) <= dl[e] + 0x1p-22)
            flip[e] = (double)gap * sp;
    }
    if (amax_b == 0.0f)
        return;
    const float tb = (amax_b / 6.0f) / SP;
    for (int nb = -1; nb <= 1; nb += 2) {
        const int p2 = p + nb;
        if (p2 < 0 || p2 > 126)
            continue;
        const double mid = 0.5 * ((double)oracle_e4m3_value(p) + oracle_e4m3_value(p2));
        if (fabs((double)tb - mid) > (dmax + 0x1p-21) * mid)
            continue;
        const float sp2 = oracle_e4m3_value(p2);
        const float r2 = 1.0f / (sp2 * SP);
        for (int e = 0; e < 16; ++e) {
            float y2 = pf[e] * r2, gap2 = 0.0f;
            double dv = fabs((double)E2M1_MAG[oracle_e2m1_code(y2)] * sp2 - ph[e]);
            if (pf[e] > 0.0f && e2m1_mid_distance(y2, &gap2) <= dl[e] + 0x1p-22)
                dv += (double)gap2 * sp2;
            if (dv > flip[e])
                flip[e] = dv;
        }
    }
}

/* Online-softmax state of one query over a run of keys: running max m, sum
 * l, and per output element the unnormalized sum acc, its magnitude sum mg,
 * the flip allowance bd, rs (the partial sums |acc| at tile starts) and mp
 * (the magnitude sum of the tiles before the last possible rise of the
 * running max, whose P was coded against an earlier max). nres
 * counts tiles that may move the running max, ntiles the tiles visited, dmax
 * is the largest p allowance, arun the largest score magnitude sum
 * sum_d |q_d k_d| / sqrt(D) of the keys visited. */
typedef struct {
    double m, l, dmax, arun;
    int64_t nres, ntiles;
    double *acc, *mg, *bd, *rs, *mp;
} sstate_t;

typedef struct {
    double *s, *dl, *A;
    float *pf, *ph;
} stile_t;

static void state_clear(sstate_t *st, int64_t D)
{
    st->m = -INFINITY;
    st->l = 0.0;
    st->dmax = 0.0;
    st->arun = 0.0;
    st->nres = st->ntiles = 0;
    for (int64_t d = 0; d < D; ++d)
        st->acc[d] = st->mg[d] = st->bd[d] = st->rs[d] = st->mp[d] = 0.0;
}

/* Keys [lo, hi) in tiles of `tile` keys from lo (a last tile may be short),
 * folded into the state st. kv[t * D + d]: key t with the query's and its
 * own tensor scale folded in (score = q . kv / sqrt(D)); vv[t * D + d] * vfac[t]:
 * value t. */
static void fold_tiles(int64_t D, int64_t tile, const float *q, const double *kv,
                       const float *vv, const double *vfac, int64_t lo, int64_t hi,
                       sstate_t *st, stile_t *w)
{
    const float SP = 1.0f / 2688.0f;
    const double tau = 1.0 / sqrt((double)D);
    double *s = w->s, *dl = w->dl, *A = w->A;
    float *pf = w->pf, *ph = w->ph;
    for (int64_t t0 = lo; t0 < hi; t0 += tile) {
        double mt = -INFINITY, amax_abs = 0.0;
        for (int64_t u = 0; u < tile; ++u) {
            int64_t j = t0 + u;
            s[u] = -INFINITY;
            A[u] = 0.0;
            if (j < hi) {
                double dot = 0.0, ab = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    double pr = (double)q[d] * kv[j * D + d];
                    dot += pr;
                    ab += fabs(pr);
                }
                s[u] = tau * dot;
                A[u] = tau * ab;
                if (s[u] > mt)
                    mt = s[u];
                if (A[u] > amax_abs)
                    amax_abs = A[u];
            }
        }
        if (amax_abs > st->arun)
            st->arun = amax_abs;
        double mn = st->m > mt ? st->m : mt;
        if (mn == -INFINITY)
            continue;
        /* a binary32 score carries up to amax_abs (D + 2) 2^-24 of FP32 sum
           error and a few roundings of s and the max: a tile whose max comes
           within twice that of the running max may move it there */
        const double serr = amax_abs * (double)(D + 2) * 0x1p-24 +
                            (fabs(st->m == -INFINITY ? mt : st->m) + fabs(mt)) * 0x1p-21;
        const int rise = st->m != -INFINITY && mt + 2.0 * serr >= st->m;
        if (rise)
            st->nres += 1;
        st->ntiles += 1;
        double alpha = (st->m == -INFINITY) ? 0.0 : exp(st->m - mn);
        double psum = 0.0;
        for (int64_t u = 0; u < tile; ++u) {
            pf[u] = (s[u] == -INFINITY) ? 0.0f : (float)exp(s[u] - mn);
            psum += pf[u];
            /* relative error binary32 scores and exp can put on p = exp(s - m):
               the FP32 sums of s and of the running max's own score (each at
               most (D + 2) u times its magnitude sum; the max's is at most
               arun), the roundings of s, m and their difference, and exp */
            dl[u] = (s[u] == -INFINITY)
                        ? 0.0
                        : (A[u] + st->arun) * (double)(D + 2) * 0x1p-24 +
                              (fabs(s[u]) + fabs(mn)) * 0x1p-21 + 0x1p-20;
            if (dl[u] > st->dmax)
                st->dmax = dl[u];
        }
        st->l = alpha * st->l + psum;
        for (int64_t d = 0; d < D; ++d) {
            st->acc[d] *= alpha;
            st->mg[d] *= alpha;
            st->bd[d] *= alpha;
            st->rs[d] = st->rs[d] * alpha + fabs(st->acc[d]);
            /* the tiles before a possible rise of the max: their P was coded
               against a running max other than the final one */
            st->mp[d] = rise ? st->mg[d] : st->mp[d] * alpha;
        }
        for (int64_t u0 = 0; u0 < tile; u0 += 16) {
            uint8_t cb[8];
            double flip[16];
            int p = search_block(pf + u0, SP, 0, 0, cb, NULL);
            float sp = oracle_e4m3_value(p);
            for (int e = 0; e < 16; ++e) {
                int nib = (cb[e / 2] >> ((e & 1) * 4)) & 0xF;
                ph[u0 + e] = E2M1_MAG[nib & 7] * sp;
            }
            p_block_allowance(pf + u0, dl + u0, p, ph + u0, flip);
            for (int e = 0; e < 16; ++e) {
                int64_t j = t0 + u0 + e;
                if (j >= hi || pf[u0 + e] == 0.0f)
                    continue;
                for (int64_t d = 0; d < D; ++d) {
                    double v = (double)vv[j * D + d] * vfac[j];
                    st->acc[d] += (double)ph[u0 + e] * v;
                    st->mg[d] += (double)ph[u0 + e] * fabs(v);
                    st->bd[d] += flip[e] * fabs(v);
                }
            }
        }
        st->m = mn;
    }
}

/* Combine the units' states (O = S_P sum w_u acc_u / sum w_u l_u, w_u =
 * exp(m_u - M), M = max m_u; a unit with no key has m_u = -inf) into row r
 * of the outputs. mpre: the magnitude of the keys whose P was coded against a
 * running max other than the overall one: the tiles before the last possible
 * rise in the unit that holds M (when no other unit's max comes within dmax
 * of it), every key of the other units. */
static void write_row(const sstate_t *us, int64_t nunits, int64_t D, int64_t r, double *O,
                      double *mag, double *bound, double *rs, double *usum, double *mpre,
                      double *rowinfo)
{
    const double SP = (double)(1.0f / 2688.0f);
    double M = -INFINITY;
    int64_t top = -1;
    for (int64_t u = 0; u < nunits; ++u)
        if (us[u].m > M) {
            M = us[u].m;
            top = u;
        }
    double L = 0.0, dmax = 0.0;
    int64_t nres = 0, ntiles = 0, live = 0;
    for (int64_t u = 0; u < nunits; ++u) {
        if (us[u].m == -INFINITY)
            continue;
        L += exp(us[u].m - M) * us[u].l;
        live += 1;
        if (us[u].nres > nres)
            nres = us[u].nres;
        if (us[u].ntiles > ntiles)
            ntiles = us[u].ntiles;
        if (us[u].dmax > dmax)
            dmax = us[u].dmax;
    }
    for (int64_t u = 0; u < nunits; ++u)
        if (u != top && us[u].m != -INFINITY && us[u].m >= M - 2.0 * dmax)
            top = -1; /* another unit's max may be the largest in binary32 */
    double f = (L > 0.0) ? SP / L : 0.0;
    for (int64_t d = 0; d < D; ++d) {
        double o = 0.0, mg = 0.0, bd = 0.0, r2 = 0.0, ua = 0.0, mp = 0.0;
        for (int64_t u = 0; u < nunits; ++u) {
            if (us[u].m == -INFINITY)
                continue;
            double wu = exp(us[u].m - M);
            o += wu * us[u].acc[d];
            mg += wu * us[u].mg[d];
            bd += wu * us[u].bd[d];
            r2 += wu * us[u].rs[d];
            ua += fabs(wu * us[u].acc[d]);
            mp += wu * (u == top ? us[u].mp[d] : us[u].mg[d]);
        }
        O[r * D + d] = o * f;
        if (mag)
            mag[r * D + d] = mg * f;
        if (bound)
            bound[r * D + d] = bd * f;
        if (rs)
            rs[r * D + d] = r2 * f;
        if (usum)
            usum[r * D + d] = live > 1 ? ua * f : 0.0;
        if (mpre)
            mpre[r * D + d] = live > 1 ? mp * f : us[top < 0 ? 0 : top].mp[d] * f;
    }
    if (rowinfo) {
        rowinfo[4 * r + 0] = (double)nres;
        rowinfo[4 * r + 1] = (double)ntiles;
        rowinfo[4 * r + 2] = dmax;
        rowinfo[4 * r + 3] = (double)live;
    }
}

typedef struct {
    const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
    float qg, kg, vg;
    int64_t B, Hq, Hkv, Nq, Nk, D, tile;
    int causal;
    double *O, *mag, *bound, *rs, *usum, *mpre, *rowinfo;
    int64_t r0, r1; /* rows (b, h, i) of this job */
} ajob_t;

static void *attention_rows(void *arg)
{
    const ajob_t *J = (const ajob_t *)arg;
    const int64_t D = J->D, Nk = J->Nk, T = J->tile;
    const double qk = (double)J->qg * (double)J->kg;
    const size_t nk = (size_t)(Nk > 0 ? Nk : 1);
    float *q = malloc(sizeof(float) * D), *tmp = malloc(sizeof(float) * D);
    double *kv = malloc(sizeof(double) * D * nk);
    float *vv = malloc(sizeof(float) * D * nk);
    double *vfac = malloc(sizeof(double) * nk);
    double *sbuf = malloc(sizeof(double) * 5 * D);
    sstate_t st = {0, 0, 0, 0, 0, 0, sbuf, sbuf + D, sbuf + 2 * D, sbuf + 3 * D, sbuf + 4 * D};
    stile_t w = {malloc(sizeof(double) * T), malloc(sizeof(double) * T),
                 malloc(sizeof(double) * T), malloc(sizeof(float) * T), malloc(sizeof(float) * T)};
    int64_t cached_head = -1;
    for (int64_t r = J->r0; r < J->r1; ++r) {
        int64_t i = r % J->Nq, bh = r / J->Nq;
        int64_t b = bh / J->Hq, h = bh % J->Hq;
        int64_t kvh = b * J->Hkv + h / (J->Hq / J->Hkv);
        if (kvh != cached_head) {
            for (int64_t j = 0; j < Nk; ++j) {
                int64_t row = kvh * Nk + j;
                decode_row(J->kc + row * (D / 2), J->ks + row * (D / 16), D, tmp);
                for (int64_t d = 0; d < D; ++d)
                    kv[j * D + d] = (double)tmp[d] * qk;
                decode_row(J->vc + row * (D / 2), J->vs + row * (D / 16), D, vv + j * D);
                vfac[j] = (double)J->vg;
            }
            cached_head = kvh;
        }
        decode_row(J->qc + r * (D / 2), J->qs + r * (D / 16), D, q);
        /* visible keys: [0, Nk), or with causal [0, i + Nk - Nq] */
        int64_t hi = J->causal ? i + Nk - J->Nq + 1 : Nk;
        if (hi > Nk)
            hi = Nk;
        state_clear(&st, D);
        if (hi > 0)
            fold_tiles(D, T, q, kv, vv, vfac, 0, hi, &st, &w);
        write_row(&st, 1, D, r, J->O, J->mag, J->bound, J->rs, J->usum, J->mpre, J->rowinfo);
    }
    free(q); free(tmp); free(kv); free(vv); free(vfac); free(sbuf);
    free(w.s); free(w.dl); free(w.A); free(w.pf); free(w.ph);
    return NULL;
}

int oracle_attention_nvfp4(const uint8_t *qc, const uint8_t *qs, float qg, const uint8_t *kc,
                           const uint8_t *ks, float kg, const uint8_t *vc, const uint8_t *vs,
                           float vg, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                           int64_t D, int64_t tile, int causal, double *O, double *mag,
                           double *bound, double *rs, double *usum, double *mpre, double *rowinfo,
                           int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Nq < 0 || Nk < 0 || D <= 0 || D % 16 ||
        tile <= 0 || tile % 16 || !O)
        return ORACLE_EINVAL;
    int64_t rows = B * Hq * Nq;
    if (rows == 0)
        return ORACLE_OK;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > rows)
        nthreads = (int)rows;
    pthread_t th[256];
    int running[256];
    ajob_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (ajob_t){qc, qs, kc, ks, vc, vs, qg, kg, vg, B, Hq, Hkv, Nq, Nk, D, tile,
                           causal, O, mag, bound, rs, usum, mpre, rowinfo, rows * t / nthreads,
                           rows * (t + 1) / nthreads};
        running[t] = nthreads > 1 && pthread_create(&th[t], NULL, attention_rows, &jobs[t]) == 0;
        if (!running[t])
            attention_rows(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (running[t])
            pthread_join(th[t], NULL);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention over the attention-sink KV cache ([SSA] アテンション・シンク対応  */
/* 混合精度キャッシング: the first and last KV blocks stay in full precision, */
/* the middle is NVFP4). The cache holds T tokens: token t < n_first in      */
/* head[t], t >= max(n_first, T - n_last) in the ring tail[t mod n_last]     */
/* (bf16), the rest coded at middle row t - n_first under the tensor scale.  */
/* Reading: keys are visited segment by segment (head, middle, tail, each in */
/* token order) in tiles of `tile` keys that never straddle two segments (a */
/* segment's last tile may be short); everything else is the attention      */
/* above. All T keys are visible.                                            */
/*                                                                          */
/* Split keys (split > 0, a multiple of the tile). The pages describe the   */
/* attention's online softmax but not how one query's keys are spread over  */
/* parallel workers; this reading lets a decode step with few queries do    */
/* so. The keys fall into units: the head, the tail, and the middle cut     */
/* into pieces of `split` tokens from n_first (the last may be short). Each */
/* unit runs the online softmax and the coding of P above from its own      */
/* running max, alone; the unit states (m_u, l_u, acc_u) then combine       */
/* exactly: with M = max m_u and w_u = exp(m_u - M), O = S_P sum w_u acc_u  */
/* / sum w_u l_u. split = 0 folds the three segments into one state.        */
/* ------------------------------------------------------------------------ */
typedef struct {
    const uint8_t *qc, *qs;
    float qg;
    const uint16_t *kh, *kt, *vh, *vt;
    const uint8_t *kc, *ks, *vc, *vs;
    float kg, vg;
    int64_t B, Hq, Hkv, Nq, T, D, nf, nl, cap, tile, split;
    double *O, *mag, *bound, *rs, *usum, *mpre, *rowinfo;
    int64_t r0, r1;
} cjob_t;

static void *attention_cache_rows(void *arg)
{
    const cjob_t *J = (const cjob_t *)arg;
    const int64_t D = J->D, T = J->T, tile = J->tile;
    float *q = malloc(sizeof(float) * D), *tmp = malloc(sizeof(float) * D);
    double *kv = malloc(sizeof(double) * D * (size_t)(T > 0 ? T : 1));
    float *vv = malloc(sizeof(float) * D * (size_t)(T > 0 ? T : 1));
    double *vfac = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    stile_t w = {malloc(sizeof(double) * tile), malloc(sizeof(double) * tile),
                 malloc(sizeof(double) * tile), malloc(sizeof(float) * tile),
                 malloc(sizeof(float) * tile)};
    const int64_t mid_lo = J->nf, mid_hi = T - J->nl > J->nf ? T - J->nl : J->nf;
    /* the units whose softmax states are combined: the three segments folded
       into one state (no split), or head, each piece of `split` middle keys and
       tail each with its own state */
    const int64_t npieces = J->split > 0 ? (mid_hi - mid_lo + J->split - 1) / J->split : 0;
    const int64_t nunits = J->split > 0 ? 2 + npieces : 1;
    double *ubuf = malloc(sizeof(double) * (size_t)(5 * D * nunits + 1));
    sstate_t *us = malloc(sizeof(sstate_t) * (size_t)nunits);
    for (int64_t u = 0; u < nunits; ++u) {
        double *b = ubuf + 5 * D * u;
        us[u] = (sstate_t){0, 0, 0, 0, 0, 0, b, b + D, b + 2 * D, b + 3 * D, b + 4 * D};
    }
    int64_t cached = -1;
    for (int64_t r = J->r0; r < J->r1; ++r) {
        int64_t bh = r / J->Nq;
        int64_t b = bh / J->Hq, h = bh % J->Hq;
        int64_t kvh = b * J->Hkv + h / (J->Hq / J->Hkv);
        if (kvh != cached) {
            /* key t with the query's tensor scale (and a coded key's own) folded in */
            for (int64_t t = 0; t < T; ++t) {
                double *kd = kv + t * D;
                float *vd = vv + t * D;
                if (t < J->nf || t >= mid_hi) {
                    const uint16_t *kr, *vr;
                    if (t < J->nf) {
                        kr = J->kh + (kvh * J->nf + t) * D;
                        vr = J->vh + (kvh * J->nf + t) * D;
                    } else {
                        kr = J->kt + (kvh * J->nl + t % J->nl) * D;
                        vr = J->vt + (kvh * J->nl + t % J->nl) * D;
                    }
                    for (int64_t d = 0; d < D; ++d) {
                        kd[d] = (double)bf16_bits_to_float(kr[d]) * (double)J->qg;
                        vd[d] = bf16_bits_to_float(vr[d]);
                    }
                    vfac[t] = 1.0;
                } else {
                    int64_t row = kvh * J->cap + (t - J->nf);
                    decode_row(J->kc + row * (D / 2), J->ks + row * (D / 16), D, tmp);
                    for (int64_t d = 0; d < D; ++d)
                        kd[d] = (double)tmp[d] * ((double)J->kg * (double)J->qg);
                    decode_row(J->vc + row * (D / 2), J->vs + row * (D / 16), D, vd);
                    vfac[t] = (double)J->vg;
                }
            }
            cached = kvh;
        }
        decode_row(J->qc + r * (D / 2), J->qs + r * (D / 16), D, q);
        const int64_t head_hi = J->nf < T ? J->nf : T;
        const int64_t tail_lo = mid_hi > J->nf ? mid_hi : J->nf;
        for (int64_t u = 0; u < nunits; ++u)
            state_clear(&us[u], D);
        if (J->split <= 0) {
            fold_tiles(D, tile, q, kv, vv, vfac, 0, head_hi, &us[0], &w);
            fold_tiles(D, tile, q, kv, vv, vfac, mid_lo, mid_hi, &us[0], &w);
            fold_tiles(D, tile, q, kv, vv, vfac, tail_lo, T, &us[0], &w);
        } else {
            fold_tiles(D, tile, q, kv, vv, vfac, 0, head_hi, &us[0], &w);
            fold_tiles(D, tile, q, kv, vv, vfac, tail_lo, T, &us[1], &w);
            for (int64_t k = 0; k < npieces; ++k) {
                int64_t lo = mid_lo + k * J->split, hi = lo + J->split;
                fold_tiles(D, tile, q, kv, vv, vfac, lo, hi < mid_hi ? hi : mid_hi, &us[2 + k],
                           &w);
            }
        }
        write_row(us, nunits, D, r, J->O, J->mag, J->bound, J->rs, J->usum, J->mpre, J->rowinfo);
    }
    free(q); free(tmp); free(kv); free(vv); free(vfac); free(ubuf); free(us);
    free(w.s); free(w.dl); free(w.A); free(w.pf); free(w.ph);
    return NULL;
}

int oracle_attention_kv_cache(const uint8_t *qc, const uint8_t *qs, float qg, const uint16_t *kh,
                              const uint16_t *kt, const uint8_t *kc, const uint8_t *ks, float kg,
                              const uint16_t *vh, const uint16_t *vt, const uint8_t *vc,
                              const uint8_t *vs, float vg, int64_t B, int64_t Hq, int64_t Hkv,
                              int64_t Nq, int64_t T, int64_t D, int64_t nf, int64_t nl, int64_t cap,
                              int64_t tile, int64_t split, double *O, double *mag, double *bound,
                              double *rs, double *usum, double *mpre, double *rowinfo,
                              int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Nq < 0 || T < 0 || D <= 0 || D % 16 ||
        D > 1024 || nf < 0 || nl < 0 || cap < 0 || tile <= 0 || tile % 16 || split < 0 ||
        (split > 0 && split % tile) || !O)
        return ORACLE_EINVAL;
    int64_t mid = T - nf - nl;
    if (mid > cap)
        return ORACLE_EINVAL;
    int64_t rows = B * Hq * Nq;
    if (rows == 0)
        return ORACLE_OK;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > rows)
        nthreads = (int)rows;
    pthread_t th[256];
    int running[256];
    cjob_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (cjob_t){qc, qs, qg, kh, kt, vh, vt, kc, ks, vc, vs, kg, vg, B, Hq, Hkv, Nq, T,
                           D, nf, nl, cap, tile, split, O, mag, bound, rs, usum, mpre, rowinfo,
                           rows * t / nthreads, rows * (t + 1) / nthreads};
        running[t] = nthreads > 1 && pthread_create(&th[t], NULL, attention_cache_rows, &jobs[t]) == 0;
        if (!running[t])
            attention_cache_rows(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (running[t])
            pthread_join(th[t], NULL);
    return ORACLE_OK;
}
