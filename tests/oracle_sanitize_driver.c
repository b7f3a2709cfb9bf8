/* Drives every oracle entry point once on small seeded inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py).
 * TEST INFRASTRUCTURE: it links only the oracle. Exit status 0 when every call
 * returns success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quantize(const void *, int, int64_t, int64_t, int, int, int, int, float *, uint8_t *,
                    uint8_t *, int8_t *, int);
int oracle_dequantize(const uint8_t *, const uint8_t *, float, int64_t, int64_t, int, void *);
int oracle_quantize_kv_sink(const void *, int, int64_t, int64_t, int64_t, int64_t, int64_t,
                            int64_t, int, int, int, int, float *, uint8_t *, uint8_t *, void *,
                            int);
int oracle_dequantize_kv_sink(const uint8_t *, const uint8_t *, float, const void *, int, int64_t,
                              int64_t, int64_t, int64_t, int64_t, int64_t, int, void *);
int oracle_hadamard128(const void *, int, int64_t, float *, int);
int oracle_hadamard128_rht(const void *, int, int64_t, const uint32_t *, float *, int);
int oracle_balance_exponents(const void *, const void *, int, int64_t, int64_t, int64_t, int8_t *);
int oracle_quantize_balanced(const void *, int, int64_t, int64_t, const int8_t *, int, int,
                             const uint32_t *, int, int, int, float *, uint8_t *, uint8_t *, int);
int oracle_hadamard128_balanced(const void *, int, int64_t, int64_t, const int8_t *, int,
                                const uint32_t *, float *, int);
int oracle_quantize_rht(const void *, int, int64_t, int64_t, const uint32_t *, int, int, int,
                        float *, uint8_t *, uint8_t *, int);
int oracle_quantize_mxfp4(const void *, int, int64_t, int64_t, int, int, uint8_t *, uint8_t *,
                          int);
int oracle_dequantize_mxfp4(const uint8_t *, const uint8_t *, int64_t, int64_t, int, void *);
int oracle_attention_nvfp4(const uint8_t *, const uint8_t *, float, const uint8_t *,
                           const uint8_t *, float, const uint8_t *, const uint8_t *, float, int64_t,
                           int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, double *,
                           double *, double *, double *, double *, double *, double *, int);
int oracle_attention_kv_cache(const uint8_t *, const uint8_t *, float, const uint16_t *,
                              const uint16_t *, const uint8_t *, const uint8_t *, float,
                              const uint16_t *, const uint16_t *, const uint8_t *,
                              const uint8_t *, float, int64_t, int64_t, int64_t, int64_t, int64_t,
                              int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, double *,
                              double *, double *, double *, double *, double *, double *, int);

static uint64_t state = 88172645463325252ull;
static double uniform(void) { /* xorshift64 */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) * 0x1p-53;
}
static float gauss(void) {
    double u = uniform() + 1e-300, v = uniform();
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

#define CHECK(call)                                             \
    do {                                                        \
        int rc_ = (call);                                       \
        if (rc_) {                                              \
            fprintf(stderr, "%s failed: %d\n", #call, rc_);     \
            return 1;                                           \
        }                                                       \
    } while (0)

int main(void) {
    enum { R = 37, K = 256, B = 1, H = 2, T = 200, D = 128, NF = 32, NL = 40 };
    float *x = malloc(sizeof(float) * R * K);
    uint16_t *xb = malloc(sizeof(uint16_t) * R * K);
    for (int i = 0; i < R * K; ++i) {
        x[i] = gauss();
        xb[i] = bf16(x[i]);
    }
    x[5] = NAN; /* one non-finite block in the FP32 tensor */
    uint8_t *codes = malloc(R * K / 2), *scales = malloc(R * K / 16);
    int8_t *fsel = malloc(R * K / 16);
    float g = 0.0f, *y = malloc(sizeof(float) * R * K);
    CHECK(oracle_quantize(x, 0, R, K, -2, 6, 0, 0, &g, codes, scales, fsel, 3));
    CHECK(oracle_quantize(xb, 1, R, K, -8, 8, 1, 0, &g, codes, scales, NULL, 2));
    CHECK(oracle_dequantize(codes, scales, g, R, K, 0, y));
    CHECK(oracle_dequantize(codes, scales, g, R, K, 1, xb));
    CHECK(oracle_hadamard128(xb, 1, R * K / 128, y, 2));
    uint32_t signs[4] = {0x12345678u, 0x9abcdef0u, 0x0f0f0f0fu, 0xdeadbeefu};
    CHECK(oracle_hadamard128_rht(xb, 1, R * K / 128, signs, y, 2));
    CHECK(oracle_quantize_rht(xb, 1, R, K, signs, -8, 8, 0, &g, codes, scales, 2));
    /* the balancing pair: calibration, both sides, with and without the transform */
    int8_t *e = malloc(K);
    CHECK(oracle_balance_exponents(xb, x, 1, R, 0, K, e)); /* K rows 0: every e is 0 */
    CHECK(oracle_balance_exponents(xb, xb, 1, R / 2, R - R / 2, K, e));
    for (int j = 0; j < K; j += 7) e[j] = (int8_t)(j % 5 - 2);
    e[3] = 100; /* clamped */
    CHECK(oracle_quantize_balanced(xb, 1, R, K, e, -1, 0, NULL, -2, 6, 0, &g, codes, scales, 2));
    CHECK(oracle_quantize_balanced(x, 0, R, K, e, 1, 0, NULL, -8, 8, 0, &g, codes, scales, 2));
    CHECK(oracle_quantize_balanced(xb, 1, R * 2, 128, e, 1, 1, signs, -8, 8, 0, &g, codes, scales,
                                   2));
    CHECK(oracle_hadamard128_balanced(xb, 1, R * 2, 128, e, -1, NULL, y, 2));
    free(e);
    CHECK(oracle_quantize_mxfp4(x, 0, R, K, -1, 1, codes, scales, 2));
    CHECK(oracle_dequantize_mxfp4(codes, scales, R, K, 1, xb));

    uint16_t *kv = malloc(sizeof(uint16_t) * B * H * T * D);
    for (int i = 0; i < B * H * T * D; ++i) kv[i] = bf16(gauss());
    const int TM = T - NF - NL;
    uint8_t *kc = malloc(B * H * TM * D / 2), *ks = malloc(B * H * TM * D / 16);
    uint16_t *sink = malloc(sizeof(uint16_t) * B * H * (NF + NL) * D);
    uint16_t *yk = malloc(sizeof(uint16_t) * B * H * T * D);
    float kg = 0.0f;
    CHECK(oracle_quantize_kv_sink(kv, 1, B, H, T, D, NF, NL, -2, 6, 0, 0, &kg, kc, ks, sink, 2));
    CHECK(oracle_dequantize_kv_sink(kc, ks, kg, sink, 1, B, H, T, D, NF, NL, 1, yk));

    /* attention: Q [1, 2, 20, 128], K = V = the coded middle [1, 1, TM * 2, 128] */
    const int NQ = 20, NK = 2 * TM;
    uint8_t *qc = malloc(B * H * NQ * D / 2), *qs = malloc(B * H * NQ * D / 16);
    float qg = 0.0f;
    CHECK(oracle_quantize(kv, 1, B * H * NQ, D, -2, 6, 0, 0, &qg, qc, qs, NULL, 1));
    const int64_t NO = (int64_t)B * H * NQ * D;
    double *O = malloc(sizeof(double) * (NO * 6 + (int64_t)B * H * NQ * 4));
    double *RI = O + 6 * NO;
    CHECK(oracle_attention_nvfp4(qc, qs, qg, kc, ks, kg, kc, ks, kg, B, H, 1, NQ, NK, D, 32, 1, O,
                                 O + NO, O + 2 * NO, O + 3 * NO, O + 4 * NO, O + 5 * NO, RI, 2));
    /* the sink cache: head NF, tail ring NL, middle rows = the coded middle */
    CHECK(oracle_attention_kv_cache(qc, qs, qg, sink, sink + B * H * NF * D, kc, ks, kg, sink,
                                    sink + B * H * NF * D, kc, ks, kg, B, H, 1, NQ, NF + TM + NL, D,
                                    NF, NL, TM, 32, 0, O, O + NO, O + 2 * NO, O + 3 * NO,
                                    O + 4 * NO, O + 5 * NO, RI, 2));
    /* the same with the middle split into pieces of 64 tokens */
    CHECK(oracle_attention_kv_cache(qc, qs, qg, sink, sink + B * H * NF * D, kc, ks, kg, sink,
                                    sink + B * H * NF * D, kc, ks, kg, B, H, 1, NQ, NF + TM + NL, D,
                                    NF, NL, TM, 32, 64, O, O + NO, O + 2 * NO, O + 3 * NO,
                                    O + 4 * NO, O + 5 * NO, RI, 2));
    free(x); free(xb); free(codes); free(scales); free(fsel); free(y); free(kv); free(kc);
    free(ks); free(sink); free(yk); free(qc); free(qs); free(O);
    puts("oracle sanitizer run: ok");
    return 0;
}
