/*
 * mxfp4.h -- MXFP4, the power-of-two contrast format, in the same library
 * (libnvfp4.so) and with the same conventions as nvfp4.h: device pointers,
 * caller-owned memory, calls enqueued on the caller's HIP stream (NULL: the
 * default stream), status codes of nvfp4_status, argument checks made before
 * anything is enqueued.
 *
 * Source: "NVIDIAのFP4推論が50倍の効率を実現", section 超低精度推論を支えるアーキテクチャ,
 * sets NVFP4's E4M3 block scale and FP32 tensor scale against MXFP4's simple
 * power-of-two scaling (and claims a much lower quantization error for NVFP4).
 * The page does not define MXFP4; the format read here is the OCP
 * Microscaling v1.0 one:
 *   - blocks of 32 consecutive elements of the last dimension;
 *   - one E8M0 scale byte b per block, standing for 2^(b - 127), b = 0..254;
 *     b = 255 is NaN;
 *   - E2M1 element codes, two per byte, even element in the low nibble, sign
 *     in bit 3 of the nibble (the sign of zero is the input's);
 *   - no tensor scale.
 * Scale rule: X0 = floor(log2(max |x| of the block)) - 2 (2 = the exponent of
 * E2M1's largest value 6 = 1.5 * 2^2), at least -127; an all-zero block takes
 * X0 = -127. Elements code as E2M1 of |x| * 2^-X (exact unless subnormal),
 * nearest-even, saturating at 6 (a block amax in (6, 8) * 2^X clips).
 * Offsets [f_lo, f_hi] carry ScaleSearch (ScaleSearch summary page, 手法 >
 * ScaleSearch) over to E8M0: candidates X0 + f (each step doubles the
 * scale), f = 0 first, then f_lo..f_hi, the least squared error
 * sum_i fl(fl(|x_i| - |x^_i|)^2) added left to right in FP32 wins, first
 * strictly smaller; X0 + f outside -127..127 is skipped. [0, 0] is the plain
 * OCP conversion. A block holding a NaN or Inf gets scale 255 and zero codes.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include "nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Quantize x[rows][cols] (xdt) to MXFP4: codes[rows][cols/2],
 * scales[rows][cols/32]. block must be 32, cols % 32 == 0,
 * -8 <= f_lo <= 0 <= f_hi <= 8. x and codes 16-byte aligned. No workspace. */
NVFP4_API nvfp4_status mxfp4_quantize(const void *x, nvfp4_dtype xdt, int64_t rows, int64_t cols,
                                      int block, int f_lo, int f_hi, uint8_t *codes,
                                      uint8_t *scales, void *stream);

/* Inverse: y[rows][cols] (ydt FP32, or bf16 = nearest-even of the exact FP32
 * value V * 2^X). codes and y 16-byte aligned. */
NVFP4_API nvfp4_status mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                        int64_t cols, int block, void *y, nvfp4_dtype ydt,
                                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
