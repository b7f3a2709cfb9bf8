// nvfp4_device.h -- device helpers shared by the gfx950 kernels: vector
// types, streaming loads/stores, the UE4M3 scale codec and the hardware E2M1
// converts. Compile with -ffp-contract=off.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nvfp4_internal.h"

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming accesses (read or written once): nontemporal, so they do not
// displace cached data; measured faster than plain loads/stores on these
// passes.
__device__ __forceinline__ uint4 load_stream(const void *p) {
  const u32x4 t = __builtin_nontemporal_load((const u32x4 *)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store_stream(void *p, uint32_t a, uint32_t b, uint32_t c,
                                             uint32_t d) {
  __builtin_nontemporal_store((u32x4){a, b, c, d}, (u32x4 *)p);
}

// ---------------------------------------------------------------------------
// Small device helpers.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv &f) {
  uint32_t t = __umulhi(n, f.m);
  return (uint32_t)(((uint64_t)t + n) >> f.s);
}

// Value of UE4M3 pattern p in 0..126 (4 exponent bits, bias 7; 3 mantissa
// bits; exponent field 0 is subnormal m * 2^-9). Exact in FP32.
__device__ __forceinline__ float e4m3_value(uint32_t p) {
  uint32_t e = p >> 3, m = p & 7u;
  float sub = (float)m * 0x1p-9f;
  float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// UE4M3 round-to-nearest-even with saturation at 448 (pattern 126), t >= 0.
// Normal range: keep 3 mantissa bits of the FP32 pattern with a nearest-even
// carry, then rebias the exponent (127 -> 7). Below 2^-6 the format steps by
// 2^-9, so the pattern is t * 2^9 rounded to an integer (exact scaling).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float t) {
  uint32_t b = __float_as_uint(t);
  uint32_t nrm = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - 960u;
  uint32_t sub = (uint32_t)__builtin_rintf(t * 512.0f);
  uint32_t p = t < 0x1p-6f ? sub : nrm;
  return t >= 448.0f ? 126u : p;
}

// Hardware E2M1 converts (gfx950). The byte selector must be a constant, so
// the switch folds away once the callers' loops are unrolled.
__device__ __forceinline__ uint32_t fp4_encode_pair(uint32_t old, float a, float b, int sel) {
  switch (sel & 3) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 3);
  }
}

__device__ __forceinline__ f32x2 fp4_decode_pair(uint32_t w, int sel) {
  switch (sel & 3) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

}  // namespace nvfp4
