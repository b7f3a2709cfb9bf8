// nvfp4_selfcheck.hip -- nvfp4_hw_self_check: the converter facts the attention
// kernels rely on, checked on the device at hand.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Self-check of the converter facts the kernels rely on, run on the device at
// hand: counts[0] the binary32 values t in [0, 448] whose FP32 -> FP8 (E4M3)
// convert differs from the UE4M3 nearest-even rounding e4m3_rne_sat (the
// attention's P pattern estimate); counts[1] the bytes 0..126 whose FP8 ->
// FP32 convert differs from the UE4M3 value e4m3_value (the attention's block
// scales). Every lane walks a strided range of bit patterns; counts are added
// with vector atomics.
// ---------------------------------------------------------------------------
constexpr uint32_t kCheckLast = 0x43E00000u;  // 448.0f
constexpr uint32_t kCheckGroups = 1024;

__global__ __launch_bounds__(kThreads) void hw_check_kernel(unsigned long long *counts) {
  const uint32_t stride = gridDim.x * kThreads;
  unsigned long long bad = 0;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b <= kCheckLast; b += stride) {
    const float t = __uint_as_float(b);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.0f, 0, false) & 0xFFu;
    bad += hw != e4m3_rne_sat(t);
  }
  if (bad) atomicAdd(&counts[0], bad);
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g < 127u && __builtin_amdgcn_cvt_f32_fp8((int)g, 0) != e4m3_value(g))
    atomicAdd(&counts[1], 1ull);
}

hipError_t launch_hw_check(unsigned long long *counts) {
  hipLaunchKernelGGL(hw_check_kernel, dim3(kCheckGroups), dim3(kThreads), 0, 0, counts);
  return hipGetLastError();
}

}  // namespace nvfp4

extern "C" {

nvfp4_status nvfp4_hw_self_check(int64_t *counts) {
  if (!counts) return NVFP4_EINVAL;
  unsigned long long *d = nullptr;
  if (hipMalloc(&d, 2 * sizeof(unsigned long long)) != hipSuccess) return NVFP4_EHIP;
  unsigned long long h[2] = {0, 0};
  hipError_t e = hipMemset(d, 0, sizeof(h));
  if (e == hipSuccess) e = nvfp4::launch_hw_check(d);
  if (e == hipSuccess) e = hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost);
  (void)hipFree(d);
  if (e != hipSuccess) return NVFP4_EHIP;
  counts[0] = (int64_t)h[0];
  counts[1] = (int64_t)h[1];
  return NVFP4_OK;
}

}  // extern "C"
