// Matrix-core rate probe (calibration, not part of the method): each wave issues `iters` rounds of
// four independent v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic in the
// loop. Timed over a launch that fills every compute unit with two waves per SIMD, it measures the
// bf16 matrix-core rate the part sustains at the clock it holds under that load, next to which the
// 2.4 GHz specification figure (256 CUs x 4096 FLOP per clock) can be read.
#include <hip/hip_runtime.h>

#include "k2_device.h"
#include "k2_kernels.h"

namespace k2 {

__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(0.001f * (lane + e));
    b[e] = (bf16)(0.002f * (lane - e));
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  // keeps the products live; the stored value is never expected to be read
  if (threadIdx.x == 0 && blockIdx.x == 0) out[0] = s;
}

hipError_t mfma_probe(int iters, int blocks, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace k2
