// Practical dense bf16 MFMA rate of the device: every wave runs a long chain
// of independent v_mfma_f32_32x32x16_bf16 on register operands (eight
// accumulators, so no MFMA waits for another), two waves per SIMD on every
// CU. The reported rate is the ceiling the layer's kernels can approach under
// the device's clock and power behaviour, next to the datasheet figure.
#pragma once

#include "device_common.hpp"

namespace bpt {

__device__ float g_peak_sink;

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float seed) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(seed * (float)(lane + e));
    b[e] = (bf16)(seed * (float)(lane - e));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mma(a, b, acc[j]);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[j][r];
  if (sum == 12345.678f) g_peak_sink = sum;  // keeps the chain live; practically never taken
}

}  // namespace bpt
