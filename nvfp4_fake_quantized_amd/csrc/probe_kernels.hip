// Measurement kernel (declared in attnqat_instrument.h): the sustained bf16
// MFMA rate of the device, the reference against which the attention
// kernels' MFMA rates are read.  (The compiler keeps its four accumulator
// chains in AGPRs.)
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kProbeThreads = 256;

// Each wave loads four A and four B operands of its own (so that operands
// differ between MFMAs, waves and lanes, as in the attention kernels), then
// issues iters * 16 v_mfma_f32_32x32x16_bf16 into four independent
// accumulator chains, cycling through the operand pairs.
__global__ __launch_bounds__(kProbeThreads) void k_mfma_peak(const uint16_t* a, const uint16_t* b,
                                                              float* out, int iters) {
  const int64_t t = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  bf16x8 A[4], Bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    A[i] = ld_bf16x8(a + (t * 4 + i) * 8);
    Bv[i] = ld_bf16x8(b + (t * 4 + i) * 8);
  }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero_f32x16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i & 3] = mfma32x32x16(A[i & 3], Bv[(i >> 2) & 3], acc[i & 3]);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
  out[t] = s;
}

}  // namespace

hipError_t launch_mfma_peak(const uint16_t* a, const uint16_t* b, float* out, int blocks,
                            int iters, hipStream_t stream) {
  hipLaunchKernelGGL(k_mfma_peak, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream, a, b,
                     out, iters);
  return hipGetLastError();
}

}  // namespace attnqat
