// NVFP4 fake-quantization kernels (HBM-bound codec work).
//
// One thread owns one group of 16 contiguous values ("NVFP4 Attention QAT
// Backward", §Overview: one E4M3 scale per 16 values); a wave covers 64
// consecutive groups, i.e. 2 KiB of contiguous bf16 input.  k_bwd_codec is
// the backward's preprocessing (same page, §Overview: the fused Q
// fake-quantization / delta kernel); the K/V fake-quantization runs inside the
// dK/dV kernel (each workgroup the rows of its own key block).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kThreads = 256;

struct QuantJobs3 {
  QuantJob job[3];
};

// fake_nvfp4 of group g of job J (g < J.groups)
__device__ __forceinline__ void quant_group(const QuantJob& J, int64_t g) {
  const u32x4* src = reinterpret_cast<const u32x4*>(J.src) + 2 * g;
  u32x4 lo = src[0], hi = src[1];
  float x[16];
  unpack_bf16x16(lo, hi, x);
  const float s = fq16(x);
  pack_bf16x16(x, lo, hi);
  u32x4* dst = reinterpret_cast<u32x4*>(J.dst) + 2 * g;
  dst[0] = lo;
  dst[1] = hi;
  if (J.scales) J.scales[g] = (uint8_t)e4m3_byte(s);
}

__global__ __launch_bounds__(kThreads) void k_quant_bf16(QuantJobs3 jobs) {
  const QuantJob& J = jobs.job[blockIdx.y];
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g < J.groups) quant_group(J, g);
}

// Packed NVFP4 storage: per group of 16 bf16 values, 8 bytes of E2M1 codes
// (element 2i in the low nibble of byte i, 2i+1 in the high nibble) and the
// E4M3FN scale byte.
__global__ __launch_bounds__(kThreads) void k_pack_bf16(QuantJob J, uint8_t* codes) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= J.groups) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(J.src) + 2 * g;
  const u32x4 lo = src[0], hi = src[1];
  float x[16];
  unpack_bf16x16(lo, hi, x);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float s = e4m3_scale_from_amax(amax);
  u32x2 w = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_code(x[i], s) << (4 * (i & 7));
  reinterpret_cast<u32x2*>(codes)[g] = w;
  J.scales[g] = (uint8_t)e4m3_byte(s);
}

__global__ __launch_bounds__(kThreads) void k_quant_f32(QuantJob J) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= J.groups) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(J.src) + 4 * g;
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 v = src[i];
    x[4 * i] = v[0];
    x[4 * i + 1] = v[1];
    x[4 * i + 2] = v[2];
    x[4 * i + 3] = v[3];
  }
  // same device path as the probability quantization of the dK/dV kernel:
  // FMA-refined quotient + hardware E2M1 rounding, applied to |x|
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float s = e4m3_scale_from_amax(amax);
  const FastP fq(s);
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    float y0, y1;
    fq.pair(fabsf(x[i]), fabsf(x[i + 1]), y0, y1);
    x[i] = __builtin_copysignf(y0, x[i]);
    x[i + 1] = __builtin_copysignf(y1, x[i + 1]);
  }
  f32x4* dst = reinterpret_cast<f32x4*>(J.dst) + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 v = {x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
    dst[i] = v;
  }
  if (J.scales) J.scales[g] = (uint8_t)e4m3_byte(s);
}

// Q fake-quant of group g fused with its share of delta = rowsum(O_hp * dO).
// GPR = groups per row (D / 16): 8 for D = 128, 4 for D = 64.  The GPR lanes
// of a row are consecutive and aligned within the wave; the whole wave calls
// this (the row reduction is a cross-lane shuffle), lanes past the end with
// g >= groups.
template <int GPR>
__device__ __forceinline__ void q_delta_group(const QDeltaJob& J, int64_t g) {
  const int64_t groups = J.rows * GPR;
  const bool active = g < groups;
  const int64_t gg = active ? g : 0;
  float part = 0.0f;
  {
    const u32x4* po = reinterpret_cast<const u32x4*>(J.o_hp) + 2 * gg;
    const u32x4* pd = reinterpret_cast<const u32x4*>(J.d_o) + 2 * gg;
    float o[16], d[16];
    unpack_bf16x16(po[0], po[1], o);
    unpack_bf16x16(pd[0], pd[1], d);
#pragma unroll
    for (int i = 0; i < 16; ++i) part = fmaf(o[i], d[i], part);
  }
  if (active) {
    const u32x4* src = reinterpret_cast<const u32x4*>(J.q) + 2 * g;
    u32x4 lo = src[0], hi = src[1];
    float x[16];
    unpack_bf16x16(lo, hi, x);
    const float s = fq16(x);
    pack_bf16x16(x, lo, hi);
    u32x4* dst = reinterpret_cast<u32x4*>(J.q_hat) + 2 * g;
    dst[0] = lo;
    dst[1] = hi;
    J.q_scale[g] = (uint8_t)e4m3_byte(s);
  }
  // reduce the row's partial dot products over its GPR lanes (fixed order)
#pragma unroll
  for (int off = 1; off < GPR; off <<= 1) part += __shfl_xor(part, off, 64);
  if (active && (g % GPR) == 0) J.delta[g / GPR] = part;
}

// Q + delta over all rows; blocks past the end exit.
template <int GPR>
__global__ __launch_bounds__(kThreads) void k_bwd_codec(QDeltaJob qd) {
  const int64_t g0 = (int64_t)blockIdx.x * kThreads;
  if (g0 < qd.rows * GPR) q_delta_group<GPR>(qd, g0 + threadIdx.x);  // uniform per workgroup
}

inline unsigned grid_for(int64_t groups) {
  return (unsigned)((groups + kThreads - 1) / kThreads);
}

}  // namespace

hipError_t launch_quant_bf16(const QuantJob* jobs, int njobs, hipStream_t stream,
                             const LaunchEvents* ev) {
  QuantJobs3 j3 = {};
  int64_t maxg = 0;
  for (int i = 0; i < njobs; ++i) {
    j3.job[i] = jobs[i];
    if (jobs[i].groups > maxg) maxg = jobs[i].groups;
  }
  if (maxg == 0) return hipSuccess;
  return launch(k_quant_bf16, dim3(grid_for(maxg), njobs), dim3(kThreads), stream, ev, j3);
}

hipError_t launch_pack_bf16(const QuantJob& job, uint8_t* codes, hipStream_t stream) {
  if (job.groups == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_bf16, dim3(grid_for(job.groups)), dim3(kThreads), 0, stream, job,
                     codes);
  return hipGetLastError();
}

hipError_t launch_quant_f32(const QuantJob& job, hipStream_t stream) {
  if (job.groups == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_f32, dim3(grid_for(job.groups)), dim3(kThreads), 0, stream, job);
  return hipGetLastError();
}

hipError_t launch_bwd_codec(const QDeltaJob& qd, int head_dim, hipStream_t stream,
                            const LaunchEvents* ev) {
  const int gpr = head_dim / 16;
  const int64_t groups = qd.rows * gpr;
  if (groups == 0) return hipSuccess;
  const dim3 grid(grid_for(groups));
  if (gpr == 8) return launch(k_bwd_codec<8>, grid, dim3(kThreads), stream, ev, qd);
  return launch(k_bwd_codec<4>, grid, dim3(kThreads), stream, ev, qd);
}

}  // namespace attnqat
