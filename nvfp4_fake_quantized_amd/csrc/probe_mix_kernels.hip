// Measurement kernels (declared in attnqat_instrument.h): how MFMA and VALU
// instructions share a SIMD, and the LDS bank behaviour of write patterns.
// The AGPR-accumulator MFMAs are inline assembly (the compiler chooses the
// accumulator form per function); their hazards are handled where noted.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

// ---- MFMA / VALU issue mix --------------------------------------------------

// One MFMA into an accumulator held in VGPRs (the compiler's choice for these
// kernels) or, with AG, in AGPRs.  The AGPR form is written as inline
// assembly: the compiler picks the accumulator form per function.
template <bool AG>
__device__ __forceinline__ f32x16 probe_mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (AG) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
  } else {
    return mfma32x32x16(a, b, c);
  }
}

// MODE 0: MFMAs only; 1: VALU only; 2: both, interleaved in every wave (NV
// fp32 FMAs after each MFMA); 3 (512 threads): waves 0-3 MFMAs only, waves
// 4-7 VALU only -- waves w and w + 4 of a workgroup share a SIMD, so every
// SIMD runs one wave of each.  Each wave runs iters * 8 MFMA slots into two
// accumulator chains; the FMAs form 8 independent chains.
template <int MODE, int NV, bool AG>
__global__ __launch_bounds__(512) void k_issue_mix(const uint16_t* in, float* out, int iters) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int wave = threadIdx.x >> 6;
  const bool do_m = MODE == 0 || MODE == 2 || (MODE == 3 && wave < 4);
  const bool do_v = MODE == 1 || MODE == 2 || (MODE == 3 && wave >= 4);
  const bf16x8 A = ld_bf16x8(in + 8 * (t & 1023));
  const bf16x8 B = ld_bf16x8(in + 8 * ((t + 5) & 1023));
  f32x16 acc0 = zero_f32x16(), acc1 = zero_f32x16();
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 1e-3f * (float)((t + i) & 255);
  const float c0 = 0.999f, c1 = 1e-4f;
  if (do_m && do_v) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k & 1) acc1 = probe_mfma<AG>(A, B, acc1);
        else acc0 = probe_mfma<AG>(A, B, acc0);
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j & 7] = __builtin_fmaf(v[j & 7], c0, c1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if (do_m) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k & 1) acc1 = probe_mfma<AG>(A, B, acc1);
        else acc0 = probe_mfma<AG>(A, B, acc0);
      }
    }
  } else if (do_v) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j & 7] = __builtin_fmaf(v[j & 7], c0, c1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // results of inline-assembly MFMAs are not tracked by the compiler's hazard
  // checks: let the last ones retire before the accumulators are read
  if constexpr (AG) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += v[i];
  out[t] = s;
}

template <int MODE, int NV>
hipError_t launch_issue_mix_m(bool agpr, const uint16_t* in, float* out, int blocks, int threads,
                              int iters, hipStream_t stream) {
  if (agpr)
    return launch(k_issue_mix<MODE, NV, true>, dim3(blocks), dim3(threads), stream, nullptr, in,
                  out, iters);
  return launch(k_issue_mix<MODE, NV, false>, dim3(blocks), dim3(threads), stream, nullptr, in,
                out, iters);
}

// ---- LDS write patterns --------------------------------------------------------

// Element offset (16-bit elements) of the write of lane `lane`, slot i (0..3),
// in a 4 KiB per-wave region, for the patterns documented in
// attnqat_instrument.h.  Each pattern stays below element 1024.
template <int P>
__device__ __forceinline__ int lds_pattern_offset(int lane, int i) {
  const int r = lane & 31, h = lane >> 5;
  if constexpr (P == 0) return 4 * lane + 256 * (i & 1);                    // 8 B, linear
  else if constexpr (P == 1) return r * 32 + 16 * h + 4 * i;                // 8 B, rows of 64 B
  else if constexpr (P == 2) return r * 32 + ((16 * h + 4 * i) ^ (4 * ((r >> 2) & 7)));
  else if constexpr (P == 3) return 8 * lane;                               // 16 B, linear
  else if constexpr (P == 4) return r * 32 + 8 * (((2 * h + (i & 1))) ^ ((r >> 2) & 3));
  else return r * 32 + 8 * (((2 * h + (i & 1))) ^ ((r >> 1) & 3));         // 16 B, row pairs
}

template <int P>
__global__ __launch_bounds__(256) void k_lds_write(float* out, int iters) {
  constexpr bool W16 = P >= 3;
  __shared__ __attribute__((aligned(16))) uint16_t buf[4][2048];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t* tile = buf[wave];
  u32x4 v = {(uint32_t)lane, 1u, 2u, (uint32_t)blockIdx.x};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = lds_pattern_offset<P>(lane, i);
      if constexpr (W16) *reinterpret_cast<u32x4*>(tile + o) = v;
      else *reinterpret_cast<u32x2*>(tile + o) = u32x2{v[0], v[1]};
      v[0] += 1u;
      // keep every store: no merging or elimination across slots
      asm volatile("" ::: "memory");
    }
  }
  __syncthreads();
  out[blockIdx.x * 256 + threadIdx.x] = (float)tile[4 * lane];
}

template <int P>
hipError_t launch_lds_write_p(float* out, int blocks, int iters, hipStream_t stream) {
  return launch(k_lds_write<P>, dim3(blocks), dim3(256), stream, nullptr, out, iters);
}

}  // namespace

hipError_t launch_issue_mix(int mode, int valu_per_mfma, bool agpr, const uint16_t* in,
                            float* out, int blocks, int threads, int iters,
                            hipStream_t stream) {
  const bool v16 = valu_per_mfma == 16;
  switch (mode) {
    case 0: return launch_issue_mix_m<0, 8>(agpr, in, out, blocks, threads, iters, stream);
    case 1:
      return v16 ? launch_issue_mix_m<1, 16>(agpr, in, out, blocks, threads, iters, stream)
                 : launch_issue_mix_m<1, 8>(agpr, in, out, blocks, threads, iters, stream);
    case 2:
      return v16 ? launch_issue_mix_m<2, 16>(agpr, in, out, blocks, threads, iters, stream)
                 : launch_issue_mix_m<2, 8>(agpr, in, out, blocks, threads, iters, stream);
    default:
      return v16 ? launch_issue_mix_m<3, 16>(agpr, in, out, blocks, threads, iters, stream)
                 : launch_issue_mix_m<3, 8>(agpr, in, out, blocks, threads, iters, stream);
  }
}

hipError_t launch_lds_write(int pattern, float* out, int blocks, int iters, hipStream_t stream) {
  switch (pattern) {
    case 0: return launch_lds_write_p<0>(out, blocks, iters, stream);
    case 1: return launch_lds_write_p<1>(out, blocks, iters, stream);
    case 2: return launch_lds_write_p<2>(out, blocks, iters, stream);
    case 3: return launch_lds_write_p<3>(out, blocks, iters, stream);
    case 4: return launch_lds_write_p<4>(out, blocks, iters, stream);
    default: return launch_lds_write_p<5>(out, blocks, iters, stream);
  }
}

}  // namespace attnqat
