// Host-side launchers of the attnqat kernels.  Each returns hipSuccess or the
// launch error; arguments are validated by the C-ABI layer beforehand.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace attnqat {

// Optional start/stop events of one launch.  hipExtLaunchKernel has the
// dispatch itself record them (kernel start and end timestamps), so timing a
// kernel adds no packets to the stream and no gap between kernels.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename... Params, size_t... I>
inline hipError_t launch_packed(void (*kernel)(Params...), dim3 grid, dim3 block,
                                hipStream_t stream, const LaunchEvents* ev,
                                std::tuple<Params...>& values, std::index_sequence<I...>) {
  void* args[] = {static_cast<void*>(&std::get<I>(values))...};
  if (ev == nullptr)
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream,
                            ev->start, ev->stop, 0);
}

// Launches kernel<<<grid, block, 0, stream>>>(args...), with ev's events when
// ev is given; returns the launch status.
template <typename... Params, typename... Args>
inline hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream,
                         const LaunchEvents* ev, Args&&... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  std::tuple<Params...> values(std::forward<Args>(args)...);
  return launch_packed(kernel, grid, block, stream, ev, values,
                       std::index_sequence_for<Params...>{});
}

// Per-problem pointers and sizes passed to the attention kernels.  All
// tensors are contiguous BHSD; bf16 tensors are raw 16-bit words.
struct AttnArgs {
  const uint16_t* q_hat;  // (BH, nq, D)
  const uint16_t* k_hat;  // (BH, nkv, D)
  const uint16_t* v_hat;  // (BH, nkv, D)
  const uint16_t* d_o;    // (BH, nq, D)       backward only
  const float* lse;       // (BH, nq)          backward input / forward output
  const float* delta;     // (BH, nq)          backward only
  uint16_t* o_hp;         // (BH, nq, D)       forward output
  float* lse_out;         // (BH, nq)          forward output
  uint16_t* dq;           // (BH, nq, D)
  uint16_t* dk;           // (BH, nkv, D)
  uint16_t* dv;           // (BH, nkv, D)
  uint16_t* o_q;          // (BH, nq, D)       quantized forward output (second pass)
  const uint8_t* k_codes;   // (BH, nkv, D/2)  packed NVFP4 K^ (forward from packed K/V)
  const uint8_t* k_scales;  // (BH, nkv, D/16)
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  // forward split over keys (kv_splits > 1): per split, unnormalized O^T
  // (fp32) and the exponent base and sum, merged by a second kernel
  float* o_part;          // (BH, kv_splits, nq, D)
  float* ml_part;         // (BH, kv_splits, nq, 2): base (log2 units), sum
  int kv_splits;          // 0 or 1: no split
  int kv_decode;          // 1: 32-query tiles (k_fwd_dec), kv_splits >= 1 key runs
  // k_fwd and k_fwd_dec: when q_in is set, the kernel fake-quantizes its Q
  // rows itself and the first key run of each query tile writes Q^ and its
  // scale bytes to q_hat_out / q_scale_out
  const uint16_t* q_in;   // (BH, nq, D) bf16
  uint16_t* q_hat_out;
  uint8_t* q_scale_out;   // (BH, nq, D/16)
  // k_dkdv and k_fwd_dec (from bf16 K/V): when k_in is set, the kernel
  // fake-quantizes the K and V rows it owns (k_dkdv: its key block, whose
  // first query run writes them; k_fwd_dec: its key tiles) and writes K^, V^
  // and their scale bytes (k_dq, which runs after k_dkdv, reads them)
  const uint16_t* k_in;   // (BH, nkv, D) bf16
  const uint16_t* v_in;
  uint16_t* k_hat_out;
  uint16_t* v_hat_out;
  uint8_t* k_scale_out;   // (BH, nkv, D/16)
  uint8_t* v_scale_out;
  // backward over few tiles: the key loop of k_dq split over dq_splits
  // workgroups and the query loop of k_dkdv over dkdv_splits, each writing
  // fp32 partial sums that a reduction adds up in a fixed order
  float* dq_part;         // (dq_splits, BH, nq, D)
  float* dkdv_part;       // (dkdv_splits, 2, BH, nkv, D): dK, then dV, unscaled
  int dq_splits;          // 0 or 1: no split
  int dkdv_splits;
  int bh;                 // batch * heads
  int nq, nkv;
  int causal;
  float softmax_scale;
  float p_scale;
};

// One tensor to fake-quantize along its contiguous dim in groups of 16.
struct QuantJob {
  const void* src;
  void* dst;
  uint8_t* scales;  // may be null
  int64_t groups;   // number of 16-element groups
};

// fake_nvfp4 over up to three bf16 tensors in one launch.
hipError_t launch_quant_bf16(const QuantJob* jobs, int njobs, hipStream_t stream,
                             const LaunchEvents* ev = nullptr);
// Packed NVFP4 codes (2 per byte) and scale bytes of one bf16 tensor.
hipError_t launch_pack_bf16(const QuantJob& job, uint8_t* codes, hipStream_t stream);
// fake_nvfp4 over one fp32 tensor.
hipError_t launch_quant_f32(const QuantJob& job, hipStream_t stream);
// The backward's preprocessing: Q fake-quant fused with
// delta = rowsum(O_hp * dO) (fp32); D in {64, 128}.
struct QDeltaJob {
  const uint16_t* q;
  const uint16_t* o_hp;
  const uint16_t* d_o;
  uint16_t* q_hat;
  uint8_t* q_scale;
  float* delta;
  int64_t rows;  // batch * heads * seqlen_q
};
hipError_t launch_bwd_codec(const QDeltaJob& qd, int head_dim, hipStream_t stream,
                            const LaunchEvents* ev = nullptr);

hipError_t launch_fwd(const AttnArgs& a, int head_dim, hipStream_t stream,
                      const LaunchEvents* ev = nullptr);
// The same forward with K^ and V^ given as packed NVFP4 (a.k_codes ...).
hipError_t launch_fwd_packed(const AttnArgs& a, int head_dim, hipStream_t stream);
// O = P^F V^ from Q^, K^, V^ and the forward's lse (a.lse), into a.o_q.
hipError_t launch_fwd_out(const AttnArgs& a, int head_dim, hipStream_t stream,
                          const LaunchEvents* ev = nullptr);
hipError_t launch_bwd_dq(const AttnArgs& a, int head_dim, hipStream_t stream,
                         const LaunchEvents* ev = nullptr);
// One sum of split partials: out[i] = bf16(scale * sum_s part[s * stride + i])
// for i < n (n % 4 == 0), s = 0 .. splits-1 in order.
struct SumJob {
  const float* part;
  uint16_t* out;
  int64_t stride, n;
  int splits;
  float scale;
};
// Up to three sums (dQ, dK, dV) in one launch.
hipError_t launch_sum_parts(const SumJob* jobs, int njobs, hipStream_t stream,
                            const LaunchEvents* ev = nullptr);
hipError_t launch_bwd_dkdv(const AttnArgs& a, int head_dim, hipStream_t stream,
                           const LaunchEvents* ev = nullptr);
// Sustained bf16 MFMA rate probe: blocks of 256 threads, each thread reading
// 32 bf16 of a and of b at offset 32 * thread.
hipError_t launch_mfma_peak(const uint16_t* a, const uint16_t* b, float* out, int blocks,
                            int iters, hipStream_t stream);
// MFMA / VALU issue-mix probe (mode 0..3, valu_per_mfma 8 or 16), blocks of
// `threads` (256 or 512) threads; in holds >= 8192 bf16, out >= blocks*threads.
hipError_t launch_issue_mix(int mode, int valu_per_mfma, bool agpr, const uint16_t* in,
                            float* out, int blocks, int threads, int iters, hipStream_t stream);
// LDS write-pattern probe (pattern 0..5), blocks of 256 threads; out >=
// blocks*256 floats.
hipError_t launch_lds_write(int pattern, float* out, int blocks, int iters, hipStream_t stream);

}  // namespace attnqat
