/*
 * attnqat_instrument.h -- measurement entry points of libattnqat.so.
 *
 * These are not part of the operation's interface (attnqat.h): they run the
 * same kernels as attnqat_fwd, attnqat_fwd_quantized and attnqat_bwd and
 * additionally have each launch record caller-created HIP events, for
 * benchmarks that time each kernel of the backward ("NVFP4 Attention QAT
 * Backward", §Overview) without synchronizing inside the call.
 * Conventions, arguments and errors as in attnqat.h.
 */
#ifndef ATTNQAT_INSTRUMENT_H_
#define ATTNQAT_INSTRUMENT_H_

#include "attnqat.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Instrumented variants for measurement: identical work and results, and
 * each kernel launch has its dispatch record a caller-created start and stop
 * event (hipExtLaunchKernel), so per-kernel durations can be read with
 * hipEventElapsedTime(events[2i], events[2i+1]) without synchronizing inside
 * the call and without extra packets or gaps between the kernels.
 * attnqat_fwd_timed: 4 events; kernel 0 the Q/K/V fake-quant (K/V only at
 *   head_dim 128, where the attention kernel quantizes Q; an empty span when
 *   the forward takes 32-query tiles, which quantize Q, K and V inside the
 *   attention kernel), kernel 1 the attention forward (when the forward
 *   covers the keys in runs -- see attnqat_fwd -- its pair spans the
 *   attention launch and the merge launch).
 * attnqat_fwd_quantized_timed: 6 events; kernels 0 and 1 as above, kernel 2
 *   the second (quantized-output) pass.
 * attnqat_bwd_timed: 6 events; kernel 0 the preprocessing (Q fake-quant fused
 *   with delta), kernel 1 dQ (on small problems with split loops -- see
 *   attnqat_bwd -- its pair also spans the launch that adds the partial sums
 *   of dQ, dK and dV), kernel 2 dK/dV with the K/V fake-quant (launched
 *   before dQ).
 * A NULL array or NULL event is ATTNQAT_ERR_INVALID_ARGUMENT. */
ATTNQAT_API int attnqat_fwd_timed(const attnqat_problem* p, const void* q, const void* k,
                                  const void* v, void* o_hp, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream,
                                  hipEvent_t* events);
ATTNQAT_API int attnqat_fwd_quantized_timed(const attnqat_problem* p, const void* q,
                                            const void* k, const void* v, void* o_hp,
                                            float* lse, void* o, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream,
                                            hipEvent_t* events);
ATTNQAT_API int attnqat_bwd_timed(const attnqat_problem* p, const void* q, const void* k,
                                  const void* v, const void* o_hp, const void* d_o,
                                  const float* lse, void* dq, void* dk, void* dv,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream,
                                  hipEvent_t* events);

/* The device's sustained bf16 MFMA rate on changing operands: `blocks`
 * workgroups of 256 threads, each thread reading 32 bf16 values of a and of b
 * at offset 32 * (global thread index) as MFMA operands, then issuing
 * iters * 16 v_mfma_f32_32x32x16_bf16 (32768 flops each per wave) into four
 * independent accumulator chains and writing one float per thread to out.
 * The caller times the call (e.g. with events around it): flops =
 * blocks * 4 * iters * 16 * 32768.  a, b hold >= 32 * 256 * blocks bf16 each,
 * out >= 256 * blocks floats, all 16-byte aligned; blocks in [1, 2^20],
 * iters in [1, 2^20], else ATTNQAT_ERR_INVALID_ARGUMENT. */
ATTNQAT_API int attnqat_probe_mfma_peak(const void* a, const void* b, float* out, int blocks,
                                        int iters, hipStream_t stream);

/* How MFMA and VALU instructions share a SIMD: `blocks` workgroups of
 * `threads` (256: one wave per SIMD, 512: two) threads; every wave runs
 * iters * 8 slots.  mode 0: one v_mfma_f32_32x32x16_bf16 per slot (two
 * accumulator chains); 1: valu_per_mfma (8 or 16) independent fp32 FMAs per
 * slot; 2: both in every wave, interleaved; 3 (threads = 512 only): waves
 * 0-3 the MFMAs, waves 4-7 the FMAs, so that each SIMD runs one wave of each
 * (waves w and w + 4 share a SIMD).  agpr != 0 keeps the MFMA accumulators in AGPRs instead of
 * VGPRs.  Operands are read from `in` (>= 8192 bf16); one float per thread is
 * written to out (>= blocks * threads floats).  The caller times the call.
 * Out-of-range arguments: ATTNQAT_ERR_INVALID_ARGUMENT. */
ATTNQAT_API int attnqat_probe_issue_mix(int mode, int valu_per_mfma, int agpr, const void* in,
                                        float* out, int blocks, int threads, int iters,
                                        hipStream_t stream);

/* LDS write patterns, for bank-conflict counters (SQ_LDS_BANK_CONFLICT):
 * `blocks` workgroups of 256 threads; every wave writes 4 stores per
 * iteration into its own 4 KiB region, lane l at row r = l % 32, half
 * h = l / 32, store i:
 *   0: 8-byte stores at byte 8l (+512 for odd i)           linear
 *   1: 8-byte stores, row r of 64 bytes, column 16h + 4i    unswizzled rows
 *   2: as 1 with the column XOR 4 * ((r >> 2) & 7)
 *   3: 16-byte stores at byte 16l                           linear
 *   4: 16-byte stores, row r of 64 bytes, 16-byte chunk (2h + i % 2) XOR ((r >> 2) & 3)
 *   5: as 4 with the chunk XOR ((r >> 1) & 3)  (the dK/dV kernel's tiles)
 * out >= blocks * 256 floats.  The caller times the call. */
ATTNQAT_API int attnqat_probe_lds_write(int pattern, float* out, int blocks, int iters,
                                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTNQAT_INSTRUMENT_H_ */
