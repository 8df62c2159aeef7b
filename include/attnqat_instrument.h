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
 * attnqat_fwd_timed: 4 events; kernel 0 the Q/K/V fake-quant, kernel 1 the
 *   attention forward.
 * attnqat_fwd_quantized_timed: 6 events; kernels 0 and 1 as above, kernel 2
 *   the second (quantized-output) pass.
 * attnqat_bwd_timed: 6 events; kernel 0 the preprocessing (Q fake-quant fused
 *   with delta, and K/V fake-quant, in one launch), kernel 1 dQ, kernel 2
 *   dK/dV.
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

#ifdef __cplusplus
}
#endif

#endif /* ATTNQAT_INSTRUMENT_H_ */
