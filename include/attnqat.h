/*
 * attnqat.h -- C ABI of the MI355X (gfx950) NVFP4 fake-quantized attention
 * QAT library (libattnqat.so).
 *
 * The operation is the one defined in "NVFP4 Attention QAT Backward"
 * (cuDNN frontend docs), §Overview, formula block:
 *
 *   Q^, K^, V^ = fake_nvfp4(Q), fake_nvfp4(K), fake_nvfp4(V)
 *   P          = softmax(softmax_scale * Q^ K^T)          (unquantized)
 *   O_hp       = P V^                                     (forward auxiliary)
 *   dS         = P * (dO V^T - rowsum(O_hp * dO))
 *   dQ         = softmax_scale * dS K^,  dK = softmax_scale * dS^T Q^   (STE)
 *   dV         = fake_nvfp4(P)^T dO      (P grouped in 16s along keys)
 *
 * fake_nvfp4 (same page, §Overview): per 16 contiguous values, an E4M3FN
 * block scale s = RNE(amax / 6) (saturating at 448) and E2M1 codes
 * c = RNE(|x| / s) by precise division (exact midpoints round to even),
 * then x^ = sign(x) * c * s.  x^ is exact in bf16.
 *
 * Conventions (after the page's §Class API and §Tensor contract):
 *  - Tensors are contiguous BHSD: (batch, heads, seqlen, head_dim), bf16
 *    (raw 16-bit words), lse fp32 (batch, heads, seqlen_q), natural log.
 *    Every pointer is a device pointer, 16-byte aligned, on the current
 *    HIP device.
 *  - The caller owns every buffer.  No call allocates device memory or keeps
 *    a pointer after it returns; fwd/bwd take a caller-supplied workspace
 *    whose size comes from the *_workspace_bytes queries.
 *  - Calls are asynchronous on the given stream (0 = the null stream).
 *    Buffers belong to the call until the stream has passed it.
 *  - A call only launches kernels on its stream (no allocation, memset or
 *    host synchronization), so calls can be recorded into a HIP graph by
 *    stream capture and replayed; make one call on the device before the
 *    capture (the first call looks up the device's architecture).
 *  - Arguments are validated on the host before anything is enqueued; on
 *    error nothing is launched and outputs are untouched.
 *  - Outputs are fully overwritten, never accumulated into.  Results are
 *    bitwise deterministic (no atomics).
 *  - The library is stateless apart from a per-device architecture check
 *    cache; concurrent calls on different streams are safe when each call
 *    has its own workspace and outputs.
 *  - Limits (§Current support and limitations of the same page, plus
 *    head_dim 64): MHA only, head_dim in {64, 128}, causal is
 *    self-attention only (seqlen_q == seqlen_kv), no dropout, bias,
 *    padding masks or GQA.  NaN/Inf inputs are unsupported.  At most 2^28
 *    rows per tensor (batch * heads * max(seqlen_q, seqlen_kv)).
 */
#ifndef ATTNQAT_H_
#define ATTNQAT_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTNQAT_API __attribute__((visibility("default")))

/* Status codes. */
#define ATTNQAT_OK 0
#define ATTNQAT_ERR_INVALID_ARGUMENT (-1) /* null pointer, size <= 0, non-finite or <= 0 scale */
#define ATTNQAT_ERR_UNSUPPORTED (-2)      /* head_dim, causal cross-attention, > 2^28 rows, device not gfx950 */
#define ATTNQAT_ERR_MISALIGNED (-3)       /* a pointer is not 16-byte aligned */
#define ATTNQAT_ERR_WORKSPACE_TOO_SMALL (-4)
#define ATTNQAT_ERR_HIP (-5)              /* a HIP runtime call or kernel launch failed */

/* Element types for attnqat_fake_nvfp4. */
#define ATTNQAT_DTYPE_BF16 0
#define ATTNQAT_DTYPE_F32 1

/* Which workspace layout attnqat_workspace_layout describes. */
#define ATTNQAT_WS_FWD 0
#define ATTNQAT_WS_BWD 1

/* One attention problem.  softmax_scale must be the forward's (the page's
 * default is 1/sqrt(128)); p_scale pre-scales P before its fake
 * quantization in dV: P^F = fake_nvfp4(p_scale * P) / p_scale.  1.0 is the
 * literal formula; any finite value > 0 is accepted. */
typedef struct attnqat_problem {
  int32_t batch;
  int32_t heads;
  int32_t seqlen_q;
  int32_t seqlen_kv;
  int32_t head_dim; /* 64 or 128 */
  int32_t causal;   /* 0 or 1; 1 requires seqlen_q == seqlen_kv */
  float softmax_scale;
  float p_scale;
} attnqat_problem;

/* Byte offsets into a workspace (see attnqat_workspace_layout).  Absent
 * parts are SIZE_MAX. */
typedef struct attnqat_ws_layout {
  size_t total_bytes;
  size_t q_hat;   /* bf16 (B,H,Nq,D): fake_nvfp4(Q) */
  size_t k_hat;   /* bf16 (B,H,Nkv,D) */
  size_t v_hat;   /* bf16 (B,H,Nkv,D) */
  size_t q_scale; /* uint8 E4M3FN (B,H,Nq,D/16): the block scales of Q^ */
  size_t k_scale; /* uint8 (B,H,Nkv,D/16) */
  size_t v_scale; /* uint8 (B,H,Nkv,D/16) */
  size_t delta;   /* fp32 (B,H,Nq): rowsum(O_hp * dO); backward only */
} attnqat_ws_layout;

/* A short English description of a status code (static storage). */
ATTNQAT_API const char* attnqat_status_string(int status);

/* Library ABI version (major * 100 + minor). */
ATTNQAT_API int attnqat_version(void);

/* Validates a problem on the host only (no HIP call): sizes > 0,
 * head_dim in {64,128}, causal only with seqlen_q == seqlen_kv, finite
 * scales > 0.  Returns ATTNQAT_OK or the error code. */
ATTNQAT_API int attnqat_check_support(const attnqat_problem* p);

/* Checks that HIP device `device` is a gfx950 (MI355X class) GPU.  Returns
 * ATTNQAT_OK, ATTNQAT_ERR_UNSUPPORTED or ATTNQAT_ERR_HIP. */
ATTNQAT_API int attnqat_check_device(int device);

/* Workspace sizes, in bytes, for attnqat_fwd / attnqat_bwd (host only). */
ATTNQAT_API int attnqat_fwd_workspace_bytes(const attnqat_problem* p, size_t* bytes);
ATTNQAT_API int attnqat_bwd_workspace_bytes(const attnqat_problem* p, size_t* bytes);

/* Where each intermediate lives in the fwd (which = ATTNQAT_WS_FWD) or bwd
 * (ATTNQAT_WS_BWD) workspace, so callers can read Q^/K^/V^, their scales
 * and delta after a call (host only). */
ATTNQAT_API int attnqat_workspace_layout(const attnqat_problem* p, int which,
                                         attnqat_ws_layout* out);

/* fake_nvfp4 along rows: x is (rows, row_len) of `dtype` (bf16 or fp32),
 * row_len % 16 == 0, groups of 16 contiguous values along each row.
 * Writes x_hat (same dtype and shape; may alias x) and, when `scales` is
 * not NULL, the E4M3FN byte of every group (rows, row_len/16).  rows == 0
 * is a no-op.  Results are bit-exact to the definition above.  At most
 * 2^35 elements (rows * row_len) per call: beyond that,
 * ATTNQAT_ERR_UNSUPPORTED.  x and x_hat 16-byte aligned.
 * (Page: "NVFP4 Attention QAT Backward", §Overview.) */
ATTNQAT_API int attnqat_fake_nvfp4(const void* x, int dtype, void* x_hat, uint8_t* scales,
                                   int64_t rows, int64_t row_len, hipStream_t stream);

/* Packed NVFP4 storage of a bf16 tensor (rows, row_len), row_len % 16 == 0:
 * the same rounding as attnqat_fake_nvfp4, kept as 4-bit E2M1 codes (bit 3
 * the sign, bits 0-2 the magnitude index into 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 * element 2i in the low nibble and 2i+1 in the high nibble of byte i of the
 * row) in `codes` (rows, row_len/2) and the E4M3FN scale bytes in `scales`
 * (rows, row_len/16); value = code * scale.  4.5 bits per element instead
 * of 16 (Attn-QAT summary, Key claims: the FP4 forward kernel keeps Q and K
 * in block-scaled NVFP4).  x and codes 16-byte aligned; rows == 0 is a
 * no-op; at most 2^35 elements per call (ATTNQAT_ERR_UNSUPPORTED beyond);
 * bit-exact to the definition. */
ATTNQAT_API int attnqat_nvfp4_pack(const void* x, uint8_t* codes, uint8_t* scales,
                                   int64_t rows, int64_t row_len, hipStream_t stream);

/* QAT forward producing the backward's auxiliaries (page §High-level
 * wrapper: O_hp is softmax(Q^ K^T * scale) V^ saved before probability
 * quantization; lse its natural-log log-sum-exp).
 * In: q (B,H,Nq,D), k, v (B,H,Nkv,D) bf16.  Out: o_hp (B,H,Nq,D) bf16,
 * lse (B,H,Nq) fp32.  The workspace (>= attnqat_fwd_workspace_bytes) holds
 * Q^/K^/V^ and their scales afterwards (attnqat_workspace_layout).
 * Few queries, or a short problem: non-causal with at most 32 queries per
 * head, a kernel with 32-query tiles deals the key tiles of each head out
 * to `splits` = min(ceil(512 / (B*H)), max(1, key tiles of 32 / 8))
 * workgroups, which also fake-quantize Q, K and V themselves (each key tile
 * is read once; no separate quantization pass); otherwise (causal too), when the 128-query tiles over all
 * heads number fewer than 256, the keys are split over workgroups (splits =
 * min(ceil(512 / tiles), key tiles / 4), used when >= 2).  Either way a
 * second launch merges the partial results, and the workspace size then
 * includes them (B*H*Nq*splits*(4*D + 8) bytes, after the parts named by
 * attnqat_workspace_layout).  The results are the same forward up to the
 * fp32 rounding order. */
ATTNQAT_API int attnqat_fwd(const attnqat_problem* p, const void* q, const void* k,
                            const void* v, void* o_hp, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* attnqat_fwd with K^ and V^ given in packed NVFP4 storage (for instance a
 * cache written by attnqat_nvfp4_pack): k_codes, v_codes (B,H,Nkv,D/2) and
 * k_scales, v_scales (B,H,Nkv,D/16).  The kernels dequantize them exactly
 * (to bf16, or to fp16 with at most 32 queries per head, where Q^, K^ and
 * V^ are multiplied in fp16: every E2M1 code times an E4M3 scale is exact
 * in both), so they compute attnqat_fwd's o_hp and lse from the same K^/V^
 * values on the K and V the codes were made from: lse equal up to the fp32
 * rounding order, o_hp too, except that with at most 32 queries per head
 * the probabilities enter P V^ rounded to fp16 instead of bf16 (o_hp then
 * differs by up to that bf16 rounding).  q is fake-quantized as in
 * attnqat_fwd (the workspace holds Q^ and its scales afterwards; its K^/V^
 * parts are not written).  Covers the keys as attnqat_fwd does.  With few
 * queries against long K/V, where the forward reads mostly K and V, the
 * packed storage moves 72 instead of 256 bytes per key and head at D = 128.
 * q, the code arrays, o_hp, lse and the workspace 16-byte aligned; errors
 * as attnqat_fwd. */
ATTNQAT_API int attnqat_fwd_packed(const attnqat_problem* p, const void* q,
                                   const uint8_t* k_codes, const uint8_t* k_scales,
                                   const uint8_t* v_codes, const uint8_t* v_scales, void* o_hp,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* The full QAT forward: attnqat_fwd's work plus the quantized, user-visible
 * output O = P^F V^ (Attn-QAT summary, §Method: the FP32 softmax P is
 * fake-quantized to P^F and combined with V^F).  P is the normalized
 * softmax exp(scale Q^ K^T - lse) and P^F = fake_nvfp4(p_scale P) / p_scale
 * in groups of 16 consecutive keys from key 0 (masked keys count as 0) --
 * the P^F whose transpose attnqat_bwd multiplies into dO for dV.  Computed
 * as a second pass over the keys after the first pass has produced lse.
 * Arguments as attnqat_fwd, plus o (B,H,Nq,D) bf16 (16-byte aligned, not
 * aliasing the other buffers).  Errors as attnqat_fwd; a NULL o is
 * ATTNQAT_ERR_INVALID_ARGUMENT. */
ATTNQAT_API int attnqat_fwd_quantized(const attnqat_problem* p, const void* q, const void* k,
                                      const void* v, void* o_hp, float* lse, void* o,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* QAT backward (page §Overview formula block and four-kernel structure:
 * Q fake-quant + delta, K/V fake-quant, dQ, dK/dV).
 * In: q, o_hp, d_o (B,H,Nq,D) bf16; k, v (B,H,Nkv,D) bf16; lse (B,H,Nq)
 * fp32 from the matching forward.  Out: dq (B,H,Nq,D), dk, dv (B,H,Nkv,D)
 * bf16.  The workspace (>= attnqat_bwd_workspace_bytes) holds Q^/K^/V^,
 * their scales and delta afterwards.  Launches: Q fake-quant fused with
 * delta; dK/dV, whose workgroups also fake-quantize the K and V rows of
 * their key block and write K^/V^; then dQ, which reads them.
 * Small problems: when the key blocks of 128 (over all heads) number fewer
 * than 256, the dK/dV kernel splits its query loop over s_kv =
 * min(ceil(256 / key blocks), query sub-tiles of 32 / 4) workgroups (when
 * >= 2); when the query blocks of 128 number fewer than 256, the dQ kernel
 * splits its key loop over s_q = min(ceil(512 / query blocks), key tiles
 * of 32 / 4) workgroups (when >= 2).  The splits write fp32 partial sums
 * (s_q*B*H*Nq*D*4 and s_kv*2*B*H*Nkv*D*4 bytes of the workspace, after the
 * parts named by attnqat_workspace_layout) that a reduction adds up in a
 * fixed order, so results stay deterministic; they equal the unsplit
 * results up to the fp32 rounding order. */
ATTNQAT_API int attnqat_bwd(const attnqat_problem* p, const void* q, const void* k,
                            const void* v, const void* o_hp, const void* d_o,
                            const float* lse, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* attnqat_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results as attnqat_bwd, with the workspace taken from
 * a static device array of ATTNQAT_NOALLOC_MAX_WORKSPACE_BYTES that the
 * library holds on every GPU it runs on until the process ends (its address
 * is looked up once per device, on the first call there).  The call itself
 * allocates nothing.  Where attnqat_bwd_workspace_bytes exceeds that size
 * only because of the small-problem split loops' partial sums, the loops
 * run unsplit; problems that do not fit even so return
 * ATTNQAT_ERR_UNSUPPORTED.  All calls on one GPU share its array:
 * calls that overlap on one GPU (different streams or threads) race and must
 * be serialized by the caller; the array keeps the last call's contents,
 * which no call depends on.  Other arguments and errors as attnqat_bwd. */
#define ATTNQAT_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)64 << 20)
ATTNQAT_API int attnqat_bwd_noalloc(const attnqat_problem* p, const void* q, const void* k,
                                    const void* v, const void* o_hp, const void* d_o,
                                    const float* lse, void* dq, void* dk, void* dv,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTNQAT_H_ */
