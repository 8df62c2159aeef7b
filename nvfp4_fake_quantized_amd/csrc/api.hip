// C ABI of libattnqat.so: host-side validation, workspace layout and the
// ordered kernel launches (declared in include/attnqat.h).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "attnqat.h"
#include "attnqat_instrument.h"
#include "kernels.hpp"

namespace {

using attnqat::AttnArgs;
using attnqat::QuantJob;

constexpr size_t kAlign = 256;
// Codec calls: at most 2^35 elements, so that every codec launch stays below
// 2^32 threads (one thread per 16 values for the fp32 and packing kernels).
constexpr int64_t kMaxCodecElements = (int64_t)1 << 35;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate_problem(const attnqat_problem* p) {
  if (p == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (p->batch <= 0 || p->heads <= 0 || p->seqlen_q <= 0 || p->seqlen_kv <= 0 ||
      p->head_dim <= 0)
    return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (!(isfinite(p->softmax_scale) && p->softmax_scale > 0.0f)) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (!(isfinite(p->p_scale) && p->p_scale > 0.0f)) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (p->causal != 0 && p->causal != 1) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (p->head_dim != 64 && p->head_dim != 128) return ATTNQAT_ERR_UNSUPPORTED;
  if (p->causal && p->seqlen_q != p->seqlen_kv) return ATTNQAT_ERR_UNSUPPORTED;
  // launch sizes: the codec launch has one thread per 16 values of a tensor
  // (grid.x * block.x < 2^32); 2^28 rows is beyond what fits the device anyway
  const int64_t rows = (int64_t)p->batch * p->heads *
                       (p->seqlen_q > p->seqlen_kv ? p->seqlen_q : p->seqlen_kv);
  if (rows > (int64_t)1 << 28) return ATTNQAT_ERR_UNSUPPORTED;
  return ATTNQAT_OK;
}

struct Layout {
  size_t q_hat, k_hat, v_hat, q_scale, k_scale, v_scale, delta, o_part, ml_part, dq_part,
      dkdv_part, total;
  int kv_splits;
  int kv_decode;
  int dq_splits, dkdv_splits;
};

// Backward over few tiles.  k_dkdv runs one workgroup of 128 keys per CU and
// k_dq two of 128 queries; when a problem has fewer key blocks (or query
// blocks) than CUs the chip is underfilled, so the query loop of k_dkdv is
// split over up to ceil(256 / key blocks) workgroups (at least 4 sub-tiles
// of 32 queries each) and the key loop of k_dq over up to
// ceil(512 / query blocks) (at least 4 key tiles of 32 each).  (Measured:
// the splits pay on the smallest grids; at 256 query blocks, one per CU,
// a dQ split already costs more in partial sums than it gains.)  Their fp32 partial sums take splits * B*H*N*D*4 bytes (dK and dV:
// twice that) of the backward workspace.
struct BwdPlan {
  int dq_splits, dkdv_splits;
};
BwdPlan bwd_plan(const attnqat_problem* p) {
  const int64_t bh = (int64_t)p->batch * p->heads;
  const int64_t kblocks = bh * (((int64_t)p->seqlen_kv + 127) / 128);
  const int64_t qblocks = bh * (((int64_t)p->seqlen_q + 127) / 128);
  const int64_t qsub = ((int64_t)p->seqlen_q + 31) / 32;   // query sub-tiles of a key block
  const int64_t ktiles = ((int64_t)p->seqlen_kv + 31) / 32;  // key tiles of a query block
  BwdPlan b = {1, 1};
  if (kblocks < 256) {
    const int64_t want = (256 + kblocks - 1) / kblocks, cap = qsub / 4;
    const int64_t s = want < cap ? want : cap;
    b.dkdv_splits = s >= 2 ? (int)s : 1;
  }
  if (qblocks < 256) {
    const int64_t want = (512 + qblocks - 1) / qblocks, cap = ktiles / 4;
    const int64_t s = want < cap ? want : cap;
    b.dq_splits = s >= 2 ? (int)s : 1;
  }
  return b;
}

// How the forward covers the keys:
//  * non-causal, at most 32 queries per head: the 32-query-tile forward, its key tiles
//    dealt out to `splits` workgroups of 4 waves per head, enough for about
//    512 workgroups (two per CU) with at least 2 key tiles (64 keys) per
//    wave;
//  * otherwise (causal too), when the 128-query tiles of all heads cannot
//    fill the chip's 256 CUs: the keys are split so that about 512
//    workgroups run, with at least 4 key tiles (128 keys) per split (causal:
//    of the last query tile's keys; earlier tiles' later splits get none);
// Both write per-run partial results (unnormalized O in fp32, the run's
// exponent base and sum) of bh * splits * Nq * (4 D + 8) bytes to the
// forward workspace.
struct FwdPlan {
  int splits;
  int decode;
};
FwdPlan fwd_plan(const attnqat_problem* p) {
  const int64_t bh = (int64_t)p->batch * p->heads;
  const int64_t ktiles = ((int64_t)p->seqlen_kv + 31) / 32;
  if (!p->causal && p->seqlen_q <= 32) {
    const int64_t want = (512 + bh - 1) / bh;
    const int64_t cap = ktiles / 8 > 1 ? ktiles / 8 : 1;
    return {(int)(want < cap ? want : cap), 1};
  }
  const int64_t wgs = bh * ((p->seqlen_q + 127) / 128);
  if (wgs >= 256) return {1, 0};
  const int64_t want = (512 + wgs - 1) / wgs;
  const int64_t s = want < ktiles / 4 ? want : ktiles / 4;
  return {s >= 2 ? (int)s : 1, 0};
}

// split_ok = false: the backward without split loops (no partial sums).
Layout make_layout(const attnqat_problem* p, bool bwd, bool split_ok = true) {
  const size_t bh = (size_t)p->batch * p->heads;
  const size_t nq = bh * p->seqlen_q, nkv = bh * p->seqlen_kv;
  const size_t D = p->head_dim;
  Layout L;
  size_t off = 0;
  L.q_hat = off;   off = align_up(off + nq * D * 2);
  L.k_hat = off;   off = align_up(off + nkv * D * 2);
  L.v_hat = off;   off = align_up(off + nkv * D * 2);
  L.q_scale = off; off = align_up(off + nq * D / 16);
  L.k_scale = off; off = align_up(off + nkv * D / 16);
  L.v_scale = off; off = align_up(off + nkv * D / 16);
  L.o_part = L.ml_part = L.dq_part = L.dkdv_part = SIZE_MAX;
  L.kv_splits = 1;
  L.kv_decode = 0;
  L.dq_splits = L.dkdv_splits = 1;
  if (bwd) {
    L.delta = off;
    off = align_up(off + nq * 4);
    const BwdPlan plan = split_ok ? bwd_plan(p) : BwdPlan{1, 1};
    L.dq_splits = plan.dq_splits;
    L.dkdv_splits = plan.dkdv_splits;
    if (L.dq_splits > 1) {
      L.dq_part = off;
      off = align_up(off + (size_t)L.dq_splits * nq * D * 4);
    }
    if (L.dkdv_splits > 1) {
      L.dkdv_part = off;
      off = align_up(off + (size_t)L.dkdv_splits * 2 * nkv * D * 4);
    }
  } else {
    L.delta = SIZE_MAX;
    const FwdPlan plan = fwd_plan(p);
    L.kv_splits = plan.splits;
    L.kv_decode = plan.decode;
    if (L.kv_splits > 1 || L.kv_decode) {
      L.o_part = off;
      off = align_up(off + nq * L.kv_splits * D * 4);
      L.ml_part = off;
      off = align_up(off + nq * L.kv_splits * 8);
    }
  }
  L.total = off;
  return L;
}

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
int8_t g_arch_state[256];

int device_status() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTNQAT_ERR_HIP;
  return attnqat_check_device(dev);
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off);
}

}  // namespace

extern "C" {

const char* attnqat_status_string(int status) {
  switch (status) {
    case ATTNQAT_OK: return "ok";
    case ATTNQAT_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ATTNQAT_ERR_UNSUPPORTED: return "unsupported problem or device";
    case ATTNQAT_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case ATTNQAT_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ATTNQAT_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int attnqat_version(void) { return 100; }

int attnqat_check_support(const attnqat_problem* p) { return validate_problem(p); }

int attnqat_check_device(int device) {
  if (device < 0 || device >= 256) return ATTNQAT_ERR_INVALID_ARGUMENT;
  const int8_t st = __atomic_load_n(&g_arch_state[device], __ATOMIC_RELAXED);
  if (st == 1) return ATTNQAT_OK;
  if (st == 2) return ATTNQAT_ERR_UNSUPPORTED;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return ATTNQAT_ERR_HIP;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  __atomic_store_n(&g_arch_state[device], (int8_t)(ok ? 1 : 2), __ATOMIC_RELAXED);
  return ok ? ATTNQAT_OK : ATTNQAT_ERR_UNSUPPORTED;
}

int attnqat_fwd_workspace_bytes(const attnqat_problem* p, size_t* bytes) {
  const int st = validate_problem(p);
  if (st != ATTNQAT_OK) return st;
  if (bytes == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  *bytes = make_layout(p, false).total;
  return ATTNQAT_OK;
}

int attnqat_bwd_workspace_bytes(const attnqat_problem* p, size_t* bytes) {
  const int st = validate_problem(p);
  if (st != ATTNQAT_OK) return st;
  if (bytes == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  *bytes = make_layout(p, true).total;
  return ATTNQAT_OK;
}

int attnqat_workspace_layout(const attnqat_problem* p, int which, attnqat_ws_layout* out) {
  const int st = validate_problem(p);
  if (st != ATTNQAT_OK) return st;
  if (out == nullptr || (which != ATTNQAT_WS_FWD && which != ATTNQAT_WS_BWD))
    return ATTNQAT_ERR_INVALID_ARGUMENT;
  const Layout L = make_layout(p, which == ATTNQAT_WS_BWD);
  out->total_bytes = L.total;
  out->q_hat = L.q_hat;
  out->k_hat = L.k_hat;
  out->v_hat = L.v_hat;
  out->q_scale = L.q_scale;
  out->k_scale = L.k_scale;
  out->v_scale = L.v_scale;
  out->delta = L.delta;
  return ATTNQAT_OK;
}

int attnqat_fake_nvfp4(const void* x, int dtype, void* x_hat, uint8_t* scales, int64_t rows,
                       int64_t row_len, hipStream_t stream) {
  if (dtype != ATTNQAT_DTYPE_BF16 && dtype != ATTNQAT_DTYPE_F32) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (rows < 0 || row_len <= 0 || (row_len % 16) != 0) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (rows > kMaxCodecElements / row_len) return ATTNQAT_ERR_UNSUPPORTED;
  if (rows == 0) return ATTNQAT_OK;
  if (x == nullptr || x_hat == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(x_hat)) return ATTNQAT_ERR_MISALIGNED;
  const int dst = device_status();
  if (dst != ATTNQAT_OK) return dst;
  (void)hipGetLastError();
  QuantJob job{x, x_hat, scales, rows * (row_len / 16)};
  const hipError_t e = dtype == ATTNQAT_DTYPE_BF16 ? attnqat::launch_quant_bf16(&job, 1, stream)
                                                   : attnqat::launch_quant_f32(job, stream);
  return e == hipSuccess ? ATTNQAT_OK : ATTNQAT_ERR_HIP;
}

int attnqat_nvfp4_pack(const void* x, uint8_t* codes, uint8_t* scales, int64_t rows,
                       int64_t row_len, hipStream_t stream) {
  if (rows < 0 || row_len <= 0 || (row_len % 16) != 0) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (rows > kMaxCodecElements / row_len) return ATTNQAT_ERR_UNSUPPORTED;
  if (rows == 0) return ATTNQAT_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(codes)) return ATTNQAT_ERR_MISALIGNED;
  const int dst = device_status();
  if (dst != ATTNQAT_OK) return dst;
  (void)hipGetLastError();
  QuantJob job{x, nullptr, scales, rows * (row_len / 16)};
  return attnqat::launch_pack_bf16(job, codes, stream) == hipSuccess ? ATTNQAT_OK
                                                                     : ATTNQAT_ERR_HIP;
}

}  // extern "C"

namespace {

// Start/stop events of the i-th launch of a call when an event array (two
// events per launch) is given, else none.
const attnqat::LaunchEvents* timing(const attnqat::LaunchEvents* ev, int i) {
  return ev == nullptr ? nullptr : ev + i;
}

// with_o: also the quantized output o (second pass)
int run_fwd(const attnqat_problem* p, const void* q, const void* k, const void* v, void* o_hp,
            float* lse, bool with_o, void* o, void* workspace, size_t workspace_bytes,
            hipStream_t stream, const attnqat::LaunchEvents* ev) {
  int st = validate_problem(p);
  if (st != ATTNQAT_OK) return st;
  const void* ptrs[] = {q, k, v, o_hp, lse, workspace, with_o ? o : o_hp};
  for (const void* ptr : ptrs)
    if (ptr == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTNQAT_ERR_MISALIGNED;
  const Layout L = make_layout(p, false);
  if (workspace_bytes < L.total) return ATTNQAT_ERR_WORKSPACE_TOO_SMALL;
  st = device_status();
  if (st != ATTNQAT_OK) return st;
  (void)hipGetLastError();

  const int64_t bh = (int64_t)p->batch * p->heads;
  const int64_t D = p->head_dim;
  uint16_t* qh = at<uint16_t>(workspace, L.q_hat);
  uint16_t* kh = at<uint16_t>(workspace, L.k_hat);
  uint16_t* vh = at<uint16_t>(workspace, L.v_hat);
  QuantJob jobs[3] = {
      {q, qh, at<uint8_t>(workspace, L.q_scale), bh * p->seqlen_q * D / 16},
      {k, kh, at<uint8_t>(workspace, L.k_scale), bh * p->seqlen_kv * D / 16},
      {v, vh, at<uint8_t>(workspace, L.v_scale), bh * p->seqlen_kv * D / 16},
  };
  AttnArgs a = {};
  if (L.kv_decode) {
    // 32-query tiles: every key tile is read by one wave, which fake-quantizes
    // it (and the workgroup its Q rows) in the attention kernel itself and
    // writes Q^, K^, V^ and the scale bytes; no separate quantization pass
    a.q_in = static_cast<const uint16_t*>(q);
    a.q_hat_out = qh;
    a.q_scale_out = at<uint8_t>(workspace, L.q_scale);
    a.k_in = static_cast<const uint16_t*>(k);
    a.v_in = static_cast<const uint16_t*>(v);
    a.k_hat_out = kh;
    a.v_hat_out = vh;
    a.k_scale_out = at<uint8_t>(workspace, L.k_scale);
    a.v_scale_out = at<uint8_t>(workspace, L.v_scale);
    const attnqat::LaunchEvents* e0 = timing(ev, 0);  // an empty span
    if (e0 != nullptr && (hipEventRecord(e0->start, stream) != hipSuccess ||
                          hipEventRecord(e0->stop, stream) != hipSuccess))
      return ATTNQAT_ERR_HIP;
  } else if (D == 128) {
    // K and V in one pass (each K^/V^ tile is read by every query tile of its
    // head); the attention kernel fake-quantizes each workgroup's Q rows
    a.q_in = static_cast<const uint16_t*>(q);
    a.q_hat_out = qh;
    a.q_scale_out = at<uint8_t>(workspace, L.q_scale);
    if (attnqat::launch_quant_bf16(jobs + 1, 2, stream, timing(ev, 0)) != hipSuccess)
      return ATTNQAT_ERR_HIP;
  } else if (attnqat::launch_quant_bf16(jobs, 3, stream, timing(ev, 0)) != hipSuccess) {
    // D = 64: Q in the same pass (measured faster for causal problems there)
    return ATTNQAT_ERR_HIP;
  }

  a.q_hat = qh;
  a.k_hat = kh;
  a.v_hat = vh;
  a.o_hp = static_cast<uint16_t*>(o_hp);
  a.lse_out = lse;
  a.bh = (int)bh;
  a.nq = p->seqlen_q;
  a.nkv = p->seqlen_kv;
  a.causal = p->causal;
  a.softmax_scale = p->softmax_scale;
  a.p_scale = p->p_scale;
  a.kv_splits = L.kv_splits;
  a.kv_decode = L.kv_decode;
  if (L.kv_splits > 1 || L.kv_decode) {
    a.o_part = at<float>(workspace, L.o_part);
    a.ml_part = at<float>(workspace, L.ml_part);
  }
  if (attnqat::launch_fwd(a, p->head_dim, stream, timing(ev, 1)) != hipSuccess)
    return ATTNQAT_ERR_HIP;
  if (with_o) {
    a.lse = lse;  // the first pass's output
    a.o_q = static_cast<uint16_t*>(o);
    if (attnqat::launch_fwd_out(a, p->head_dim, stream, timing(ev, 2)) != hipSuccess)
      return ATTNQAT_ERR_HIP;
  }
  return ATTNQAT_OK;
}

int run_fwd_packed(const attnqat_problem* p, const void* q, const uint8_t* k_codes,
                   const uint8_t* k_scales, const uint8_t* v_codes, const uint8_t* v_scales,
                   void* o_hp, float* lse, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  int st = validate_problem(p);
  if (st != ATTNQAT_OK) return st;
  const void* ptrs[] = {q, k_codes, k_scales, v_codes, v_scales, o_hp, lse, workspace};
  for (const void* ptr : ptrs)
    if (ptr == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  const void* aligned[] = {q, k_codes, v_codes, o_hp, lse, workspace};
  for (const void* ptr : aligned)
    if (!aligned16(ptr)) return ATTNQAT_ERR_MISALIGNED;
  const Layout L = make_layout(p, false);
  if (workspace_bytes < L.total) return ATTNQAT_ERR_WORKSPACE_TOO_SMALL;
  st = device_status();
  if (st != ATTNQAT_OK) return st;
  (void)hipGetLastError();

  const int64_t bh = (int64_t)p->batch * p->heads;
  uint16_t* qh = at<uint16_t>(workspace, L.q_hat);
  uint8_t* qs = at<uint8_t>(workspace, L.q_scale);
  AttnArgs a = {};
  // the attention kernels fake-quantize Q themselves (no separate launch)
  a.q_in = static_cast<const uint16_t*>(q);
  a.q_hat_out = qh;
  a.q_scale_out = qs;
  a.q_hat = qh;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v_codes = v_codes;
  a.v_scales = v_scales;
  a.o_hp = static_cast<uint16_t*>(o_hp);
  a.lse_out = lse;
  a.bh = (int)bh;
  a.nq = p->seqlen_q;
  a.nkv = p->seqlen_kv;
  a.causal = p->causal;
  a.softmax_scale = p->softmax_scale;
  a.p_scale = p->p_scale;
  a.kv_splits = L.kv_splits;
  a.kv_decode = L.kv_decode;
  if (L.kv_splits > 1 || L.kv_decode) {
    a.o_part = at<float>(workspace, L.o_part);
    a.ml_part = at<float>(workspace, L.ml_part);
  }
  if (attnqat::launch_fwd_packed(a, p->head_dim, stream) != hipSuccess) return ATTNQAT_ERR_HIP;
  return ATTNQAT_OK;
}

int run_bwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
            const void* o_hp, const void* d_o, const float* lse, void* dq, void* dk, void* dv,
            void* workspace, size_t workspace_bytes, hipStream_t stream,
            const attnqat::LaunchEvents* ev, bool split_ok = true) {
  int st = validate_problem(p);
  if (st != ATTNQAT_OK) return st;
  const void* ptrs[] = {q, k, v, o_hp, d_o, lse, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (ptr == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTNQAT_ERR_MISALIGNED;
  const Layout L = make_layout(p, true, split_ok);
  if (workspace_bytes < L.total) return ATTNQAT_ERR_WORKSPACE_TOO_SMALL;
  st = device_status();
  if (st != ATTNQAT_OK) return st;
  (void)hipGetLastError();

  const int64_t bh = (int64_t)p->batch * p->heads;
  const int64_t D = p->head_dim;
  uint16_t* qh = at<uint16_t>(workspace, L.q_hat);
  uint16_t* kh = at<uint16_t>(workspace, L.k_hat);
  uint16_t* vh = at<uint16_t>(workspace, L.v_hat);
  float* delta = at<float>(workspace, L.delta);

  // 1) Q fake-quantization fused with delta = rowsum(O_hp * dO); 2) the K/V
  // fake-quantization runs inside k_dkdv (below), whose workgroups each own a
  // key block: they quantize its K and V rows and write K^, V^ and the scale
  // bytes, which k_dq then reads
  const attnqat::QDeltaJob qd = {static_cast<const uint16_t*>(q),
                                 static_cast<const uint16_t*>(o_hp),
                                 static_cast<const uint16_t*>(d_o),
                                 qh,
                                 at<uint8_t>(workspace, L.q_scale),
                                 delta,
                                 bh * p->seqlen_q};
  if (attnqat::launch_bwd_codec(qd, p->head_dim, stream, timing(ev, 0)) != hipSuccess)
    return ATTNQAT_ERR_HIP;

  AttnArgs a = {};
  a.q_hat = qh;
  a.k_hat = kh;
  a.v_hat = vh;
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.delta = delta;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.bh = (int)bh;
  a.nq = p->seqlen_q;
  a.nkv = p->seqlen_kv;
  a.causal = p->causal;
  a.softmax_scale = p->softmax_scale;
  a.p_scale = p->p_scale;
  a.dq_splits = L.dq_splits;
  a.dkdv_splits = L.dkdv_splits;
  a.k_in = static_cast<const uint16_t*>(k);
  a.v_in = static_cast<const uint16_t*>(v);
  a.k_hat_out = kh;
  a.v_hat_out = vh;
  a.k_scale_out = at<uint8_t>(workspace, L.k_scale);
  a.v_scale_out = at<uint8_t>(workspace, L.v_scale);
  if (L.dq_splits > 1) a.dq_part = at<float>(workspace, L.dq_part);
  if (L.dkdv_splits > 1) a.dkdv_part = at<float>(workspace, L.dkdv_part);
  // 3) dK/dV (with the K/V fake-quant) and 4) dQ; on small problems their
  // split loops leave fp32 partial sums, added by one k_sum_parts launch
  // (timed with dQ)
  attnqat::SumJob sums[3];
  int nsums = 0;
  const int64_t nqd = bh * p->seqlen_q * D, nkd = bh * p->seqlen_kv * D;
  if (L.dq_splits > 1)
    sums[nsums++] = {a.dq_part, a.dq, nqd, nqd, L.dq_splits, p->softmax_scale};
  if (L.dkdv_splits > 1) {
    sums[nsums++] = {a.dkdv_part, a.dk, 2 * nkd, nkd, L.dkdv_splits, p->softmax_scale};
    sums[nsums++] = {a.dkdv_part + nkd, a.dv, 2 * nkd, nkd, L.dkdv_splits, 1.0f / p->p_scale};
  }
  const attnqat::LaunchEvents* e1 = timing(ev, 1);
  const attnqat::LaunchEvents e1a = {e1 ? e1->start : nullptr, nullptr};
  const attnqat::LaunchEvents e1b = {nullptr, e1 ? e1->stop : nullptr};
  if (attnqat::launch_bwd_dkdv(a, p->head_dim, stream, timing(ev, 2)) != hipSuccess)
    return ATTNQAT_ERR_HIP;
  if (attnqat::launch_bwd_dq(a, p->head_dim, stream, nsums > 0 && e1 ? &e1a : e1) !=
      hipSuccess)
    return ATTNQAT_ERR_HIP;
  if (nsums > 0 &&
      attnqat::launch_sum_parts(sums, nsums, stream, e1 ? &e1b : nullptr) != hipSuccess)
    return ATTNQAT_ERR_HIP;
  return ATTNQAT_OK;
}

// n launches' start/stop event pairs from a caller's array of 2n events, or
// false when the array or one of its events is null.
bool event_pairs(hipEvent_t* ev, int n, attnqat::LaunchEvents* out) {
  if (ev == nullptr) return false;
  for (int i = 0; i < 2 * n; ++i)
    if (ev[i] == nullptr) return false;
  for (int i = 0; i < n; ++i) out[i] = attnqat::LaunchEvents{ev[2 * i], ev[2 * i + 1]};
  return true;
}

}  // namespace

extern "C" {

int attnqat_fwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                void* o_hp, float* lse, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return run_fwd(p, q, k, v, o_hp, lse, false, nullptr, workspace, workspace_bytes, stream,
                 nullptr);
}
int attnqat_fwd_packed(const attnqat_problem* p, const void* q, const uint8_t* k_codes,
                       const uint8_t* k_scales, const uint8_t* v_codes,
                       const uint8_t* v_scales, void* o_hp, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return run_fwd_packed(p, q, k_codes, k_scales, v_codes, v_scales, o_hp, lse, workspace,
                        workspace_bytes, stream);
}
int attnqat_fwd_quantized(const attnqat_problem* p, const void* q, const void* k, const void* v,
                          void* o_hp, float* lse, void* o, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return run_fwd(p, q, k, v, o_hp, lse, true, o, workspace, workspace_bytes, stream, nullptr);
}

int attnqat_bwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                const void* o_hp, const void* d_o, const float* lse, void* dq, void* dk,
                void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_bwd(p, q, k, v, o_hp, d_o, lse, dq, dk, dv, workspace, workspace_bytes, stream,
                 nullptr);
}

int attnqat_fwd_timed(const attnqat_problem* p, const void* q, const void* k, const void* v,
                      void* o_hp, float* lse, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, hipEvent_t* events) {
  attnqat::LaunchEvents ev[2];
  if (!event_pairs(events, 2, ev)) return ATTNQAT_ERR_INVALID_ARGUMENT;
  return run_fwd(p, q, k, v, o_hp, lse, false, nullptr, workspace, workspace_bytes, stream, ev);
}
int attnqat_fwd_quantized_timed(const attnqat_problem* p, const void* q, const void* k,
                                const void* v, void* o_hp, float* lse, void* o,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* events) {
  attnqat::LaunchEvents ev[3];
  if (!event_pairs(events, 3, ev)) return ATTNQAT_ERR_INVALID_ARGUMENT;
  return run_fwd(p, q, k, v, o_hp, lse, true, o, workspace, workspace_bytes, stream, ev);
}

int attnqat_bwd_timed(const attnqat_problem* p, const void* q, const void* k, const void* v,
                      const void* o_hp, const void* d_o, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t* events) {
  attnqat::LaunchEvents ev[3];
  if (!event_pairs(events, 3, ev)) return ATTNQAT_ERR_INVALID_ARGUMENT;
  return run_bwd(p, q, k, v, o_hp, d_o, lse, dq, dk, dv, workspace, workspace_bytes, stream, ev);
}

}  // extern "C"

extern "C" int attnqat_probe_mfma_peak(const void* a, const void* b, float* out, int blocks,
                                       int iters, hipStream_t stream) {
  if (a == nullptr || b == nullptr || out == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20))
    return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return ATTNQAT_ERR_MISALIGNED;
  const int st = device_status();
  if (st != ATTNQAT_OK) return st;
  (void)hipGetLastError();
  return attnqat::launch_mfma_peak(static_cast<const uint16_t*>(a),
                                   static_cast<const uint16_t*>(b), out, blocks, iters,
                                   stream) == hipSuccess
             ? ATTNQAT_OK
             : ATTNQAT_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Backward without a workspace argument, for callers that cannot allocate.
//
// The workspace lives in a file-scope device array of kScratchBytes (each
// GPU the library runs on holds its own copy until the process ends).  In
// host code `scratch` only names the symbol: its device address on the
// current GPU comes from hipGetSymbolAddress, taken once per device on the
// first call there and kept in g_scratch.  Every call on a GPU shares that
// GPU's array, so calls that overlap on one GPU race; nothing in the array
// needs to start at zero (the backward writes every workspace byte it reads).
namespace {

constexpr size_t kScratchBytes = ATTNQAT_NOALLOC_MAX_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch[256];

// The scratch array's address on the current device, or nullptr on error.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return nullptr;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
    return nullptr;
  g_scratch[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" int attnqat_bwd_noalloc(const attnqat_problem* p, const void* q, const void* k,
                                   const void* v, const void* o_hp, const void* d_o,
                                   const float* lse, void* dq, void* dk, void* dv,
                                   hipStream_t stream) {
  const int st = validate_problem(p);
  if (st != ATTNQAT_OK) return st;
  // the split loops' partial sums only where they fit beside the rest
  const bool split_ok = make_layout(p, true).total <= kScratchBytes;
  if (make_layout(p, true, split_ok).total > kScratchBytes) return ATTNQAT_ERR_UNSUPPORTED;
  const int dst = device_status();
  if (dst != ATTNQAT_OK) return dst;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return ATTNQAT_ERR_HIP;
  return run_bwd(p, q, k, v, o_hp, d_o, lse, dq, dk, dv, ws, kScratchBytes, stream, nullptr,
                 split_ok);
}

extern "C" int attnqat_probe_issue_mix(int mode, int valu_per_mfma, int agpr, const void* in,
                                       float* out, int blocks, int threads, int iters,
                                       hipStream_t stream) {
  if (in == nullptr || out == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (mode < 0 || mode > 3 || (valu_per_mfma != 8 && valu_per_mfma != 16) ||
      (threads != 256 && threads != 512) || (mode == 3 && threads != 512) || blocks < 1 ||
      blocks > (1 << 20) || iters < 1 || iters > (1 << 20))
    return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (!aligned16(in) || !aligned16(out)) return ATTNQAT_ERR_MISALIGNED;
  const int st = device_status();
  if (st != ATTNQAT_OK) return st;
  (void)hipGetLastError();
  return attnqat::launch_issue_mix(mode, valu_per_mfma, agpr != 0,
                                   static_cast<const uint16_t*>(in), out, blocks, threads, iters,
                                   stream) == hipSuccess
             ? ATTNQAT_OK
             : ATTNQAT_ERR_HIP;
}

extern "C" int attnqat_probe_lds_write(int pattern, float* out, int blocks, int iters,
                                       hipStream_t stream) {
  if (out == nullptr) return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (pattern < 0 || pattern > 5 || blocks < 1 || blocks > (1 << 20) || iters < 1 ||
      iters > (1 << 20))
    return ATTNQAT_ERR_INVALID_ARGUMENT;
  if (!aligned16(out)) return ATTNQAT_ERR_MISALIGNED;
  const int st = device_status();
  if (st != ATTNQAT_OK) return st;
  (void)hipGetLastError();
  return attnqat::launch_lds_write(pattern, out, blocks, iters, stream) == hipSuccess
             ? ATTNQAT_OK
             : ATTNQAT_ERR_HIP;
}
