// QAT backward, query side: dQ ("NVFP4 Attention QAT Backward", §Overview
// formula block and the dQ kernel of its four-kernel split):
//
//   P  = exp(s Q^ K^T - lse)             recomputed per tile, fp32
//   dS = P * (dO V^T - delta)            delta = rowsum(O_hp * dO)
//   dQ = s dS K^                         straight-through: the unquantized P
//
// bf16 MFMA 32x32x16 with fp32 accumulation; dS is rounded to bf16 for the
// MFMA.  Layout (gfx950, wave64): each wave owns 32 queries (Q^ and dO rows
// in registers as B operands).  S^T and dP^T accumulators hold one query per
// lane, so dS^T feeds the B operand of dQ^T = K^T dS^T from registers; K^
// and V^ tiles are staged row-major in a 4-deep ring of XOR-swizzled LDS
// tiles, copied global -> LDS directly two tiles ahead, and the K^T operand
// is read with LDS transpose reads.  Software pipeline: step t issues the
// S^T/dP^T MFMAs of tile t (at raised wave priority), then the dS VALU work
// of tile t interleaved with the dQ^T MFMAs of tile t-1.  Causal launches
// hand out each head's query tiles last-first (the heaviest first).  Only
// tiles on a boundary (tails, causal
// diagonal) evaluate masks; causal tiles entirely above the diagonal are
// skipped per wave, the diagonal tile keeps the elementwise key <= query
// mask, keys >= Nkv get P = 0, loads beyond the ends read zeros and stores
// stop at the ends.  When the query blocks cannot fill the chip, the key
// tiles of each block are split over blockIdx.y: each split writes its fp32
// dQ^T partial, and k_sum_parts (launched after both attention kernels, with
// the dK/dV sums) adds the splits in order (deterministic).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kDqBM = 128;              // queries per workgroup (k_dq)

// ---------------------------------------------------------------------------
// dQ

#ifndef ATTNQAT_DQ_AHEAD
#define ATTNQAT_DQ_AHEAD 2
#endif
constexpr int kDqAhead = ATTNQAT_DQ_AHEAD;  // MFMA operand reads issued this many MFMAs ahead


// Pieces of one wave's work on one 32-key block (32 queries x 32 keys).
//
// A operand of S^T/dP^T MFMA k (S^T = K^ Q^T for even k, dP^T = V^ dO^T for
// odd k; d block k/2): rows of the K^ or V^ tile.
template <int D>
__device__ __forceinline__ bf16x8 dq_row_op(const uint16_t* sKb, const uint16_t* sVb,
                                            const RowOffsets<D>& ro, int k) {
  return ld_bf16x8(((k & 1) ? sVb : sKb) + ro.o[k >> 1]);
}

// S^T/dP^T MFMA k into s (even k) or dp (odd k; the chain starts from dp0).
__device__ __forceinline__ void dq_sdp_mfma(int k, const bf16x8& a, const bf16x8* qf,
                                            const bf16x8* df, f32x16& s, f32x16& dp,
                                            const f32x16& dp0) {
  if (k & 1)
    dp = mfma32x32x16(a, df[k >> 1], k == 1 ? dp0 : dp);
  else
    s = mfma32x32x16(a, qf[k >> 1], k == 0 ? zero_f32x16() : s);
}

// dS^T element v (dpv: dP - delta): lane half h holds key
// k0 + 8*(v/4) + 4h + v%4 of query qi.
template <bool CAUSAL, bool MASK>
__device__ __forceinline__ float dq_ds(float sv, float dpv, int v, int k0, int h, int qi, bool qok,
                                       int nkv, float lse2, float sl2) {
  float x = __builtin_fmaf(sv, sl2, -lse2);
  if (MASK) {
    const int key = k0 + 8 * (v >> 2) + 4 * h + (v & 3);
    const bool ok = qok && key < nkv && (!CAUSAL || key <= qi);
    x = ok ? x : -INFINITY;
  }
  return fast_exp2(x) * dpv;
}

// dS^T as the two bf16 B operands of dQ^T = K^T dS^T (16-key k-blocks kh:
// element e of k-block kh is key 16*kh + 8*(e/4) + 4h + e%4, matching the
// K^T column reads).
__device__ __forceinline__ void dq_pack(const float* ds, bf16x8* b) {
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const u32x4 bw = {pack_bf16x2(ds[8 * kh], ds[8 * kh + 1]),
                      pack_bf16x2(ds[8 * kh + 2], ds[8 * kh + 3]),
                      pack_bf16x2(ds[8 * kh + 4], ds[8 * kh + 5]),
                      pack_bf16x2(ds[8 * kh + 6], ds[8 * kh + 7])};
    b[kh] = __builtin_bit_cast(bf16x8, bw);
  }
}

// S^T and dP^T of one block, MFMAs only.
template <int D>
__device__ __forceinline__ void dq_sdp(const bf16x8* qf, const bf16x8* df, const uint16_t* sKb,
                                       const uint16_t* sVb, const RowOffsets<D>& ro, f32x16& s,
                                       f32x16& dp, const f32x16& dp0) {
  constexpr int NM = D / 8;
  bf16x8 a[NM];
#pragma unroll
  for (int k = 0; k < kDqAhead; ++k) a[k] = dq_row_op<D>(sKb, sVb, ro, k);
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    if (k + kDqAhead < NM) a[k + kDqAhead] = dq_row_op<D>(sKb, sVb, ro, k + kDqAhead);
    dq_sdp_mfma(k, a[k], qf, df, s, dp, dp0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// dS^T of the current block (VALU, into b) interleaved with dQ^T += K^T
// dS^T of the previous block (MFMA, b_prev and that block's tile sKp): the
// wave keeps the matrix pipe fed while it evaluates exp2.
template <int D, bool CAUSAL, bool MASK, bool ACC>
__device__ __forceinline__ void dq_ds_acc(const f32x16& s, const f32x16& dp, int k0, int h, int qi,
                                          bool qok, int nkv, float lse2, float sl2,
                                          bf16x8* b, f32x16* acc, const bf16x8* b_prev,
                                          const uint16_t* sKp, const ColOffsets<D>& co) {
  constexpr int DB = D / 32;
  constexpr int NQ = 2 * DB;    // dQ^T MFMAs
  constexpr int EPM = 16 / NQ;  // dS elements per MFMA
  static_assert(EPM % 2 == 0, "elements are packed in pairs");
  auto col_op = [&](int k) __attribute__((always_inline)) {
    return lds_operand_cols_at(sKp + 16 * (k / DB) * D, co.a[k % DB], co.b[k % DB]);
  };
  bf16x8 c[NQ];
  if (ACC) {
#pragma unroll
    for (int k = 0; k < kDqAhead; ++k) c[k] = col_op(k);
  }
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    if (ACC) {
      if (k + kDqAhead < NQ) c[k + kDqAhead] = col_op(k + kDqAhead);
      acc[k % DB] = mfma32x32x16(c[k], b_prev[k / DB], acc[k % DB]);
    }
#pragma unroll
    for (int e = 0; e < EPM; e += 2) {
      const int v = EPM * k + e;
      const float d0 = dq_ds<CAUSAL, MASK>(s[v], dp[v], v, k0, h, qi, qok, nkv, lse2, sl2);
      const float d1 =
          dq_ds<CAUSAL, MASK>(s[v + 1], dp[v + 1], v + 1, k0, h, qi, qok, nkv, lse2, sl2);
      w[v >> 1] = pin_vgpr(pack_bf16x2(d0, d1));  // made here, in this MFMA's slot
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // element e of k-block kh is key 16*kh + 8*(e/4) + 4h + e%4 (dq_pack's order)
  b[0] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
  b[1] = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
}

// dQ^T += K^T dS^T (MFMA k: 16-key k-block k / DB, d block k % DB).
template <int D>
__device__ __forceinline__ void dq_acc(f32x16* acc, const bf16x8* b, const uint16_t* sKb,
                                       const ColOffsets<D>& co) {
  constexpr int DB = D / 32;
  constexpr int NQ = 2 * DB;
  auto col_op = [&](int k) __attribute__((always_inline)) {
    return lds_operand_cols_at(sKb + 16 * (k / DB) * D, co.a[k % DB], co.b[k % DB]);
  };
  bf16x8 c[NQ];
#pragma unroll
  for (int k = 0; k < kDqAhead; ++k) c[k] = col_op(k);
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    if (k + kDqAhead < NQ) c[k + kDqAhead] = col_op(k + kDqAhead);
    acc[k % DB] = mfma32x32x16(c[k], b[k / DB], acc[k % DB]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ATTNQAT_DQ_WAVES, 8)))
void k_dq(AttnArgs a) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int BN = 32;              // keys per tile: one 32-key block
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CH = BN * CPR / 256;  // 16-byte chunks per lane per tensor per tile
  constexpr int NB = 4;               // LDS ring: tiles it-1, it read while it+1, it+2 arrive
  static_assert(CH >= 1, "tile copy needs at least one chunk per lane");
  __shared__ __attribute__((aligned(16))) uint16_t sK[NB][BN * D];  // swizzled rows
  __shared__ __attribute__((aligned(16))) uint16_t sV[NB][BN * D];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const TileId t = xcd_tile((a.nq + kDqBM - 1) / kDqBM, CAUSAL);
  const int bh = t.bh;
  const int nq = a.nq, nkv = a.nkv;
  const int qblk0 = t.tile * kDqBM;
  const int qw0 = qblk0 + wave * 32;
  const int qi = qw0 + l32;
  const bool qok = qi < nq;
  const uint16_t* Q = a.q_hat + (size_t)bh * nq * D;
  const uint16_t* dO = a.d_o + (size_t)bh * nq * D;
  const uint16_t* K = a.k_hat + (size_t)bh * nkv * D;
  const uint16_t* V = a.v_hat + (size_t)bh * nkv * D;

  bf16x8 qf[KB], df[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    qf[kb] = qok ? ld_bf16x8(Q + (size_t)qi * D + 16 * kb + 8 * h) : zero_bf16x8();
    df[kb] = qok ? ld_bf16x8(dO + (size_t)qi * D + 16 * kb + 8 * h) : zero_bf16x8();
  }
  const float lse2 = qok ? a.lse[(size_t)bh * nq + qi] * kLog2e : 0.0f;
  const float dl = qok ? a.delta[(size_t)bh * nq + qi] : 0.0f;
  const float sl2 = a.softmax_scale * kLog2e;
  // the dP^T chain starts from -delta (every element of the accumulator is
  // this lane's query), so it yields dP - delta directly
  f32x16 dp0;
#pragma unroll
  for (int i = 0; i < 16; ++i) dp0[i] = -dl;
  // LDS offsets: row reads of K^/V^ and K^T column reads (k-block rows 4h.., 4h+8..)
  const RowOffsets<D> ro(lane);
  const ColOffsets<D> co(4 * h, 4 * h + 8, lane);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();
  // keys above the workgroup's last query are masked (causal)
  const int kend = CAUSAL ? min(nkv, qblk0 + kDqBM) : nkv;
  // this workgroup's key tiles t0 .. t0 + ntiles - 1 (all unless split)
  const int ntiles_all = (kend + BN - 1) / BN;
  const int KSPL = a.dq_splits > 1 ? a.dq_splits : 1;
  const int per = (ntiles_all + KSPL - 1) / KSPL;
  const int t0 = (int)blockIdx.y * per;  // blockIdx.y < KSPL
  const int ntiles = KSPL > 1 ? max(0, min(ntiles_all - t0, per)) : ntiles_all;

  // K^/V^ tiles go global -> LDS directly (no registers). Copy instruction c
  // of this wave fills LDS chunk slots 64*(CH*wave + c) + lane; slot (row r,
  // position j) of the XOR-swizzled layout holds column chunk swz(r, j), so
  // each lane fetches that chunk (the swizzle is an involution).
  uint32_t goff[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int p = 64 * (CH * wave + c) + lane;
    goff[c] = (uint32_t)swz<D>(p / CPR, 8 * (p % CPR)) * 2u;
  }
  auto issue_tile = [&](int it) __attribute__((always_inline)) {
    const int k0 = (t0 + it) * BN;
    const int buf = it % NB;
    // rows past nkv arrive as zeros (masked out later)
    const uint32_t bytes = (uint32_t)(min(nkv - k0, BN) * D) * 2u;
    const u32x4 dk = buf_desc(K + (size_t)k0 * D, bytes);
    const u32x4 dv = buf_desc(V + (size_t)k0 * D, bytes);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      buf_ld16_lds(dk, goff[c],
                   __builtin_amdgcn_readfirstlane(lds_addr(&sK[buf][512 * (CH * wave + c)])));
      buf_ld16_lds(dv, goff[c],
                   __builtin_amdgcn_readfirstlane(lds_addr(&sV[buf][512 * (CH * wave + c)])));
    }
  };

  // Leading tiles are interior (branch-free); masks start at the first tile
  // that reaches past nkv or above the workgroup's first query (causal).
  int it_hi = min(ntiles_all, nkv / BN);
  if (CAUSAL) it_hi = min(it_hi, (qblk0 + 1) / BN);
  it_hi = max(0, min(ntiles, it_hi - t0));

  if (ntiles > 0) issue_tile(0);
  if (ntiles > 1) issue_tile(1);
  vmem_wait_all();
  __syncthreads();

  // Software pipeline over tiles: step it runs the S^T/dP^T MFMAs of tile
  // it, then its dS^T VALU work interleaved with the dQ^T MFMAs of tile it-1.
  bf16x8 b_prev[2];
  bool have_prev = false;
  auto step = [&](int it, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = it % NB;
    const int pbuf = (it + NB - 1) % NB;
    const int k0 = (t0 + it) * BN;
    if (it + 2 < ntiles) issue_tile(it + 2);
    // (boundary tiles only) every key above every query of this wave: skip;
    // every later tile is then skipped too
    if (!MASK || !(CAUSAL && qw0 + 31 < k0)) {
      f32x16 s, dp;
      // the MFMA-only phase runs at raised wave priority, so that the other
      // wave on the SIMD fills its gaps rather than competing for issue
      __builtin_amdgcn_s_setprio(1);
      dq_sdp<D>(qf, df, sK[buf], sV[buf], ro, s, dp, dp0);
      __builtin_amdgcn_s_setprio(0);
      bf16x8 b[2];
      if (have_prev)
        dq_ds_acc<D, CAUSAL, MASK, true>(s, dp, k0, h, qi, qok, nkv, lse2, sl2, b, acc,
                                         b_prev, sK[pbuf], co);
      else
        dq_ds_acc<D, CAUSAL, MASK, false>(s, dp, k0, h, qi, qok, nkv, lse2, sl2, b, acc,
                                          b_prev, sK[pbuf], co);
      b_prev[0] = b[0];
      b_prev[1] = b[1];
      have_prev = true;
    } else if (have_prev) {
      dq_acc<D>(acc, b_prev, sK[pbuf], co);
      have_prev = false;
    }
    // tile it+1 has landed (this wave's copies; the barrier covers the
    // other waves'), tile it+2 may still be in flight
    if (it + 2 < ntiles)
      vmem_wait<2 * CH>();
    else
      vmem_wait<0>();
    __syncthreads();
  };
  int it = 0;
  for (; it < it_hi; ++it) step(it, BoolTag<false>());
  for (; it < ntiles; ++it) step(it, BoolTag<true>());
  // the last block's dQ^T (its tile is still resident)
  if (have_prev) dq_acc<D>(acc, b_prev, sK[(ntiles - 1) % NB], co);

  if (KSPL > 1) {
    // this split's unscaled dQ^T row (a split without keys stores zeros)
    if (qok) {
      float* out = a.dq_part + (((size_t)blockIdx.y * a.bh + bh) * nq + qi) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(out + 32 * db + 8 * g4 + 4 * h) =
              f32x4{acc[db][4 * g4], acc[db][4 * g4 + 1], acc[db][4 * g4 + 2],
                    acc[db][4 * g4 + 3]};
      }
    }
    return;
  }
  if (qok) {
    const float sc = a.softmax_scale;
    uint16_t* out = a.dq + (size_t)bh * nq * D + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 w = {pack_bf16x2(acc[db][4 * g4] * sc, acc[db][4 * g4 + 1] * sc),
                         pack_bf16x2(acc[db][4 * g4 + 2] * sc, acc[db][4 * g4 + 3] * sc)};
        *reinterpret_cast<u32x2*>(out + 32 * db + 8 * g4 + 4 * h) = w;
      }
    }
  }
}

// The sums of SumJob, job blockIdx.y: 4 values per thread, the splits added
// in order and read 8 at a time so that their loads are in flight together.
struct SumJobs {
  SumJob j[3];
};
__global__ __launch_bounds__(256) void k_sum_parts(SumJobs jobs) {
  const SumJob& jb = jobs.j[blockIdx.y];
  const float* part = jb.part;
  const int splits = jb.splits;
  const int64_t stride = jb.stride, n = jb.n;
  const float scale = jb.scale;
  uint16_t* out = jb.out;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < splits; s0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = s0 + k < splits ? *reinterpret_cast<const f32x4*>(part + (s0 + k) * stride + i)
                             : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += v[k];
  }
  *reinterpret_cast<u32x2*>(out + i) = u32x2{pack_bf16x2(acc[0] * scale, acc[1] * scale),
                                             pack_bf16x2(acc[2] * scale, acc[3] * scale)};
}

}  // namespace

hipError_t launch_sum_parts(const SumJob* jobs, int njobs, hipStream_t stream,
                            const LaunchEvents* ev) {
  if (njobs < 1 || njobs > 3) return hipErrorInvalidValue;
  SumJobs js = {};
  int64_t nmax = 0;
  for (int i = 0; i < njobs; ++i) {
    js.j[i] = jobs[i];
    nmax = jobs[i].n > nmax ? jobs[i].n : nmax;
  }
  const dim3 grid((unsigned)((nmax / 4 + 255) / 256), (unsigned)njobs), block(256);
  return launch(k_sum_parts, grid, block, stream, ev, js);
}

hipError_t launch_bwd_dq(const AttnArgs& a, int head_dim, hipStream_t stream,
                         const LaunchEvents* ev) {
  // split over keys: fp32 partials, summed by the caller's k_sum_parts launch
  const dim3 grid((unsigned)(((a.nq + kDqBM - 1) / kDqBM) * a.bh),
                  (unsigned)(a.dq_splits > 1 ? a.dq_splits : 1));
  const dim3 block(256);
  if (head_dim == 128)
    return a.causal ? launch(k_dq<128, true>, grid, block, stream, ev, a)
                    : launch(k_dq<128, false>, grid, block, stream, ev, a);
  return a.causal ? launch(k_dq<64, true>, grid, block, stream, ev, a)
                  : launch(k_dq<64, false>, grid, block, stream, ev, a);
}

}  // namespace attnqat
