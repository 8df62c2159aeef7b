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
// and V^ tiles are staged row-major in double-buffered, XOR-swizzled LDS
// (prefetched one tile ahead through registers) and the K^T operand is read
// with LDS transpose reads.  Only tiles on a boundary (tails, causal
// diagonal) evaluate masks; causal tiles entirely above the diagonal are
// skipped per wave, the diagonal tile keeps the elementwise key <= query
// mask, keys >= Nkv get P = 0, loads beyond the ends read zeros and stores
// stop at the ends.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kDqBM = 128;              // queries per workgroup (k_dq)
constexpr int kDqBN = ATTNQAT_DQ_BN;      // keys per staged tile (k_dq; 32-key sub-tiles)

// ---------------------------------------------------------------------------
// dQ

// One 32-key sub-tile of k_dq for one wave (32 queries).
#ifndef ATTNQAT_DQ_AHEAD
#define ATTNQAT_DQ_AHEAD 2
#endif
constexpr int kDqAhead = ATTNQAT_DQ_AHEAD;  // MFMA operand reads issued this many MFMAs ahead

template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void dq_tile(const bf16x8* qf, const bf16x8* df, f32x16* acc,
                                        const uint16_t* sKb, const uint16_t* sVb,
                                        const RowOffsets<D>& ro, const ColOffsets<D>& co, int k0,
                                        int qi, bool qok, int nkv, float lse2, float dl,
                                        float sl2, int lane) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int NM = 2 * KB;  // S^T (even k) and dP^T (odd k) MFMAs
  constexpr int NQ = 2 * DB;  // dQ^T MFMAs
  const int h = lane >> 5;
  // S^T = K^ Q^T and dP^T = V^ dO^T; A operands read from LDS kDqAhead MFMAs ahead
  auto row_op = [&](int k) __attribute__((always_inline)) {
    return ld_bf16x8(((k & 1) ? sVb : sKb) + ro.o[k >> 1]);
  };
  bf16x8 a[NM];
#pragma unroll
  for (int k = 0; k < kDqAhead; ++k) a[k] = row_op(k);
  f32x16 s, dp;
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    if (k + kDqAhead < NM) a[k + kDqAhead] = row_op(k + kDqAhead);
    if (k & 1)
      dp = mfma32x32x16(a[k], df[k >> 1], k == 1 ? zero_f32x16() : dp);
    else
      s = mfma32x32x16(a[k], qf[k >> 1], k == 0 ? zero_f32x16() : s);
    __builtin_amdgcn_sched_barrier(0);
  }
  // K^T operands of dQ^T = K^T dS^T (MFMA k: key block k / DB, d block k % DB),
  // the first ones read while the VALU works
  auto col_op = [&](int k) __attribute__((always_inline)) {
    return lds_operand_cols_at(sKb + 16 * (k / DB) * D, co.a[k % DB], co.b[k % DB]);
  };
  bf16x8 c[NQ];
#pragma unroll
  for (int k = 0; k < kDqAhead; ++k) c[k] = col_op(k);
  float ds[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float x = __builtin_fmaf(s[v], sl2, -lse2);
    if (MASK) {
      const int key = k0 + 8 * (v >> 2) + 4 * h + (v & 3);
      const bool ok = qok && key < nkv && (!CAUSAL || key <= qi);
      x = ok ? x : -INFINITY;
    }
    ds[v] = fast_exp2(x) * (dp[v] - dl);
  }
  // dQ^T += K^T dS^T over two 16-key k-blocks: lane half h, element e of
  // k-block kh holds key 16*kh + 8*(e/4) + 4h + e%4 in both operands.
  bf16x8 b[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const u32x4 bw = {pack_bf16x2(ds[8 * kh], ds[8 * kh + 1]),
                      pack_bf16x2(ds[8 * kh + 2], ds[8 * kh + 3]),
                      pack_bf16x2(ds[8 * kh + 4], ds[8 * kh + 5]),
                      pack_bf16x2(ds[8 * kh + 6], ds[8 * kh + 7])};
    b[kh] = __builtin_bit_cast(bf16x8, bw);
  }
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
  constexpr int BN = kDqBN;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CH = BN * CPR / 256;  // chunks per thread per tensor per tile
  static_assert(BN % 32 == 0 && CH >= 1, "key tile must be whole 32-key sub-tiles");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * D];  // swizzled rows
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const TileId t = xcd_tile((a.nq + kDqBM - 1) / kDqBM);
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
  // LDS offsets: row reads of K^/V^ and K^T column reads (k-block rows 4h.., 4h+8..)
  const RowOffsets<D> ro(lane);
  const ColOffsets<D> co(4 * h, 4 * h + 8, lane);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();
  // keys above the workgroup's last query are masked (causal)
  const int kend = CAUSAL ? min(nkv, qblk0 + kDqBM) : nkv;
  const int ntiles = (kend + BN - 1) / BN;

  u32x4 rk[CH], rv[CH];
  uint32_t voff[CH];  // byte offset of this thread's chunks within a tile
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = tid + 256 * c;
    voff[c] = (uint32_t)((idx / CPR) * D + (idx % CPR) * 8) * 2u;
  }
  auto load_tile = [&](int k0) __attribute__((always_inline)) {
    // rows past nkv read as zeros (masked out later)
    const uint32_t bytes = (uint32_t)(min(nkv - k0, BN) * D) * 2u;
    const auto rsk = make_rsrc(K + (size_t)k0 * D, bytes);
    const auto rsv = make_rsrc(V + (size_t)k0 * D, bytes);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      rk[c] = buf_ld16(rsk, voff[c]);
      rv[c] = buf_ld16(rsv, voff[c]);
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + 256 * c;
      const int r = idx / CPR, col = (idx % CPR) * 8;
      *reinterpret_cast<u32x4*>(&sK[buf][swz<D>(r, col)]) = rk[c];
      *reinterpret_cast<u32x4*>(&sV[buf][swz<D>(r, col)]) = rv[c];
    }
  };

  auto step = [&](int it, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = it & 1;
    const int k0 = it * BN;
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile(k0 + BN);
#pragma unroll
    for (int sub = 0; sub < BN / 32; ++sub) {
      const int ks = k0 + 32 * sub;
      const uint16_t* kb = sK[buf] + 32 * sub * D;  // 32-row blocks keep the swizzle phase
      const uint16_t* vb = sV[buf] + 32 * sub * D;
      // (boundary tiles only) every key above every row of this wave: skip
      if (!MASK || !(CAUSAL && qw0 + 31 < ks))
        dq_tile<D, CAUSAL, MASK>(qf, df, acc, kb, vb, ro, co, ks, qi, qok, nkv, lse2, dl, sl2,
                                 lane);
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  };
  // Leading tiles are interior (branch-free); masks start at the first tile
  // that reaches past nkv or above the workgroup's first query (causal).
  int it_hi = min(ntiles, nkv / BN);
  if (CAUSAL) it_hi = min(it_hi, (qblk0 + 1) / BN);

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  vmem_wait_all();
  __syncthreads();
  for (int it = 0; it < it_hi; ++it) step(it, BoolTag<false>());
  for (int it = it_hi; it < ntiles; ++it) step(it, BoolTag<true>());

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

}  // namespace

hipError_t launch_bwd_dq(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)(((a.nq + kDqBM - 1) / kDqBM) * a.bh));
  if (head_dim == 128) {
    if (a.causal)
      hipLaunchKernelGGL((k_dq<128, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_dq<128, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.causal)
      hipLaunchKernelGGL((k_dq<64, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_dq<64, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attnqat
