// QAT backward attention kernels: dQ, and dK/dV with the fake-quantized P
// ("NVFP4 Attention QAT Backward", §Overview formula block and its
// four-kernel split: Q fake-quant + delta, K/V fake-quant, dQ, dK/dV).
//
//   P  = exp(s Q^ K^T - lse)             recomputed per tile, fp32
//   dS = P * (dO V^T - delta)            delta = rowsum(O_hp * dO)
//   dQ = s dS K^                         (k_dq)
//   dK = s dS^T Q^,  dV = fq(P)^T dO     (k_dkdv; fq groups 16 keys)
//
// Both kernels use bf16 MFMA 32x32x16 with fp32 accumulation.  The dS and
// fake-quantized P^F operands are rounded to bf16 for the MFMA (P^F is exact
// in bf16: an E2M1 code times an E4M3 scale has at most 6 significant bits).
//
// Layout choices (gfx950, wave64):
//  * k_dq: each wave owns 32 queries (Q^ and dO rows in registers as B
//    operands).  S^T and dP^T accumulators hold one query per lane, so dS^T
//    feeds the B operand of dQ^T = K^T dS^T from registers; K^ and V^ tiles
//    are staged row-major in double-buffered, XOR-swizzled LDS (prefetched
//    one tile ahead through registers) and the K^T operand is read with LDS
//    transpose reads.
//  * k_dkdv: each wave owns 32 keys.  Its K^ and V^ rows sit in registers as
//    A operands with the row order permuted so that, in the S^T accumulator,
//    each lane holds one query and 16 *consecutive* keys: exactly one P
//    quantization group.  The group amax, the E4M3 scale and the E2M1
//    rounding are then per-lane work with no cross-lane reduction (the
//    rounding uses the hardware FP4 conversion on an FMA-refined quotient).
//    P^F and dS are written as [query][key] rows of per-wave LDS tiles and
//    read back with LDS transpose reads as the A operands of dV = P^F^T dO
//    and dK = dS^T Q^; the B operands (dO and Q^ with lanes over d) come the
//    same way from the row-major, double-buffered Q^/dO tiles.
//  * Only tiles on a boundary (tails, causal diagonal) evaluate masks.
//  * Causal: tiles entirely above the diagonal are skipped per wave; the
//    diagonal tile keeps the elementwise key <= query mask.  Tails: keys >= Nkv
//    and queries >= Nq get P = 0 (so a short last P group is zero-padded),
//    loads beyond the ends read zeros and stores stop at the ends.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kDqBM = 128;              // queries per workgroup (k_dq)
constexpr int kDqBN = ATTNQAT_DQ_BN;      // keys per staged tile (k_dq; 32-key sub-tiles)
constexpr int kDkvBN = 128;             // keys per workgroup (k_dkdv)
constexpr int kDkvBM = 64;              // queries per staged tile (k_dkdv; two 32-query sub-tiles)

// ---------------------------------------------------------------------------
// dQ

// One 32-key sub-tile of k_dq for one wave (32 queries).
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void dq_tile(const bf16x8* qf, const bf16x8* df, f32x16* acc,
                                        const uint16_t* sKb, const uint16_t* sVb,
                                        const RowOffsets<D>& ro, const ColOffsets<D>& co, int k0,
                                        int qi, bool qok, int nkv, float lse2, float dl,
                                        float sl2, int lane) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  const int h = lane >> 5, l32 = lane & 31;
  f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    s = mfma32x32x16(ld_bf16x8(sKb + ro.o[kb]), qf[kb], s);
    dp = mfma32x32x16(ld_bf16x8(sVb + ro.o[kb]), df[kb], dp);
  }
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
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const u32x4 bw = {pack_bf16x2(ds[8 * kh], ds[8 * kh + 1]),
                      pack_bf16x2(ds[8 * kh + 2], ds[8 * kh + 3]),
                      pack_bf16x2(ds[8 * kh + 4], ds[8 * kh + 5]),
                      pack_bf16x2(ds[8 * kh + 6], ds[8 * kh + 7])};
    const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      acc[db] = mfma32x32x16(lds_operand_cols_at(sKb + 16 * kh * D, co.a[db], co.b[db]), b,
                             acc[db]);
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
  const int bh = blockIdx.y;
  const int nq = a.nq, nkv = a.nkv;
  const int qblk0 = blockIdx.x * kDqBM;
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

// ---------------------------------------------------------------------------
// dK / dV

// Row r of a wave's 32-key MFMA A operand holds key pi(r) so that the S^T
// accumulator (rows 8*(v/4) + 4h + v%4 in VGPR v of lane half h) holds key
// 16h + v: one contiguous 16-key group per lane.
__device__ __forceinline__ int key_perm(int r) {
  return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// Q^ and dO staging of k_dkdv: each ring buffer holds a BM-row tile of Q^
// followed by the same rows of dO, as bf16 rows of D elements at a pitch of
// D + 8 (16 bytes of padding keep both the 16-byte row reads and the
// transpose reads free of bank conflicts on the 64-bank LDS).  With a
// linear layout every k-block, d-block, sub-tile and tensor offset is a
// compile-time immediate of the LDS instruction: a lane needs one address
// register per access pattern and buffer.
template <int D>
struct DkdvStage {
  static constexpr int P = D + 8;             // row pitch (elements)
  static constexpr int DO = kDkvBM * P;       // dO rows after the Q^ rows
  static constexpr int BUF = 2 * kDkvBM * P;  // one ring buffer
  static constexpr int SUB = 32 * P;          // second 32-row sub-tile
  // lane offsets: row reads (row l32, columns 8h..) and column reads (rows
  // 8h + (l%16)/4, columns 16*((l/16)%2) + 4*(l%4)); the second half of a
  // column operand is 4 rows further
  __device__ static int row_off(int lane) { return (lane & 31) * P + 8 * (lane >> 5); }
  __device__ static int col_off(int lane) {
    const int j = lane & 15;
    return (8 * (lane >> 5) + (j >> 2)) * P + ((lane >> 4) & 1) * 16 + 4 * (j & 3);
  }
  // B operand of S^T / dP^T: Q^ (or dO) row block kb of the sub-tile at p
  __device__ static bf16x8 rows(const uint16_t* p, int kb) { return ld_bf16x8(p + 16 * kb); }
  // B operand of dK / dV: columns 32*db.. of query block kq of the sub-tile at p
  __device__ static bf16x8 cols(const uint16_t* p, int kq, int db) {
    return lds_operand_cols_at(p + 16 * kq * P + 32 * db, 0, 4 * P);
  }
};

// One 32-query sub-tile of k_dkdv for one wave (32 keys), self-contained and
// masked: the boundary tiles (causal diagonal, query tail, keys past nkv).
// qa / qc: the sub-tile's Q^ rows at this lane's row / column read offsets.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_tile_masked(const bf16x8* kf, const bf16x8* vf, f32x16* dk,
                                                 f32x16* dv, const uint16_t* qa,
                                                 const uint16_t* qc, const float* sLseb,
                                                 const float* sDlb, uint16_t* myPF, uint16_t* myDS,
                                                 const ColOffsets<32>& cp, int pw0, int pw1,
                                                 int q0, int kw0, int nq, int nkv, float sl2,
                                                 float psc, int lane) {
  using S = DkdvStage<D>;
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  const int h = lane >> 5, l32 = lane & 31;
  f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    s = mfma32x32x16(kf[kb], S::rows(qa, kb), s);
    dp = mfma32x32x16(vf[kb], S::rows(qa + S::DO, kb), dp);
  }
  // this lane: query q0 + l32, keys kw0 + 16h + v (v = 0..15)
  const int qj = q0 + l32;
  const float lse2 = sLseb[l32];
  const float dl = sDlb[l32];
  float p[16], ds[16];
  float amax = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = kw0 + 16 * h + v;
    const bool ok = qj < nq && key < nkv && (!CAUSAL || key <= qj);
    const float pv = fast_exp2(ok ? __builtin_fmaf(s[v], sl2, -lse2) : -INFINITY);
    ds[v] = pv * (dp[v] - dl);
    p[v] = pv * psc;
    amax = fmaxf(amax, p[v]);
  }
  const FastP fq(e4m3_scale_from_amax(amax));
  u32x4 pf[2], dsb[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y0, y1;
    fq.pair(p[2 * i], p[2 * i + 1], y0, y1);
    pf[i >> 2][i & 3] = pack_bf16x2(y0, y1);
    dsb[i >> 2][i & 3] = pack_bf16x2(ds[2 * i], ds[2 * i + 1]);
  }
  // P^F and dS as rows [query][key] of this wave's (swizzled) tiles
  *reinterpret_cast<u32x4*>(myPF + pw0) = pf[0];
  *reinterpret_cast<u32x4*>(myPF + pw1) = pf[1];
  *reinterpret_cast<u32x4*>(myDS + pw0) = dsb[0];
  *reinterpret_cast<u32x4*>(myDS + pw1) = dsb[1];
  wave_lds_fence();
  // dV += P^F^T dO and dK += dS^T Q^: A operands are key columns of the
  // [query][key] tiles, B operands are d columns of the [query][d] tiles.
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    const bf16x8 ap = lds_operand_cols_at(myPF + 16 * kq * 32, cp.a[0], cp.b[0]);
    const bf16x8 as = lds_operand_cols_at(myDS + 16 * kq * 32, cp.a[0], cp.b[0]);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dv[db] = mfma32x32x16(ap, S::cols(qc + S::DO, kq, db), dv[db]);
      dk[db] = mfma32x32x16(as, S::cols(qc, kq, db), dk[db]);
    }
  }
  wave_lds_fence();
}

// One slot of the interior software pipeline of k_dkdv (one wave, 32 keys).
// It runs the VALU work of sub-tile i (softmax recompute from lse, dS, the
// P fake-quant, the P^F/dS rows written to LDS) and, interleaved with it,
// the dV/dK MFMAs of sub-tile i-1 (from its P^F/dS tiles) and the S^T/dP^T
// MFMAs of sub-tile i+1.  The three streams are independent, so the MFMA
// pipe and the VALU overlap; scheduling fences keep the interleave and the
// LDS operands of each MFMA are read one step ahead.
template <int D>
__device__ __forceinline__ void dkdv_slot(
    // sub-tile i: S^T/dP^T accumulators, lse (log2 units) and delta of this
    // lane's query, destination P^F/dS tiles
    const f32x16& s, const f32x16& dp, float lse2, float dl, uint16_t* pfB, uint16_t* dsB,
    // sub-tile i-1: its P^F/dS tiles and its staged Q^ rows (column reads)
    const uint16_t* pfC, const uint16_t* dsC, const uint16_t* qc,
    // sub-tile i+1: its staged Q^ rows (row reads) and the S^T/dP^T results
    const uint16_t* qa, f32x16& sA, f32x16& dA,
    const bf16x8* kf, const bf16x8* vf, f32x16* dk, f32x16* dv, const ColOffsets<32>& cp,
    int pw0, int pw1, float sl2, float psc) {
  using S = DkdvStage<D>;
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int NC = 4 * DB;  // dV/dK MFMAs (2 k-blocks of 16 queries x DB x {dV, dK})
  constexpr int NA = 2 * KB;  // S^T/dP^T MFMAs
  constexpr int NS = 16;      // steps (VALU: 8 softmax steps, 8 quant steps)
  static_assert(NC <= NS && NA <= NS, "MFMA streams must fit the VALU steps");
  // B operands of the C stream (column reads) and of the A stream (row reads)
  auto opC = [&](int k) __attribute__((always_inline)) {
    return S::cols((k & 1) ? qc : qc + S::DO, k / (2 * DB), (k / 2) % DB);
  };
  auto opA = [&](int k) __attribute__((always_inline)) {
    return S::rows((k & 1) ? qa + S::DO : qa, k / 2);
  };
  constexpr int PD = ATTNQAT_DKDV_PREFETCH;  // LDS operand reads run PD steps ahead
  bf16x8 apC[2], asC[2], bC[NS + PD], bA[NS + PD];
  apC[0] = lds_operand_cols_at(pfC, cp.a[0], cp.b[0]);
  asC[0] = lds_operand_cols_at(dsC, cp.a[0], cp.b[0]);
#pragma unroll
  for (int k = 0; k < PD; ++k) {
    if (k < NC) bC[k] = opC(k);
    if (k < NA) bA[k] = opA(k);
  }
  sA = zero_f32x16();
  dA = zero_f32x16();
  float p[16], ds[16], amax = 0.0f, sc = 0.0f;
  u32x4 pf[2], dsb[2];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    // operands PD steps ahead
    if (k + PD < NC) bC[k + PD] = opC(k + PD);
    if (k + PD < NA) bA[k + PD] = opA(k + PD);
    if (k + PD == 2 * DB) {
      apC[1] = lds_operand_cols_at(pfC + 16 * 32, cp.a[0], cp.b[0]);
      asC[1] = lds_operand_cols_at(dsC + 16 * 32, cp.a[0], cp.b[0]);
    }
    if (k < NC) {
      const int kq = k / (2 * DB), db = (k / 2) % DB;
      if (k & 1)
        dk[db] = mfma32x32x16(asC[kq], bC[k], dk[db]);
      else
        dv[db] = mfma32x32x16(apC[kq], bC[k], dv[db]);
    }
    if (k < NA) {
      if (k & 1)
        dA = mfma32x32x16(vf[k / 2], bA[k], dA);
      else
        sA = mfma32x32x16(kf[k / 2], bA[k], sA);
    }
    if (k < 8) {
#pragma unroll
      for (int e = 2 * k; e < 2 * k + 2; ++e) {
        const float pv = fast_exp2(__builtin_fmaf(s[e], sl2, -lse2));
        ds[e] = pv * (dp[e] - dl);
        p[e] = pv * psc;
        amax = fmaxf(amax, p[e]);
      }
      if (k == 7) sc = e4m3_scale_from_amax(amax);
    } else {
      const int i = k - 8;
      const FastP fq(sc);
      float y0, y1;
      fq.pair(p[2 * i], p[2 * i + 1], y0, y1);
      pf[i >> 2][i & 3] = pin_vgpr(pack_bf16x2(y0, y1));
      dsb[i >> 2][i & 3] = pin_vgpr(pack_bf16x2(ds[2 * i], ds[2 * i + 1]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  *reinterpret_cast<u32x4*>(pfB + pw0) = pf[0];
  *reinterpret_cast<u32x4*>(pfB + pw1) = pf[1];
  *reinterpret_cast<u32x4*>(dsB + pw0) = dsb[0];
  *reinterpret_cast<u32x4*>(dsB + pw1) = dsb[1];
  wave_lds_fence();
}

// S^T/dP^T MFMAs of one sub-tile alone (fills the pipeline).
template <int D>
__device__ __forceinline__ void dkdv_fill(const uint16_t* qa, f32x16& sA, f32x16& dA,
                                          const bf16x8* kf, const bf16x8* vf) {
  using S = DkdvStage<D>;
  constexpr int KB = D / 16;
  sA = zero_f32x16();
  dA = zero_f32x16();
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    sA = mfma32x32x16(kf[kb], S::rows(qa, kb), sA);
    dA = mfma32x32x16(vf[kb], S::rows(qa + S::DO, kb), dA);
  }
}

// dV/dK MFMAs of one sub-tile alone (drains the pipeline).
template <int D>
__device__ __forceinline__ void dkdv_drain(const uint16_t* pfC, const uint16_t* dsC,
                                           const uint16_t* qc, f32x16* dk, f32x16* dv,
                                           const ColOffsets<32>& cp) {
  using S = DkdvStage<D>;
  constexpr int DB = D / 32;
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    const bf16x8 ap = lds_operand_cols_at(pfC + 16 * kq * 32, cp.a[0], cp.b[0]);
    const bf16x8 as = lds_operand_cols_at(dsC + 16 * kq * 32, cp.a[0], cp.b[0]);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dv[db] = mfma32x32x16(ap, S::cols(qc + S::DO, kq, db), dv[db]);
      dk[db] = mfma32x32x16(as, S::cols(qc, kq, db), dk[db]);
    }
  }
  wave_lds_fence();
}

// Workgroup: 4 waves x 32 keys.  Each wave keeps its K^/V^ rows in registers
// (A operands of S^T = K^ Q^T and dP^T = V dO^T, rows in key_perm order) and
// its dK/dV accumulators.  Query tiles of 64 rows (two 32-query sub-tiles)
// are staged in a ring of three LDS buffers: tile t+1 is written after
// sub-tile 0 of tile t and published by the one barrier per tile, and tile
// t+2 is then fetched into registers.  A tile's buffer is read from the
// second half of the tile before it to the first half of the tile after it;
// the third buffer lets the single barrier separate those reads from the
// next write of the same buffer.
//
// Interior tiles (no masks) run the slot pipeline over the sub-tile
// sequence; boundary tiles (causal diagonal first, a partial query tile
// last, everything when the workgroup's keys pass nkv) run self-contained
// masked sub-tiles, and the pipeline is filled and drained around the
// interior run.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ATTNQAT_DKDV_WAVES, 8)))
void k_dkdv(AttnArgs a) {
  using S = DkdvStage<D>;
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int BM = kDkvBM;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CH = BM * CPR / 256;  // chunks per thread per tensor per tile
  constexpr int NBUF = 3;
  static_assert(BM == 64 && CH >= 1 && kDkvBN % BM == 0, "two 32-query sub-tiles per tile");
  __shared__ __attribute__((aligned(16))) uint16_t sQO[NBUF * S::BUF];
  // per wave [query][key] tiles of P^F and dS, indexed by sub-tile parity
  __shared__ __attribute__((aligned(16))) uint16_t sPF[4][2][32 * 32];
  __shared__ __attribute__((aligned(16))) uint16_t sDS[4][2][32 * 32];
  __shared__ float sLse[NBUF][BM];
  __shared__ float sDl[NBUF][BM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y;
  const int nq = a.nq, nkv = a.nkv;
  const int kblk0 = blockIdx.x * kDkvBN;
  const int kw0 = kblk0 + wave * 32;
  const uint16_t* Q = a.q_hat + (size_t)bh * nq * D;
  const uint16_t* dO = a.d_o + (size_t)bh * nq * D;
  const uint16_t* K = a.k_hat + (size_t)bh * nkv * D;
  const uint16_t* V = a.v_hat + (size_t)bh * nkv * D;
  const float* LSE = a.lse + (size_t)bh * nq;
  const float* DL = a.delta + (size_t)bh * nq;

  bf16x8 kf[KB], vf[KB];
  {
    const int kr = kw0 + key_perm(l32);
    const bool ok = kr < nkv;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      kf[kb] = ok ? ld_bf16x8(K + (size_t)kr * D + 16 * kb + 8 * h) : zero_bf16x8();
      vf[kb] = ok ? ld_bf16x8(V + (size_t)kr * D + 16 * kb + 8 * h) : zero_bf16x8();
    }
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = zero_f32x16();
    dv[db] = zero_f32x16();
  }
  const float sl2 = a.softmax_scale * kLog2e;
  const float psc = a.p_scale;
  // LDS: this lane's row / column read positions in a staged tile, and its
  // column reads and row writes of the per-wave [query][key] tiles
  const uint16_t* const qrow = sQO + S::row_off(lane);
  const uint16_t* const qcol = sQO + S::col_off(lane);
  const ColOffsets<32> cp(8 * h, 8 * h + 4, lane);
  const int pw0 = swz<32>(l32, 16 * h), pw1 = swz<32>(l32, 16 * h + 8);
  uint16_t* const pf0 = sPF[wave][0];
  uint16_t* const pf1 = sPF[wave][1];
  uint16_t* const ds0 = sDS[wave][0];
  uint16_t* const ds1 = sDS[wave][1];

  // query tiles: below the workgroup's first key everything is masked (causal)
  const int qfirst = CAUSAL ? kblk0 : 0;
  const int ntiles = qfirst < nq ? (nq - qfirst + BM - 1) / BM : 0;

  u32x4 rq[CH], rd[CH];
  float rl = 0.0f, rdl = 0.0f;
  uint32_t voff[CH];  // byte offset of this thread's chunks within a tile
  int soff[CH];       // their element offset in a staged buffer
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = tid + 256 * c;
    voff[c] = (uint32_t)((idx / CPR) * D + (idx % CPR) * 8) * 2u;
    soff[c] = (idx / CPR) * S::P + (idx % CPR) * 8;
  }
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    // rows past nq read as zeros (masked out later); lse/delta are only
    // scaled when stored, so nothing waits for these loads here
    const int q0 = qfirst + t * BM;
    const int rows = min(nq - q0, BM);
    const uint32_t bytes = (uint32_t)(rows * D) * 2u;
    const auto rsq = make_rsrc(Q + (size_t)q0 * D, bytes);
    const auto rsd = make_rsrc(dO + (size_t)q0 * D, bytes);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      rq[c] = buf_ld16(rsq, voff[c]);
      rd[c] = buf_ld16(rsd, voff[c]);
    }
    if (tid < BM) {
      rl = buf_ldf(make_rsrc(LSE + q0, (uint32_t)rows * 4u), (uint32_t)tid * 4u);
      rdl = buf_ldf(make_rsrc(DL + q0, (uint32_t)rows * 4u), (uint32_t)tid * 4u);
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    uint16_t* const b = sQO + buf * S::BUF;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      *reinterpret_cast<u32x4*>(b + soff[c]) = rq[c];
      *reinterpret_cast<u32x4*>(b + S::DO + soff[c]) = rd[c];
    }
    if (tid < BM) {
      sLse[buf][tid] = rl * kLog2e;
      sDl[buf][tid] = rdl;
    }
  };
  // between the two sub-tiles of tile t: publish tile t+1, fetch tile t+2
  auto advance = [&](int t, int nbuf) __attribute__((always_inline)) {
    if (t + 1 < ntiles) store_tile(nbuf);
    __syncthreads();
    if (t + 2 < ntiles) load_tile(t + 2);
  };
  // self-contained masked sub-tile (skipped when every query is below the
  // wave's first key)
  auto masked_sub = [&](int t, int buf, int sub) __attribute__((always_inline)) {
    const int qs = qfirst + t * BM + 32 * sub;
    const int o = buf * S::BUF + sub * S::SUB;
    if (!(CAUSAL && qs + 31 < kw0))
      dkdv_tile_masked<D, CAUSAL>(kf, vf, dk, dv, qrow + o, qcol + o, sLse[buf] + 32 * sub,
                                  sDl[buf] + 32 * sub, pf0, ds0, cp, pw0, pw1, qs, kw0, nq, nkv,
                                  sl2, psc, lane);
  };
  auto masked_step = [&](int t, int buf, int nbuf) __attribute__((always_inline)) {
    masked_sub(t, buf, 0);
    advance(t, nbuf);
    masked_sub(t, buf, 1);
  };

  // Tiles needing masks: the causal diagonal (queries below the workgroup's
  // last key) at the start, a partial query tile at the end, or all tiles
  // when the workgroup's keys run past nkv.
  int it_lo = 0, it_hi = ntiles;
  if (kblk0 + kDkvBN > nkv) {
    it_lo = ntiles;
  } else {
    if (CAUSAL) it_lo = min(ntiles, (kblk0 + kDkvBN - 1 - qfirst + BM - 1) / BM);
    if (nq % BM != 0) it_hi = max(it_lo, ntiles - 1);
  }

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  vmem_wait_all();
  __syncthreads();
  if (ntiles > 1) load_tile(1);
  int buf = 0;  // t % NBUF
  int t = 0;
  for (; t < it_lo; ++t) {
    const int nbuf = buf == NBUF - 1 ? 0 : buf + 1;
    masked_step(t, buf, nbuf);
    buf = nbuf;
  }
  if (it_lo < it_hi) {
    // The first slot's dV/dK stream has no previous sub-tile: give it zero
    // P^F/dS tiles (with the current tile's finite Q^/dO as the other operand)
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(pf1 + pw0) = z;
    *reinterpret_cast<u32x4*>(pf1 + pw1) = z;
    *reinterpret_cast<u32x4*>(ds1 + pw0) = z;
    *reinterpret_cast<u32x4*>(ds1 + pw1) = z;
    wave_lds_fence();
    f32x16 s0, dp0, s1, dp1;
    dkdv_fill<D>(qrow + buf * S::BUF, s0, dp0, kf, vf);
    // column-read position in the previous tile's buffer (the current one at first)
    const uint16_t* cprev = qcol + buf * S::BUF;
    for (; t < it_hi; ++t) {
      const int nbuf = buf == NBUF - 1 ? 0 : buf + 1;
      const uint16_t* const rcur = qrow + buf * S::BUF;
      const uint16_t* const rnext = qrow + nbuf * S::BUF;
      const uint16_t* const ccur = qcol + buf * S::BUF;
      // sub-tile 0: C = sub-tile 1 of the previous tile, A = sub-tile 1
      dkdv_slot<D>(s0, dp0, sLse[buf][l32], sDl[buf][l32], pf0, ds0, pf1, ds1, cprev + S::SUB,
                   rcur + S::SUB, s1, dp1, kf, vf, dk, dv, cp, pw0, pw1, sl2, psc);
      advance(t, nbuf);
      // sub-tile 1: C = sub-tile 0, A = sub-tile 0 of the next tile (its
      // result is unused after the last interior tile)
      dkdv_slot<D>(s1, dp1, sLse[buf][32 + l32], sDl[buf][32 + l32], pf1, ds1, pf0, ds0, ccur,
                   rnext, s0, dp0, kf, vf, dk, dv, cp, pw0, pw1, sl2, psc);
      cprev = ccur;
      buf = nbuf;
    }
    dkdv_drain<D>(pf1, ds1, cprev + S::SUB, dk, dv, cp);
  }
  for (; t < ntiles; ++t) {
    const int nbuf = buf == NBUF - 1 ? 0 : buf + 1;
    masked_step(t, buf, nbuf);
    buf = nbuf;
  }

  // dK / dV accumulators: lane -> d = 32*db + l32, VGPR v -> key kw0 + 8*(v/4) + 4h + v%4
  const float ksc = a.softmax_scale;
  const float vsc = 1.0f / psc;
  uint16_t* DK = a.dk + (size_t)bh * nkv * D;
  uint16_t* DV = a.dv + (size_t)bh * nkv * D;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = kw0 + 8 * (v >> 2) + 4 * h + (v & 3);
    if (key < nkv) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        DK[(size_t)key * D + 32 * db + l32] = (uint16_t)f32_to_bf16_bits(dk[db][v] * ksc);
        DV[(size_t)key * D + 32 * db + l32] = (uint16_t)f32_to_bf16_bits(dv[db][v] * vsc);
      }
    }
  }
}

}  // namespace

hipError_t launch_bwd_dq(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((a.nq + kDqBM - 1) / kDqBM, a.bh);
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

hipError_t launch_bwd_dkdv(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((a.nkv + kDkvBN - 1) / kDkvBN, a.bh);
  if (head_dim == 128) {
    if (a.causal)
      hipLaunchKernelGGL((k_dkdv<128, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_dkdv<128, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.causal)
      hipLaunchKernelGGL((k_dkdv<64, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_dkdv<64, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attnqat
