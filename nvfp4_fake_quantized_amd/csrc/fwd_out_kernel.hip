// Quantized, user-visible QAT forward output O = P^F V^ (Attn-QAT summary,
// §Method: the FP32 softmax probabilities are fake-quantized to P^F and
// combined with V^F to form the low-precision output).
//
// P is the normalized softmax P = exp(s Q^ K^T - lse), with the row's lse
// from the first forward pass, and P^F = fake_nvfp4(p_scale P) / p_scale in
// groups of 16 consecutive keys from key 0 -- the same P^F whose transpose
// the backward multiplies into dO for dV ("NVFP4 Attention QAT Backward",
// §Overview formula block), so dV is the straight-through gradient of this
// O.  This is the second pass of a two-pass forward; the first (k_fwd)
// produces O_hp and lse.
//
// gfx950 design (wave64, bf16 MFMA 32x32x16, fp32 accumulation): a
// workgroup of 4 waves owns 128 queries, each wave 32 (Q^ rows in VGPRs as
// the B operand of S^T = K^ Q^T).  The K^ rows of each 32-key tile are read
// in the permuted order pi, so the S^T accumulator gives every lane one query
// and 16 consecutive keys: one P group, whose amax, E4M3 scale and E2M1
// codes are per-lane work.  P^F^T then feeds the B operand of
// O^T = V^T P^F^T straight from registers, with the MFMA's k index mapped to
// keys so that lane half h supplies its own keys (16h + 8kb + i for k-block
// kb); the V^T operand reads the matching key rows with LDS transpose reads.
// Tiles reach a 4-deep LDS ring by direct global-to-LDS copies two tiles
// ahead, and step t issues the S^T MFMAs of tile t, then the P^F VALU work of
// tile t interleaved with the O^T MFMAs of tile t-1.  Masks (keys past nkv,
// causal keys above the query) give P = 0; only boundary tiles evaluate them.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kOutBM = 128;  // queries per workgroup
#ifndef ATTNQAT_FWDQ_AHEAD
#define ATTNQAT_FWDQ_AHEAD 2
#endif
constexpr int kOutAhead = ATTNQAT_FWDQ_AHEAD;  // MFMA operand reads issued this many ahead

// S^T = K^ Q^T of one 32-key tile, K^ rows in the order pi.
template <int D>
__device__ __forceinline__ void out_s(const bf16x8* qf, const uint16_t* sKb,
                                      const RowOffsets<D>& ro, f32x16& s) {
  constexpr int KB = D / 16;
  bf16x8 a[KB];
#pragma unroll
  for (int k = 0; k < kOutAhead; ++k) a[k] = ld_bf16x8(sKb + ro.o[k]);
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    if (k + kOutAhead < KB) a[k + kOutAhead] = ld_bf16x8(sKb + ro.o[k + kOutAhead]);
    s = mfma32x32x16(a[k], qf[k], k == 0 ? zero_f32x16() : s);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// V^T operand of O^T MFMA k: k-block kb = k / DB, d block k % DB; lane half h
// reads key rows 16h + 8kb .. +7 (ColOffsets cb[kb]).
template <int D>
__device__ __forceinline__ bf16x8 out_v_op(const uint16_t* sVb, const ColOffsets<D>* cb, int k) {
  constexpr int DB = D / 32;
  return lds_operand_cols_at(sVb, cb[k / DB].a[k % DB], cb[k / DB].b[k % DB]);
}

template <int D>
__device__ __forceinline__ void out_pv(f32x16* o, const bf16x8* b, const uint16_t* sVb,
                                       const ColOffsets<D>* cb) {
  constexpr int DB = D / 32;
  constexpr int NQ = 2 * DB;
  bf16x8 c[NQ];
#pragma unroll
  for (int k = 0; k < kOutAhead; ++k) c[k] = out_v_op<D>(sVb, cb, k);
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    if (k + kOutAhead < NQ) c[k + kOutAhead] = out_v_op<D>(sVb, cb, k + kOutAhead);
    o[k % DB] = mfma32x32x16(c[k], b[k / DB], o[k % DB]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// P, its group scale and P^F (bf16, into b) for one tile from S^T, with the
// O^T MFMAs of the previous tile (b_prev, sVp) interleaved when ACC.  Lane
// half h, VGPR v holds key k0 + 16h + v of query qi.
template <int D, bool CAUSAL, bool MASK, bool ACC, bool UNIT_P>
__device__ __forceinline__ void out_pf_pv(const f32x16& s, bf16x8* b, f32x16* o,
                                          const bf16x8* b_prev, const uint16_t* sVp,
                                          const ColOffsets<D>* cb, int k0, int h, int qi,
                                          int nkv, float sl2, float lse2, float psc) {
  constexpr int DB = D / 32;
  constexpr int NQ = 2 * DB;
  // VALU work items: 16 probabilities with the group amax, the scale,
  // 4 groups of 4 quotients, the codes, 8 dequantized pairs
  constexpr int NW = 16 + 1 + 4 + 1 + 8;
  bf16x8 c[NQ];
  if (ACC) {
#pragma unroll
    for (int k = 0; k < kOutAhead; ++k) c[k] = out_v_op<D>(sVp, cb, k);
  }
  int lim = 16;  // keys v < lim are valid (below nkv, not above the query)
  if (MASK) lim = (CAUSAL ? min(nkv, qi + 1) : nkv) - (k0 + 16 * h);
  float p[16];
  float amax = 0.0f, sc = 0.0f;
  f32x4 q4[4];
  uint32_t codes[2];
  uint32_t w[8];
  auto item = [&](int i) __attribute__((always_inline)) {
    if (i < 16) {
      float x = __builtin_fmaf(s[i], sl2, -lse2);
      if (MASK) x = i < lim ? x : -INFINITY;
      const float pv = fast_exp2(x);
      p[i] = UNIT_P ? pv : pv * psc;
      amax = fmaxf(amax, p[i]);
    } else if (i == 16) {
      sc = e4m3_scale_from_amax(amax);
    } else if (i < 21) {
      // a zero scale divides by 1 instead (its codes are then multiplied by 0)
      const FastP fq(sc > 0.0f ? sc : 1.0f);
      const int g = i - 17;
#pragma unroll
      for (int e = 0; e < 4; ++e) q4[g][e] = fq.quotient(p[4 * g + e]);
    } else if (i == 21) {
      codes[0] = FastP::codes8(q4[0], q4[1]);
      codes[1] = FastP::codes8(q4[2], q4[3]);
    } else {
      const int e = i - 22;
      float y0, y1;
      FastP::dequant_codes(codes[e >> 2], e & 3, sc, y0, y1);
      w[e] = pack_bf16x2(y0, y1);
    }
  };
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    if (ACC) {
      if (k + kOutAhead < NQ) c[k + kOutAhead] = out_v_op<D>(sVp, cb, k + kOutAhead);
      o[k % DB] = mfma32x32x16(c[k], b_prev[k / DB], o[k % DB]);
    }
    const int i0 = k * NW / NQ, i1 = (k + 1) * NW / NQ;
#pragma unroll
    for (int i = 0; i < NW; ++i)
      if (i >= i0 && i < i1) item(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  // k-block kb of the B operand: this lane's keys 16h + 8kb .. +7
  b[0] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
  b[1] = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
}

template <int D, bool CAUSAL, bool UNIT_P>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ATTNQAT_FWD_WAVES, 8)))
void k_fwd_out(AttnArgs a) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int BN = 32;              // keys per tile
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CH = BN * CPR / 256;  // 16-byte chunks per lane per tensor per tile
  constexpr int NB = 4;               // LDS ring: tiles t-1, t read while t+1, t+2 arrive
  static_assert(CH >= 1, "tile copy needs at least one chunk per lane");
  __shared__ __attribute__((aligned(16))) uint16_t sK[NB][BN * D];  // swizzled rows
  __shared__ __attribute__((aligned(16))) uint16_t sV[NB][BN * D];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const TileId t = xcd_tile((a.nq + kOutBM - 1) / kOutBM, CAUSAL);
  const int bh = t.bh;
  const int nq = a.nq, nkv = a.nkv;
  const int qblk0 = t.tile * kOutBM;
  const int qw0 = qblk0 + wave * 32;
  const int qi = qw0 + l32;
  const bool qok = qi < nq;
  const uint16_t* Q = a.q_hat + (size_t)bh * nq * D;
  const uint16_t* K = a.k_hat + (size_t)bh * nkv * D;
  const uint16_t* V = a.v_hat + (size_t)bh * nkv * D;

  bf16x8 qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qf[kb] = qok ? ld_bf16x8(Q + (size_t)qi * D + 16 * kb + 8 * h) : zero_bf16x8();
  // rows past nq: P = exp2(0 - 0) stays finite and is never stored
  const float lse2 = qok ? a.lse[(size_t)bh * nq + qi] * kLog2e : 0.0f;
  const float sl2 = a.softmax_scale * kLog2e;
  const float psc = a.p_scale;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero_f32x16();
  // K^ rows in the order pi; V^T key rows 16h + 8kb + 0..3 and + 4..7
  const RowOffsets<D> ro(lane, key_perm(l32));
  const ColOffsets<D> cb[2] = {ColOffsets<D>(16 * h, 16 * h + 4, lane),
                               ColOffsets<D>(16 * h + 8, 16 * h + 12, lane)};
  const int kend = CAUSAL ? min(nkv, qblk0 + kOutBM) : nkv;
  const int ntiles = (kend + BN - 1) / BN;

  // K^/V^ tiles go global -> LDS directly. Copy instruction c of this wave
  // fills LDS chunk slots 64*(CH*wave + c) + lane; slot (row r, position j)
  // of the XOR-swizzled layout holds column chunk swz(r, j) (an involution).
  uint32_t goff[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int p = 64 * (CH * wave + c) + lane;
    goff[c] = (uint32_t)swz<D>(p / CPR, 8 * (p % CPR)) * 2u;
  }
  auto issue_tile = [&](int it) __attribute__((always_inline)) {
    const int k0 = it * BN;
    const int buf = it % NB;
    // rows past nkv arrive as zeros (masked out)
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
  int it_hi = min(ntiles, nkv / BN);
  if (CAUSAL) it_hi = min(it_hi, (qblk0 + 1) / BN);

  if (ntiles > 0) issue_tile(0);
  if (ntiles > 1) issue_tile(1);
  vmem_wait_all();
  __syncthreads();

  bf16x8 b_prev[2];
  bool have_prev = false;
  auto step = [&](int it, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = it % NB;
    const int pbuf = (it + NB - 1) % NB;
    const int k0 = it * BN;
    if (it + 2 < ntiles) issue_tile(it + 2);
    // (boundary tiles only) every key above every query of this wave: skip;
    // every later tile is then skipped too
    if (!MASK || !(CAUSAL && qw0 + 31 < k0)) {
      f32x16 s;
      // the MFMA-only phase runs at raised wave priority (the other wave on
      // the SIMD fills its gaps)
      __builtin_amdgcn_s_setprio(1);
      out_s<D>(qf, sK[buf], ro, s);
      __builtin_amdgcn_s_setprio(0);
      bf16x8 b[2];
      if (have_prev)
        out_pf_pv<D, CAUSAL, MASK, true, UNIT_P>(s, b, o, b_prev, sV[pbuf], cb, k0, h, qi, nkv,
                                                 sl2, lse2, psc);
      else
        out_pf_pv<D, CAUSAL, MASK, false, UNIT_P>(s, b, o, b_prev, sV[pbuf], cb, k0, h, qi,
                                                  nkv, sl2, lse2, psc);
      b_prev[0] = b[0];
      b_prev[1] = b[1];
      have_prev = true;
    } else if (have_prev) {
      out_pv<D>(o, b_prev, sV[pbuf], cb);
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
  if (have_prev) out_pv<D>(o, b_prev, sV[(ntiles - 1) % NB], cb);

  if (qok) {
    const float inv = UNIT_P ? 1.0f : 1.0f / psc;  // P^F = fq(p_scale P) / p_scale
    uint16_t* O = a.o_q + (size_t)bh * nq * D + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 w = {pack_bf16x2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                         pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(O + 32 * db + 8 * g4 + 4 * h) = w;
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_out_d(const AttnArgs& a, hipStream_t stream, const LaunchEvents* ev) {
  const dim3 grid((unsigned)(((a.nq + kOutBM - 1) / kOutBM) * a.bh)), block(256);
  if (a.p_scale == 1.0f) return launch(k_fwd_out<D, CAUSAL, true>, grid, block, stream, ev, a);
  return launch(k_fwd_out<D, CAUSAL, false>, grid, block, stream, ev, a);
}

}  // namespace

hipError_t launch_fwd_out(const AttnArgs& a, int head_dim, hipStream_t stream,
                          const LaunchEvents* ev) {
  if (head_dim == 128)
    return a.causal ? launch_out_d<128, true>(a, stream, ev) : launch_out_d<128, false>(a, stream, ev);
  return a.causal ? launch_out_d<64, true>(a, stream, ev) : launch_out_d<64, false>(a, stream, ev);
}

}  // namespace attnqat
