// QAT forward on the fake-quantized Q^, K^, V^: O_hp = softmax(s Q^ K^T) V^
// and the natural-log lse ("NVFP4 Attention QAT Backward", §High-level
// wrapper: O_hp is the value saved before probability quantization; the
// Attn-QAT summary, fix 1, gives its reason).
//
// Work decomposition (gfx950, wave64, bf16 MFMA 32x32x16, fp32 accumulate):
//  * a workgroup of 4 waves owns 128 queries; each wave owns 32 queries and
//    keeps its Q^ rows in registers as the B operand of S^T = K^ Q^T;
//  * the key loop stages 32-key tiles of K^ and V^ row-major (XOR-swizzled
//    16-byte chunks) in a 4-deep LDS ring, copied global -> LDS directly two
//    tiles ahead; the V^T operand is read with LDS transpose reads;
//  * software pipeline: step t issues the S^T MFMAs of tile t (at raised
//    wave priority), then the softmax VALU work of tile t interleaved with
//    the O^T MFMAs of tile t-1;
//  * a PACKED instance reads K^/V^ from packed NVFP4 storage (E2M1 codes
//    and E4M3 scale bytes) through registers one tile ahead and writes the
//    exactly dequantized bf16 values into the same LDS tiles;
//  * S^T's accumulator layout puts one query per lane (and 16 of its keys in
//    VGPRs), so the online-softmax row statistics are per lane (plus one
//    exchange with the lane 32 away), and P^T feeds the B operand of
//    O^T = V^T P^T straight from registers;
//  * the exponent base m (a running max) moves only when some row's tile
//    max exceeds it by more than 2^8 (until then P stays below 256, which
//    bf16 holds with the same relative rounding); the rescale of the
//    accumulator that a move needs is applied just before the next tile's
//    P^T V^ is added;
//  * only boundary tiles (the last key tiles: tail, causal diagonal) evaluate
//    masks; the leading tiles run a branch-free loop;
//  * causal: tiles with every key above the wave's last query are skipped
//    (and the key loop ends at the workgroup's last query); the diagonal
//    tile keeps the elementwise key <= query mask; keys >= Nkv are masked
//    and rows >= Nq are never stored (non-aligned tails);
//  * split over keys (when the query tiles alone cannot fill the chip: few
//    queries against long K/V, or a short causal problem): blockIdx.y picks
//    a run of the workgroup's key tiles; each split stores its unnormalized
//    O^T (fp32) with its exponent base and sum (a split whose keys all lie
//    above the causal diagonal stores base -inf and sum 0), and k_fwd_combine
//    merges the splits into O_hp and lse.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kFwdBM = 128;  // queries per workgroup
#ifndef ATTNQAT_FWD_AHEAD
#define ATTNQAT_FWD_AHEAD 2
#endif
constexpr int kFwdAhead = ATTNQAT_FWD_AHEAD;  // MFMA operand reads issued this many MFMAs ahead
#ifndef ATTNQAT_FWD_RESCALE_LOG2
#define ATTNQAT_FWD_RESCALE_LOG2 8
#endif
// The running max m used as the exponent base moves only when some row's
// tile max exceeds it by more than this (log2 units); until then P = 2^(x - m)
// may reach 2^kRescaleLog2 (exact in bf16's range, same relative rounding),
// and O, l and the stored max stay consistent with the base actually used.
constexpr float kRescaleLog2 = ATTNQAT_FWD_RESCALE_LOG2;

// S^T = K^ Q^T of one 32-key tile (A operands read kFwdAhead MFMAs ahead).
template <int D>
__device__ __forceinline__ void fwd_s(const bf16x8* qf, const uint16_t* sKb,
                                      const RowOffsets<D>& ro, f32x16& s) {
  constexpr int KB = D / 16;
  bf16x8 a[KB];
#pragma unroll
  for (int k = 0; k < kFwdAhead; ++k) a[k] = ld_bf16x8(sKb + ro.o[k]);
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    if (k + kFwdAhead < KB) a[k + kFwdAhead] = ld_bf16x8(sKb + ro.o[k + kFwdAhead]);
    s = mfma32x32x16(a[k], qf[k], k == 0 ? zero_f32x16() : s);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T P^T of one tile (MFMA k: 16-key k-block k / DB, d block k % DB;
// lane half h, element e of k-block kh holds key 16*kh + 8*(e/4) + 4h + e%4
// in both operands).
template <int D>
__device__ __forceinline__ bf16x8 fwd_v_op(const uint16_t* sVb, const ColOffsets<D>& co, int k) {
  constexpr int DB = D / 32;
  return lds_operand_cols_at(sVb + 16 * (k / DB) * D, co.a[k % DB], co.b[k % DB]);
}
template <int D>
__device__ __forceinline__ void fwd_pv(f32x16* o, const bf16x8* b, const uint16_t* sVb,
                                       const ColOffsets<D>& co) {
  constexpr int DB = D / 32;
  constexpr int NQ = 2 * DB;
  bf16x8 c[NQ];
#pragma unroll
  for (int k = 0; k < kFwdAhead; ++k) c[k] = fwd_v_op<D>(sVb, co, k);
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    if (k + kFwdAhead < NQ) c[k + kFwdAhead] = fwd_v_op<D>(sVb, co, k + kFwdAhead);
    o[k % DB] = mfma32x32x16(c[k], b[k / DB], o[k % DB]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T *= alpha when the exponent base moved at the previous tile (its pending
// factor); the caller applies it before adding that tile's P^T V^.
template <int D>
__device__ __forceinline__ void fwd_rescale(f32x16* o, bool& pending, float alpha) {
  constexpr int DB = D / 32;
  if (pending) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    pending = false;
  }
}

// Online-softmax update of (m, l) with the S^T of one tile (m: the exponent
// base in log2 units, at least the row max minus kRescaleLog2), producing
// P^T in bf16 (b), interleaved with the O^T MFMAs of the previous tile
// (b_prev, sVp) when ACC.  O^T then holds every earlier tile against the old
// base; when the base moved (for some row of the wave), the factor
// exp2(m_old - m_new) is left pending in (pending, alpha) and applied to O^T
// before this tile's P^T V^ is added.
template <int D, bool CAUSAL, bool MASK, bool ACC>
__device__ __forceinline__ void fwd_softmax_pv(const f32x16& s, float& m, float& l, bf16x8* b,
                                               f32x16* o, const bf16x8* b_prev,
                                               const uint16_t* sVp, const ColOffsets<D>& co,
                                               bool& pending, float& alpha, int k0, int h,
                                               int qi, int nkv, float sl2) {
  constexpr int DB = D / 32;
  constexpr int NQ = 2 * DB;
  if (ACC) fwd_rescale<D>(o, pending, alpha);
  // VALU work items: 16 scaled (and masked) scores with the running tile max,
  // the row max across the lane pair, 16 exponentials with their sum, 8 packs
  constexpr int NW = 16 + 1 + 16 + 8;
  bf16x8 c[NQ];
  if (ACC) {
#pragma unroll
    for (int k = 0; k < kFwdAhead; ++k) c[k] = fwd_v_op<D>(sVp, co, k);
  }
  float tmax = -INFINITY, mnew = m, base = 0.0f, psum = 0.0f;
  bool up = false;
  float xs[16], pv[16];
  uint32_t w[8];
  auto item = [&](int i) __attribute__((always_inline)) {
    if (i < 16) {
      // the max of the raw scores (sl2 > 0: the max of the scaled ones after
      // one multiply, with the same rounding)
      float x = s[i];
      if (MASK) {
        const int key = k0 + 8 * (i >> 2) + 4 * h + (i & 3);
        const bool ok = key < nkv && (!CAUSAL || key <= qi);
        x = ok ? x : -INFINITY;
      }
      xs[i] = x;
      tmax = fmaxf(tmax, x);
    } else if (i == 16) {
      tmax = fmaxf(tmax, xor32(tmax)) * sl2;
      up = __any(tmax > m + kRescaleLog2);
      mnew = up ? fmaxf(m, tmax) : m;
      base = (mnew == -INFINITY) ? 0.0f : mnew;
    } else if (i < 33) {
      const int e = i - 17;
      pv[e] = fast_exp2(fmaf(xs[e], sl2, -base));
      psum += pv[e];
    } else {
      const int e = i - 33;
      w[e] = pack_bf16x2(pv[2 * e], pv[2 * e + 1]);
    }
  };
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    if (ACC) {
      if (k + kFwdAhead < NQ) c[k + kFwdAhead] = fwd_v_op<D>(sVp, co, k + kFwdAhead);
      o[k % DB] = mfma32x32x16(c[k], b_prev[k / DB], o[k % DB]);
    }
    const int i0 = k * NW / NQ, i1 = (k + 1) * NW / NQ;
#pragma unroll
    for (int i = 0; i < NW; ++i)
      if (i >= i0 && i < i1) item(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  b[0] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
  b[1] = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
  // rescale only when the base moved for some row; otherwise alpha would be exactly 1
  if (up) {
    alpha = fast_exp2(m - base);
    l *= alpha;
    pending = true;
  }
  l += psum;
  m = mnew;
}

template <int D, bool CAUSAL, bool PACKED, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ATTNQAT_FWD_WAVES, 8)))
void k_fwd(AttnArgs a) {
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
  const TileId t = xcd_tile((a.nq + kFwdBM - 1) / kFwdBM, CAUSAL);
  const int bh = t.bh;
  const int nq = a.nq, nkv = a.nkv;
  const int qblk0 = t.tile * kFwdBM;
  const int qw0 = qblk0 + wave * 32;
  const int qi = qw0 + l32;
  // with raw Q (q_in set) the workgroup fake-quantizes its own query rows
  // (a lane holds 8 columns of a 16-value group, the lane 32 away the other
  // 8), and the first key run writes Q^ and its scale bytes
  const bool qfuse = a.q_in != nullptr;
  const uint16_t* Q = (qfuse ? a.q_in : a.q_hat) + (size_t)bh * nq * D;
  const uint16_t* K = a.k_hat + (size_t)bh * nkv * D;
  const uint16_t* V = a.v_hat + (size_t)bh * nkv * D;

  bf16x8 qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qf[kb] = (qi < nq) ? ld_bf16x8(Q + (size_t)qi * D + 16 * kb + 8 * h) : zero_bf16x8();
  if (qfuse) {
    const bool wr = qi < nq && (!SPLIT || blockIdx.y == 0);
    const size_t row = (size_t)bh * nq + qi;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint32_t sb;
      qf[kb] = fq_half_group<32>(qf[kb], sb);
      if (wr) {
        *reinterpret_cast<bf16x8*>(a.q_hat_out + row * D + 16 * kb + 8 * h) = qf[kb];
        if (h == 0) a.q_scale_out[row * KB + kb] = (uint8_t)sb;
      }
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero_f32x16();
  float m = -INFINITY, l = 0.0f;
  const float sl2 = a.softmax_scale * kLog2e;
  // LDS offsets: K^ row reads and V^T column reads (k-block rows 4h.., 4h+8..)
  const RowOffsets<D> ro(lane);
  const ColOffsets<D> co(4 * h, 4 * h + 8, lane);
  const int kend = CAUSAL ? min(nkv, qblk0 + kFwdBM) : nkv;
  // key tiles t0 .. t0 + ntiles - 1 (all of them unless split over keys)
  int t0 = 0, ntiles = (kend + BN - 1) / BN;
  if constexpr (SPLIT) {
    const int per = (ntiles + a.kv_splits - 1) / a.kv_splits;
    t0 = (int)blockIdx.y * per;
    ntiles = max(0, min(ntiles, t0 + per) - t0);
  }

  // K^/V^ tiles go global -> LDS directly. Copy instruction c of this wave
  // fills LDS chunk slots 64*(CH*wave + c) + lane; slot (row r, position j)
  // of the XOR-swizzled layout holds column chunk swz(r, j) (an involution).
  uint32_t goff[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int p = 64 * (CH * wave + c) + lane;
    goff[c] = (uint32_t)swz<D>(p / CPR, 8 * (p % CPR)) * 2u;
  }
  auto issue_tile = [&](int it, int buf) __attribute__((always_inline)) {
    const int k0 = (t0 + it) * BN;
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
  // Packed K^/V^ (NVFP4 storage): thread g of the workgroup owns group g of
  // a tile (row g / GPR, columns 16 (g % GPR) ..): it loads the 8 code bytes
  // and the scale byte of K^ and of V^ one tile ahead, and at the end of the
  // step writes the dequantized bf16 values (exact) into the swizzled tile.
  constexpr int GPR = D / 16;             // groups per row
  constexpr int NG = BN * GPR;            // groups per tile
  const int pg = tid % NG, pr = pg / GPR, pgi = pg % GPR;
  const bool pown = tid < NG;
  const uint8_t* KC = a.k_codes + (size_t)bh * nkv * (D / 2);
  const uint8_t* KS = a.k_scales + (size_t)bh * nkv * GPR;
  const uint8_t* VC = a.v_codes + (size_t)bh * nkv * (D / 2);
  const uint8_t* VS = a.v_scales + (size_t)bh * nkv * GPR;
  u32x2 pkc = {0u, 0u}, pvc = {0u, 0u};
  uint32_t pks = 0u, pvs = 0u;
  auto load_packed = [&](int it) __attribute__((always_inline)) {
    const int k0 = (t0 + it) * BN;
    const int rows = min(nkv - k0, BN);  // rows past nkv read as zeros
    const auto rkc = make_rsrc(KC + (size_t)k0 * (D / 2), (uint32_t)rows * (D / 2));
    const auto rvc = make_rsrc(VC + (size_t)k0 * (D / 2), (uint32_t)rows * (D / 2));
    const auto rks = make_rsrc(KS + (size_t)k0 * GPR, (uint32_t)rows * GPR);
    const auto rvs = make_rsrc(VS + (size_t)k0 * GPR, (uint32_t)rows * GPR);
    const uint32_t off = (uint32_t)pg * 8u;
    pkc = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rkc, off, 0, 0));
    pvc = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rvc, off, 0, 0));
    pks = __builtin_amdgcn_raw_buffer_load_b8(rks, (uint32_t)pg, 0, 0);
    pvs = __builtin_amdgcn_raw_buffer_load_b8(rvs, (uint32_t)pg, 0, 0);
  };
  auto store_packed = [&](int buf) __attribute__((always_inline)) {
    if (!pown) return;
    auto put = [&](uint16_t* tile, u32x2 cw, uint32_t sb) __attribute__((always_inline)) {
      const float sc = e4m3_value(sb);
      u32x4 w[2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float y0, y1;
        FastP::dequant_codes(cw[i >> 2], i & 3, sc, y0, y1);
        w[i >> 2][i & 3] = pack_bf16x2(y0, y1);
      }
      *reinterpret_cast<u32x4*>(tile + swz<D>(pr, 16 * pgi)) = w[0];
      *reinterpret_cast<u32x4*>(tile + swz<D>(pr, 16 * pgi + 8)) = w[1];
    };
    put(sK[buf], pkc, pks);
    put(sV[buf], pvc, pvs);
  };

  // Leading tiles are interior (branch-free); masks start at the first tile
  // that reaches past nkv or above the workgroup's first query (causal).
  int it_hi = min(ntiles, max(0, nkv / BN - t0));
  if (CAUSAL) it_hi = min(it_hi, max(0, (qblk0 + 1) / BN - t0));

  if constexpr (PACKED) {
    if (ntiles > 0) {
      load_packed(0);
      store_packed(0);
    }
    if (ntiles > 1) load_packed(1);
  } else {
    if (ntiles > 0) issue_tile(0, 0);
    if (ntiles > 1) issue_tile(1, 1);
    vmem_wait_all();
  }
  __syncthreads();

  bf16x8 b_prev[2];
  bool have_prev = false;
  bool pending = false;  // O^T rescale by alpha before the next P^T V^ (see fwd_softmax_pv)
  float alpha = 1.0f;
  // buf = it % NB (a constant in the loop unrolled by NB: LDS addresses are
  // then the lane's offset plus an immediate)
  auto step = [&](int it, int buf, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int pbuf = (buf + NB - 1) % NB;
    const int k0 = (t0 + it) * BN;
    if constexpr (!PACKED) {
      if (it + 2 < ntiles) issue_tile(it + 2, (buf + 2) % NB);
    }
    // (boundary tiles only) every key above every query of this wave: skip;
    // every later tile is then skipped too
    if (!MASK || !(CAUSAL && qw0 + 31 < k0)) {
      f32x16 s;
      // the MFMA-only phase runs at raised wave priority (the other wave on
      // the SIMD fills its gaps)
      __builtin_amdgcn_s_setprio(1);
      fwd_s<D>(qf, sK[buf], ro, s);
      __builtin_amdgcn_s_setprio(0);
      bf16x8 b[2];
      if (have_prev)
        fwd_softmax_pv<D, CAUSAL, MASK, true>(s, m, l, b, o, b_prev, sV[pbuf], co, pending,
                                              alpha, k0, h, qi, nkv, sl2);
      else
        fwd_softmax_pv<D, CAUSAL, MASK, false>(s, m, l, b, o, b_prev, sV[pbuf], co, pending,
                                               alpha, k0, h, qi, nkv, sl2);
      b_prev[0] = b[0];
      b_prev[1] = b[1];
      have_prev = true;
    } else if (have_prev) {
      fwd_rescale<D>(o, pending, alpha);
      fwd_pv<D>(o, b_prev, sV[pbuf], co);
      have_prev = false;
    }
    if constexpr (PACKED) {
      // buffer (it+1) % NB last held tile it-3
      if (it + 1 < ntiles) store_packed((buf + 1) % NB);
      if (it + 2 < ntiles) load_packed(it + 2);
    } else {
      // tile it+1 has landed (this wave's copies; the barrier covers the
      // other waves'), tile it+2 may still be in flight
      if (it + 2 < ntiles)
        vmem_wait<2 * CH>();
      else
        vmem_wait<0>();
    }
    __syncthreads();
  };
  int it = 0;
  if constexpr (D == 128) {  // (at D = 64 the unrolled loop costs occupancy and is slower)
    for (; it + NB <= it_hi; it += NB) {
      static_for<NB>([&](auto j) __attribute__((always_inline)) {
        step(it + decltype(j)::value, decltype(j)::value, BoolTag<false>());
      });
    }
  }
  for (; it < it_hi; ++it) step(it, it % NB, BoolTag<false>());
  for (; it < ntiles; ++it) step(it, it % NB, BoolTag<true>());
  // the last tile's O^T (its tile is still resident)
  if (have_prev) {
    fwd_rescale<D>(o, pending, alpha);
    fwd_pv<D>(o, b_prev, sV[(ntiles - 1) % NB], co);
  }

  const float lt = l + xor32(l);
  if constexpr (SPLIT) {
    // this split's unnormalized O^T row, its max (log2 units) and its sum;
    // a split without keys stores m = -inf, l = 0 and O = 0
    if (qi < nq) {
      const size_t row = ((size_t)bh * a.kv_splits + blockIdx.y) * nq + qi;
      float* op = a.o_part + row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 w = {o[db][4 * g4], o[db][4 * g4 + 1], o[db][4 * g4 + 2],
                           o[db][4 * g4 + 3]};
          *reinterpret_cast<f32x4*>(op + 32 * db + 8 * g4 + 4 * h) = w;
        }
      }
      if (h == 0) *reinterpret_cast<f32x2*>(a.ml_part + 2 * row) = f32x2{m, lt};
    }
    return;
  }
  if (qi < nq) {
    const float inv = 1.0f / lt;
    uint16_t* O = a.o_hp + (size_t)bh * nq * D + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 w = {pack_bf16x2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                         pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(O + 32 * db + 8 * g4 + 4 * h) = w;
      }
    }
    if (h == 0) a.lse_out[(size_t)bh * nq + qi] = (m + __builtin_log2f(lt)) * kLn2;
  }
}

// Merge of the key runs of k_fwd<..., SPLIT> and k_fwd_dec: per query row,
// with m_s a run's exponent base (O_s and l_s are sums of exp2(x - m_s)), M
// the largest base and w_s = exp2(m_s - M), O_hp = sum_s w_s O_s / L and
// lse = (M + log2 L) ln 2, L = sum_s w_s l_s.  One thread per 4 columns
// of a row (D/4 threads per row); the runs are read 32 at a time (their
// loads in flight together: one memory round trip for up to 32 runs) and
// folded into a running max with rescaled sums.
template <int D>
__global__ __launch_bounds__(256) void k_fwd_combine(AttnArgs a, int64_t rows) {
  constexpr int TPR = D / 4;  // threads per row
  constexpr int B8 = 32;      // runs per batch
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / TPR;  // bh * nq + q
  if (row >= rows) return;
  const int c4 = (int)(g % TPR);
  const int S = a.kv_splits;
  const int64_t bh = row / a.nq, q = row % a.nq;
  const float* ml = a.ml_part + ((size_t)bh * S * a.nq + q) * 2;
  const size_t sstride = (size_t)a.nq * 2;  // run stride in ml_part
  const float* op = a.o_part + ((size_t)bh * S * a.nq + q) * D + 4 * c4;
  float M = -INFINITY, L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < S; s0 += B8) {
    f32x2 mls[B8];
    f32x4 v[B8];
#pragma unroll
    for (int k = 0; k < B8; ++k) {
      const bool in = s0 + k < S;
      mls[k] = in ? *reinterpret_cast<const f32x2*>(ml + (s0 + k) * sstride) : f32x2{-INFINITY, 0.0f};
      v[k] = in ? *reinterpret_cast<const f32x4*>(op + (size_t)(s0 + k) * a.nq * D)
                : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float bm = M;
#pragma unroll
    for (int k = 0; k < B8; ++k) bm = fmaxf(bm, mls[k][0]);
    const float base = bm == -INFINITY ? 0.0f : bm;
    const float r = fast_exp2(M - base);  // 0 while M is -inf (L and acc are 0 then)
    L *= r;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= r;
#pragma unroll
    for (int k = 0; k < B8; ++k) {
      const float w = fast_exp2(mls[k][0] - base);
      L = __builtin_fmaf(w, mls[k][1], L);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, v[k][e], acc[e]);
    }
    M = bm;
  }
  const float inv = 1.0f / L;
  uint16_t* O = a.o_hp + (size_t)row * D + 4 * c4;
  *reinterpret_cast<u32x2*>(O) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                       pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  if (c4 == 0) a.lse_out[row] = (M + __builtin_log2f(L)) * kLn2;
}

// ---------------------------------------------------------------------------
// Forward for few queries against long K/V (non-causal, Nq <= 32 per head):
// the same QAT forward with 32-query tiles, so that a decode-like problem
// does not compute 128-query tiles that are mostly padding, and so that the
// K/V stream (bf16 or packed NVFP4) is what bounds it.
//  * a workgroup of 4 waves owns 32 queries of one head; its waves work on
//    their own (no barrier in the key loop).  The W = 4 * splits waves of a
//    head deal the key tiles out round-robin (wave g takes tiles g, g + W,
//    ...), so that at any time the waves of a head stream neighbouring tiles
//    rather than W distant runs (measured no faster than contiguous runs,
//    and no slower); each wave visits its tiles from the last one down, so
//    the only partial tile of the head comes first and only that step
//    evaluates a mask;
//  * the workgroup's Q^ rows sit in LDS and are read as the B operand of
//    S^T = K^ Q^T (given the raw Q rows, the kernel fake-quantizes them
//    itself, and the first key run writes Q^ and its scale bytes to the
//    workspace);
//  * bf16 K^ rows go global -> registers (A operands) one tile ahead, V^
//    tiles global -> LDS directly one tile ahead; given raw K/V instead,
//    both go to registers one tile ahead, and at the start of the tile's step
//    the wave fake-quantizes them (each key tile has one owner), writes V^
//    into its LDS tile and K^, V^ and their scale bytes to the workspace;
//  * packed K^/V^: codes and scale bytes of two tiles ahead in registers,
//    dequantized to fp16 (exact: see dec_scale) and multiplied on fp16 MFMAs
//    (Q^ staged in fp16, also exact; P^T rounded to fp16, finer than the bf16
//    of the other paths).  K^ operands are dequantized beside the S^T MFMAs
//    (the head dimension is split between the lane halves as h*D/2 + 8j + e
//    for MFMA j, the order of a dot product's terms being free, so that a
//    lane's codes of a key row are one contiguous run); V^ is dequantized
//    beside the O^T MFMAs of the previous tile and written with 16-byte
//    stores whose rows are chosen so that each group of 8 lanes hits 8
//    different bank groups;
//  * V^ is read from a per-wave pair of LDS tiles in the swizzled layout of
//    k_fwd with transpose reads;
//  * at the end the 4 waves are merged in LDS (the largest of the waves'
//    exponent bases, exp2-weighted sums) into one unnormalized partial (O,
//    base, row sum) per workgroup, which k_fwd_combine merges over the
//    workgroups.
constexpr int kDecBQ = 32;  // queries per workgroup

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Every E2M1 code times an E4M3 scale is exact in fp16 (at most 6
// significant bits, magnitudes 2^-10 .. 2688).  gfx950's FP4 conversion
// applies only the power-of-two part of its f32 scale operand, so a scale
// s = 2^e * f (1 <= f < 2 with 3 fraction bits) is applied in two exact
// steps: the conversion with 2^e, then a packed fp16 multiply by f.
struct DecScale {
  float p2;     // 2^e (f32; 0 for a zero scale, whose codes are all zero)
  uint32_t f2;  // f as an fp16 pair
};
// (the scale byte is byte SEL of the word `bytes`)
template <int SEL>
__device__ __forceinline__ DecScale dec_scale(uint32_t bytes) {
  const uint32_t b = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8((int)bytes, SEL));
  return {__uint_as_float(b & 0xFF800000u), (0x3C00u | ((b >> 13) & 0x3FFu)) * 0x10001u};
}

// fp16 x8 of the 8 E2M1 codes of one dword (byte b: element 2b in the low
// nibble, 2b+1 in the high one) times the scale.
__device__ __forceinline__ u32x4 dec_dequant8(uint32_t cw, DecScale sc) {
  const f16x2 f = __builtin_bit_cast(f16x2, sc.f2);
  u32x4 w;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f16x2 c;
    switch (b) {  // the byte select is an instruction immediate
      case 0: c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc.p2, 0); break;
      case 1: c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc.p2, 1); break;
      case 2: c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc.p2, 2); break;
      default: c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc.p2, 3); break;
    }
    w[b] = __builtin_bit_cast(uint32_t, c * f);
  }
  return w;
}

// 32x32x16 MFMA on bf16 or fp16 operands (passed as 16-byte words).
template <bool F16>
__device__ __forceinline__ f32x16 dec_mfma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Row of the V^ tile whose D/2 columns (half hh = lane / 32) lane `lane`
// dequantizes (packed): within each group of 8 lanes the swizzle phases of
// the rows differ in their low 3 bits, so 16-byte stores of one chunk column
// by 8 lanes fall into 8 different 16-byte bank groups.
template <int D>
__device__ __forceinline__ int dec_v_row(int lane) {
  const int b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1;
  const int b3 = (lane >> 3) & 1, b4 = (lane >> 4) & 1;
  if constexpr (D == 128) return b0 + 4 * b1 + 8 * b2 + 2 * b3 + 16 * b4;
  else return 2 * b0 + 4 * b1 + 8 * b2 + b3 + 16 * b4;
}

template <int D, bool PACKED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_fwd_dec(AttnArgs a) {
  constexpr int KB = D / 16;       // MFMAs per S^T tile
  constexpr int DB = D / 32;
  constexpr int NQ = 2 * DB;       // MFMAs per O^T tile
  constexpr int BN = 32;           // keys per tile
  constexpr int VT = BN * D;       // bf16 elements per V^ tile
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int CH = VT / 8 / 64;  // 16-byte V^ copies per lane per tile (bf16)
  constexpr int CW = D / 64;       // 16-byte code loads per lane per tensor per tile (packed)
  constexpr int GPR = D / 16;      // scale bytes per row
  constexpr int MS = D + 4;        // merge row stride (floats): conflict-free 16-byte stores
  constexpr int QS = D + 8;        // Q^ row stride (elements): conflict-free 16-byte reads
  constexpr int RING = 4 * 2 * VT * 2;
  constexpr int MERGE = 4 * kDecBQ * MS * 4;
  constexpr int LDS = RING > MERGE ? RING : MERGE;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kDecBQ * QS];
  __shared__ float s_m[4][kDecBQ], s_l[4][kDecBQ];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int S = a.kv_splits;
  const int bh = (int)blockIdx.x / S, sp = (int)blockIdx.x % S;
  const int nq = a.nq, nkv = a.nkv;
  const int q0 = (int)blockIdx.y * kDecBQ;
  const int qi = q0 + l32;
  uint16_t* ring = reinterpret_cast<uint16_t*>(smem) + wave * 2 * VT;

  // this wave's key tiles: g, g + W, ... (W waves per head), last one first
  const int ntiles_all = (nkv + BN - 1) / BN;
  const int W = 4 * S, g = 4 * sp + wave;
  const int n = g < ntiles_all ? (ntiles_all - 1 - g) / W + 1 : 0;
  auto tile_k0 = [&](int it) __attribute__((always_inline)) { return (g + W * (n - 1 - it)) * BN; };

  // Q^ rows of the workgroup (rows past nq as zeros; fp16 for packed K^/V^)
  if (a.q_in != nullptr) {
    // fake-quantize the raw Q rows here (one 16-value group per thread, the
    // codec's arithmetic); the first key run writes Q^ and the scale bytes
    constexpr int NGRP = kDecBQ * GPR;  // groups of the tile
    for (int g = tid; g < NGRP; g += 256) {
      const int r = g / GPR, col = 16 * (g % GPR);
      const bool in = q0 + r < nq;
      const size_t off = ((size_t)bh * nq + q0 + r) * D + col;
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (in) {
        lo = *reinterpret_cast<const u32x4*>(a.q_in + off);
        hi = *reinterpret_cast<const u32x4*>(a.q_in + off + 8);
      }
      float x[16];
      unpack_bf16x16(lo, hi, x);
      const float sc = fq16(x);
      if (in && sp == 0) {
        pack_bf16x16(x, lo, hi);
        *reinterpret_cast<u32x4*>(a.q_hat_out + off) = lo;
        *reinterpret_cast<u32x4*>(a.q_hat_out + off + 8) = hi;
        a.q_scale_out[off / 16] = (uint8_t)e4m3_byte(sc);
      }
      if constexpr (PACKED) {
        f16x8 h0, h1;  // exact: E2M1 codes times E4M3 scales
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          h0[e] = (_Float16)x[e];
          h1[e] = (_Float16)x[8 + e];
        }
        *reinterpret_cast<f16x8*>(sQ + r * QS + col) = h0;
        *reinterpret_cast<f16x8*>(sQ + r * QS + col + 8) = h1;
      } else {
        pack_bf16x16(x, lo, hi);
        *reinterpret_cast<u32x4*>(sQ + r * QS + col) = lo;
        *reinterpret_cast<u32x4*>(sQ + r * QS + col + 8) = hi;
      }
    }
  } else {
    const uint16_t* Q = a.q_hat + (size_t)bh * nq * D;
#pragma unroll
    for (int c = 0; c < kDecBQ * CPR / 256; ++c) {
      const int p = 256 * c + tid, r = p / CPR, col = 8 * (p % CPR);
      const bf16x8 v = (q0 + r < nq) ? ld_bf16x8(Q + (size_t)(q0 + r) * D + col) : zero_bf16x8();
      if constexpr (PACKED) {
        f16x8 hv;  // exact: Q^ values are E2M1 codes times E4M3 scales
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (_Float16)(float)v[e];
        *reinterpret_cast<f16x8*>(sQ + r * QS + col) = hv;
      } else {
        st_bf16x8(sQ + r * QS + col, v);
      }
    }
  }
  // head-dimension column of element 0 of MFMA j's operands in lane half h
  const uint16_t* qrow = sQ + l32 * QS + (PACKED ? h * (D / 2) : 8 * h);
  constexpr int QJ = PACKED ? 8 : 16;  // column step per MFMA

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero_f32x16();
  float m = -INFINITY, l = 0.0f;
  bool pending = false;
  float alpha = 1.0f;
  const float sl2 = a.softmax_scale * kLog2e;
  const ColOffsets<D> co(4 * h, 4 * h + 8, lane);

  // ---- bf16 K^ rows (registers) and V^ tiles (LDS copies); with raw K/V
  // (k_in set) the kernel fake-quantizes them itself: each key tile belongs
  // to one wave of one key run, which writes its K^, V^ and scale bytes
  const bool fuse = !PACKED && a.k_in != nullptr;
  const uint16_t* K = (fuse ? a.k_in : a.k_hat) + (size_t)bh * nkv * D;
  const uint16_t* V = (fuse ? a.v_in : a.v_hat) + (size_t)bh * nkv * D;
  bf16x8 kr[PACKED ? 1 : KB];
  bf16x8 vraw[PACKED ? 1 : CH];
  auto load_k = [&](int it) __attribute__((always_inline)) {
    const int k0 = tile_k0(it);
    const auto r = make_rsrc(K + (size_t)k0 * D, (uint32_t)(min(nkv - k0, BN) * D) * 2u);
    const uint32_t off = (uint32_t)(l32 * D + 8 * h) * 2u;
#pragma unroll
    for (int j = 0; j < (PACKED ? 1 : KB); ++j)
      kr[j] = __builtin_bit_cast(bf16x8, buf_ld16(r, off + 32u * j));
  };
  auto copy_v = [&](int it) __attribute__((always_inline)) {
    const int k0 = tile_k0(it);
    const u32x4 d = buf_desc(V + (size_t)k0 * D, (uint32_t)(min(nkv - k0, BN) * D) * 2u);
    uint16_t* dst = ring + (it & 1) * VT;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // slot 64c + lane of the tile holds row p / CPR, column chunk swz(p)
      const int p = 64 * c + lane;
      buf_ld16_lds(d, (uint32_t)swz<D>(p / CPR, 8 * (p % CPR)) * 2u,
                   __builtin_amdgcn_readfirstlane(lds_addr(dst + 512 * c)));
    }
  };
  // raw V rows of tile it into registers, chunk for chunk as copy_v places
  // them (rows past nkv read as zeros)
  auto load_v_raw = [&](int it) __attribute__((always_inline)) {
    const int k0 = tile_k0(it);
    const auto r = make_rsrc(V + (size_t)k0 * D, (uint32_t)(min(nkv - k0, BN) * D) * 2u);
#pragma unroll
    for (int c = 0; c < (PACKED ? 1 : CH); ++c) {
      const int p = 64 * c + lane;
      vraw[c] = __builtin_bit_cast(bf16x8, buf_ld16(r, (uint32_t)swz<D>(p / CPR, 8 * (p % CPR)) * 2u));
    }
  };
  // fake-quantize tile it: K^ in place in kr (a lane holds 8 columns of a
  // 16-value group, the lane 32 away the other 8), V^ into this wave's LDS
  // tile (chunk slot p = 64c + lane holds column chunk swz_chunk(row, p % CPR);
  // the other half of its group sits in slot p ^ 1, lane ^ 1), and both to
  // the workspace with their scale bytes (rows below nkv only)
  auto quant_kv = [&](int it) __attribute__((always_inline)) {
    const int k0 = tile_k0(it);
    const size_t row0 = (size_t)bh * nkv + k0;
#pragma unroll
    for (int j = 0; j < (PACKED ? 1 : KB); ++j) {
      uint32_t sb;
      kr[j] = fq_half_group<32>(kr[j], sb);
      if (k0 + l32 < nkv) {
        *reinterpret_cast<bf16x8*>(a.k_hat_out + (row0 + l32) * D + 16 * j + 8 * h) = kr[j];
        if (h == 0) a.k_scale_out[(row0 + l32) * GPR + j] = (uint8_t)sb;
      }
    }
    uint16_t* dst = ring + (it & 1) * VT;
#pragma unroll
    for (int c = 0; c < (PACKED ? 1 : CH); ++c) {
      const int p = 64 * c + lane, r = p / CPR, lc = swz_chunk<D>(r, p % CPR);
      uint32_t sb;
      const bf16x8 vq = fq_half_group<1>(vraw[c], sb);
      *reinterpret_cast<bf16x8*>(dst + 512 * c + 8 * lane) = vq;
      if (k0 + r < nkv) {
        *reinterpret_cast<bf16x8*>(a.v_hat_out + (row0 + r) * D + 8 * lc) = vq;
        if ((lc & 1) == 0) a.v_scale_out[(row0 + r) * GPR + lc / 2] = (uint8_t)sb;
      }
    }
  };

  // ---- packed K^/V^: codes and scale bytes of two tiles in registers
  const uint8_t* KC = a.k_codes + (size_t)bh * nkv * (D / 2);
  const uint8_t* KS = a.k_scales + (size_t)bh * nkv * GPR;
  const uint8_t* VC = a.v_codes + (size_t)bh * nkv * (D / 2);
  const uint8_t* VS = a.v_scales + (size_t)bh * nkv * GPR;
  const int vr = dec_v_row<D>(lane);  // V^ row this lane dequantizes
  u32x4 kc[2][CW], vc[2][CW];
  uint32_t ks[2], vs[2];
  auto load_codes = [&](int it, auto slot_tag) __attribute__((always_inline)) {
    constexpr int sl = decltype(slot_tag)::value;
    const int k0 = tile_k0(it);
    const uint32_t rows = (uint32_t)min(nkv - k0, BN);  // rows past nkv read as zeros
    const auto rkc = make_rsrc(KC + (size_t)k0 * (D / 2), rows * (D / 2));
    const auto rks = make_rsrc(KS + (size_t)k0 * GPR, rows * GPR);
    const auto rvc = make_rsrc(VC + (size_t)k0 * (D / 2), rows * (D / 2));
    const auto rvs = make_rsrc(VS + (size_t)k0 * GPR, rows * GPR);
    const uint32_t ko = (uint32_t)(l32 * (D / 2) + h * (D / 4));
    const uint32_t vo = (uint32_t)(vr * (D / 2) + h * (D / 4));
#pragma unroll
    for (int c = 0; c < CW; ++c) kc[sl][c] = buf_ld16(rkc, ko + 16u * c);
    if constexpr (D == 128)
      ks[sl] = __builtin_amdgcn_raw_buffer_load_b32(rks, (uint32_t)(l32 * GPR + 4 * h), 0, 0);
    else
      ks[sl] = __builtin_amdgcn_raw_buffer_load_b16(rks, (uint32_t)(l32 * GPR + 2 * h), 0, 0);
#pragma unroll
    for (int c = 0; c < CW; ++c) vc[sl][c] = buf_ld16(rvc, vo + 16u * c);
    if constexpr (D == 128)
      vs[sl] = __builtin_amdgcn_raw_buffer_load_b32(rvs, (uint32_t)(vr * GPR + 4 * h), 0, 0);
    else
      vs[sl] = __builtin_amdgcn_raw_buffer_load_b16(rvs, (uint32_t)(vr * GPR + 2 * h), 0, 0);
  };
  // K^ operand j of the tile in slot sl: codes dword j of the lane's run,
  // scale byte j/2 of the lane's scale bytes
  auto k_op_packed = [&](auto j_tag, auto slot_tag) __attribute__((always_inline)) -> u32x4 {
    constexpr int j = decltype(j_tag)::value;
    constexpr int sl = decltype(slot_tag)::value;
    return dec_dequant8(kc[sl][j / 4][j % 4], dec_scale<j / 2>(ks[sl]));
  };
  // V^ piece c of the tile in slot sl (row vr, columns h*D/2 + 8c ..) into dst
  auto v_store_packed = [&](auto c_tag, auto slot_tag, uint16_t* dst) __attribute__((always_inline)) {
    constexpr int c = decltype(c_tag)::value;
    constexpr int sl = decltype(slot_tag)::value;
    *reinterpret_cast<u32x4*>(dst + swz<D>(vr, h * (D / 2) + 8 * c)) =
        dec_dequant8(vc[sl][c / 4][c % 4], dec_scale<c / 2>(vs[sl]));
  };

  // one key tile: S^T, the online softmax, O^T += V^T P^T from the tile's
  // LDS tile.  The next tile's V^ goes into the other LDS tile (it held
  // tile it-1, whose reads finished in the previous step).
  auto step = [&](int it, auto slot_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr int sl = decltype(slot_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = tile_k0(it);
    const bool more = it + 1 < n;
    f32x16 s;
    u32x4 qb[KB];
    auto ldq = [&](int j) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4*>(qrow + QJ * j);
    };
    if constexpr (PACKED) {
      u32x4 ka[KB];
      ka[0] = k_op_packed(IntTag<0>(), slot_tag);
      qb[0] = ldq(0);
      static_for<KB>([&](auto jt) __attribute__((always_inline)) {
        constexpr int j = decltype(jt)::value;
        if constexpr (j + 1 < KB) {
          ka[j + 1] = k_op_packed(IntTag<j + 1>(), slot_tag);
          qb[j + 1] = ldq(j + 1);
        }
        s = dec_mfma<true>(ka[j], qb[j], j == 0 ? zero_f32x16() : s);
        __builtin_amdgcn_sched_barrier(0);
      });
      // slot sl is free now (K^ of tile it consumed, V^ of tile it in LDS)
      if (it + 2 < n) load_codes(it + 2, slot_tag);
    } else {
      if (fuse) quant_kv(it);  // this tile's raw rows arrived during the previous step
#pragma unroll
      for (int k = 0; k < kFwdAhead; ++k) qb[k] = ldq(k);
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        if (j + kFwdAhead < KB) qb[j + kFwdAhead] = ldq(j + kFwdAhead);
        s = dec_mfma<false>(__builtin_bit_cast(u32x4, kr[j]), qb[j], j == 0 ? zero_f32x16() : s);
        __builtin_amdgcn_sched_barrier(0);
      }
      // V^ of tile it+1 before K^ of tile it+1: loads complete in issue
      // order, so the wait for K^ at the next step also covers this copy
      if (more) {
        if (fuse)
          load_v_raw(it + 1);
        else
          copy_v(it + 1);
        load_k(it + 1);
      }
    }

    // online softmax (S^T rows = keys 8*(i/4) + 4h + i%4, one query per lane)
    // (the max of the raw scores, then one multiply by sl2 > 0; the base
    // moves only past kRescaleLog2, as in k_fwd)
    float xs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) xs[i] = s[i];
    if constexpr (MASK) {
      const int rem = nkv - k0 - 4 * h;  // keys of this lane half left in the tile
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) >= rem) xs[i] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, xs[i]);
    tmax = fmaxf(tmax, xor32(tmax)) * sl2;
    const bool up = __any(tmax > m + kRescaleLog2);
    const float mnew = up ? fmaxf(m, tmax) : m;
    const float base = (mnew == -INFINITY) ? 0.0f : mnew;
    float psum = 0.0f;
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = fast_exp2(fmaf(xs[2 * e], sl2, -base));
      const float p1 = fast_exp2(fmaf(xs[2 * e + 1], sl2, -base));
      psum += p0 + p1;
      if constexpr (PACKED)
        w[e] = __builtin_bit_cast(uint32_t, f16x2{(_Float16)p0, (_Float16)p1});
      else
        w[e] = pack_bf16x2(p0, p1);
    }
    const u32x4 b[2] = {u32x4{w[0], w[1], w[2], w[3]}, u32x4{w[4], w[5], w[6], w[7]}};
    if (up) {
      alpha = fast_exp2(m - base);
      l *= alpha;
      pending = true;
    }
    l += psum;
    m = mnew;
    fwd_rescale<D>(o, pending, alpha);

    const uint16_t* sVb = ring + (it & 1) * VT;
    uint16_t* nxt = ring + ((it + 1) & 1) * VT;
    u32x4 c[NQ];
#pragma unroll
    for (int k = 0; k < kFwdAhead; ++k) c[k] = __builtin_bit_cast(u32x4, fwd_v_op<D>(sVb, co, k));
    static_for<NQ>([&](auto kt) __attribute__((always_inline)) {
      constexpr int k = decltype(kt)::value;
      if constexpr (k + kFwdAhead < NQ)
        c[k + kFwdAhead] = __builtin_bit_cast(u32x4, fwd_v_op<D>(sVb, co, k + kFwdAhead));
      o[k % DB] = dec_mfma<PACKED>(c[k], b[k / DB], o[k % DB]);
      if constexpr (PACKED) {
        if (more) v_store_packed(IntTag<k>(), IntTag<1 - sl>(), nxt);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  __syncthreads();  // Q^ staged
  if constexpr (PACKED) {
    if (n > 0) {
      load_codes(0, IntTag<0>());
      static_for<KB>([&](auto ct) __attribute__((always_inline)) {
        v_store_packed(ct, IntTag<0>(), ring);
      });
    }
    if (n > 1) load_codes(1, IntTag<1>());
  } else {
    if (n > 0) {
      if (fuse)
        load_v_raw(0);
      else
        copy_v(0);
      load_k(0);
    }
  }
  // tile 0 is the only one that can reach past nkv; the rest in slot pairs
  if (n > 0) step(0, IntTag<0>(), BoolTag<true>());
  for (int it = 1; it < n; it += 2) {
    step(it, IntTag<1>(), BoolTag<false>());
    if (it + 1 < n) step(it + 1, IntTag<0>(), BoolTag<false>());
  }

  // merge of the 4 waves: M = max of the wave maxima, each wave's O^T and
  // row sum weighted by exp2(m_w - M) (0 for a wave without keys)
  const float lt = l + xor32(l);
  __syncthreads();  // the merge buffer overlaps the V^ tiles
  if (h == 0) s_m[wave][l32] = m;
  __syncthreads();
  {
    const float M = fmaxf(fmaxf(s_m[0][l32], s_m[1][l32]), fmaxf(s_m[2][l32], s_m[3][l32]));
    const float f = fast_exp2(m - (M == -INFINITY ? 0.0f : M));
    float* mw = reinterpret_cast<float*>(smem) + (wave * kDecBQ + l32) * MS;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v = {o[db][4 * g4] * f, o[db][4 * g4 + 1] * f, o[db][4 * g4 + 2] * f,
                         o[db][4 * g4 + 3] * f};
        *reinterpret_cast<f32x4*>(mw + 32 * db + 8 * g4 + 4 * h) = v;
      }
    }
    if (h == 0) s_l[wave][l32] = lt * f;
  }
  __syncthreads();
  // thread -> query row tid % 32, columns (tid / 32) * D/8 ..
  const int q = tid & 31, part = tid >> 5;
  if (q0 + q < nq) {
    const size_t row = ((size_t)bh * S + sp) * nq + q0 + q;
    const float* src = reinterpret_cast<const float*>(smem) + q * MS + part * (D / 8);
    float* dst = a.o_part + row * D + part * (D / 8);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      f32x4 acc = *reinterpret_cast<const f32x4*>(src + 4 * i);
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + w * kDecBQ * MS + 4 * i);
        acc += v;
      }
      *reinterpret_cast<f32x4*>(dst + 4 * i) = acc;
    }
    if (part == 0) {
      const float M = fmaxf(fmaxf(s_m[0][q], s_m[1][q]), fmaxf(s_m[2][q], s_m[3][q]));
      const float L = (s_l[0][q] + s_l[1][q]) + (s_l[2][q] + s_l[3][q]);
      *reinterpret_cast<f32x2*>(a.ml_part + 2 * row) = f32x2{M, L};
    }
  }
}

}  // namespace

template <bool PACKED>
hipError_t launch_fwd_t(const AttnArgs& a, int head_dim, hipStream_t stream,
                        const LaunchEvents* ev) {
  const unsigned qtiles = (unsigned)(((a.nq + kFwdBM - 1) / kFwdBM) * a.bh);
  const dim3 block(256);
  const int64_t rows = (int64_t)a.bh * a.nq;
  const dim3 cgrid((unsigned)((rows * (head_dim / 4) + 255) / 256));
  const LaunchEvents e0 = {ev ? ev->start : nullptr, nullptr};
  const LaunchEvents e1 = {nullptr, ev ? ev->stop : nullptr};
  if (a.kv_decode && !a.causal) {
    // 32-query tiles over key runs, then the merge (one timed span)
    const dim3 grid((unsigned)(a.bh * a.kv_splits), (unsigned)((a.nq + kDecBQ - 1) / kDecBQ));
    const hipError_t st =
        head_dim == 128 ? launch(k_fwd_dec<128, PACKED>, grid, block, stream, ev ? &e0 : nullptr, a)
                        : launch(k_fwd_dec<64, PACKED>, grid, block, stream, ev ? &e0 : nullptr, a);
    if (st != hipSuccess) return st;
    return head_dim == 128
               ? launch(k_fwd_combine<128>, cgrid, block, stream, ev ? &e1 : nullptr, a, rows)
               : launch(k_fwd_combine<64>, cgrid, block, stream, ev ? &e1 : nullptr, a, rows);
  }
  if (a.kv_splits > 1) {
    // split over keys, then the merge (timed as one span: start of the
    // first launch to the end of the second)
    const dim3 grid(qtiles, (unsigned)a.kv_splits);
    const LaunchEvents* es = ev ? &e0 : nullptr;
    const hipError_t st =
        head_dim == 128
            ? (a.causal ? launch(k_fwd<128, true, PACKED, true>, grid, block, stream, es, a)
                        : launch(k_fwd<128, false, PACKED, true>, grid, block, stream, es, a))
            : (a.causal ? launch(k_fwd<64, true, PACKED, true>, grid, block, stream, es, a)
                        : launch(k_fwd<64, false, PACKED, true>, grid, block, stream, es, a));
    if (st != hipSuccess) return st;
    return head_dim == 128
               ? launch(k_fwd_combine<128>, cgrid, block, stream, ev ? &e1 : nullptr, a, rows)
               : launch(k_fwd_combine<64>, cgrid, block, stream, ev ? &e1 : nullptr, a, rows);
  }
  const dim3 grid(qtiles);
  if (head_dim == 128)
    return a.causal ? launch(k_fwd<128, true, PACKED, false>, grid, block, stream, ev, a)
                    : launch(k_fwd<128, false, PACKED, false>, grid, block, stream, ev, a);
  return a.causal ? launch(k_fwd<64, true, PACKED, false>, grid, block, stream, ev, a)
                  : launch(k_fwd<64, false, PACKED, false>, grid, block, stream, ev, a);
}

hipError_t launch_fwd(const AttnArgs& a, int head_dim, hipStream_t stream,
                      const LaunchEvents* ev) {
  return launch_fwd_t<false>(a, head_dim, stream, ev);
}

hipError_t launch_fwd_packed(const AttnArgs& a, int head_dim, hipStream_t stream) {
  return launch_fwd_t<true>(a, head_dim, stream, nullptr);
}

}  // namespace attnqat
