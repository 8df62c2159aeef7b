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
//  * the running max only triggers a rescale of the accumulator when it
//    moved for some row of the wave (otherwise the factor is exactly 1),
//    applied just before the next tile's P^T V^ is added;
//  * only boundary tiles (the last key tiles: tail, causal diagonal) evaluate
//    masks; the leading tiles run a branch-free loop;
//  * causal: tiles with every key above the wave's last query are skipped
//    (and the key loop ends at the workgroup's last query); the diagonal
//    tile keeps the elementwise key <= query mask; keys >= Nkv are masked
//    and rows >= Nq are never stored (non-aligned tails);
//  * split over keys (non-causal, when the query tiles alone cannot fill the
//    chip: few queries against long K/V): blockIdx.y picks a run of key
//    tiles; each split stores its unnormalized O^T (fp32) with its row max
//    and sum, and k_fwd_combine merges the splits into O_hp and lse.
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

// O^T *= alpha when the row max moved at the previous tile (its pending
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

// Online-softmax update of (m, l) with the S^T of one tile (m: running row
// max in log2 units), producing P^T in bf16 (b), interleaved with the O^T
// MFMAs of the previous tile (b_prev, sVp) when ACC.  O^T then holds every
// earlier tile against the old max; when the max moved (for some row of the
// wave), the factor exp2(m_old - m_new) is left pending in (pending, alpha)
// and applied to O^T before this tile's P^T V^ is added.
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
  float xs[16], pv[16];
  uint32_t w[8];
  auto item = [&](int i) __attribute__((always_inline)) {
    if (i < 16) {
      float x = s[i] * sl2;
      if (MASK) {
        const int key = k0 + 8 * (i >> 2) + 4 * h + (i & 3);
        const bool ok = key < nkv && (!CAUSAL || key <= qi);
        x = ok ? x : -INFINITY;
      }
      xs[i] = x;
      tmax = fmaxf(tmax, x);
    } else if (i == 16) {
      tmax = fmaxf(tmax, xor32(tmax));
      mnew = fmaxf(m, tmax);
      base = (mnew == -INFINITY) ? 0.0f : mnew;
    } else if (i < 33) {
      const int e = i - 17;
      pv[e] = fast_exp2(xs[e] - base);
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
  // rescale only when some row's max moved; otherwise alpha would be exactly 1
  if (__any(mnew > m)) {
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
  static_assert(!(CAUSAL && SPLIT), "the split over keys is for non-causal attention");
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
  const uint16_t* Q = a.q_hat + (size_t)bh * nq * D;
  const uint16_t* K = a.k_hat + (size_t)bh * nkv * D;
  const uint16_t* V = a.v_hat + (size_t)bh * nkv * D;

  bf16x8 qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qf[kb] = (qi < nq) ? ld_bf16x8(Q + (size_t)qi * D + 16 * kb + 8 * h) : zero_bf16x8();

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
  if (CAUSAL) it_hi = min(it_hi, (qblk0 + 1) / BN);

  if constexpr (PACKED) {
    if (ntiles > 0) {
      load_packed(0);
      store_packed(0);
    }
    if (ntiles > 1) load_packed(1);
  } else {
    if (ntiles > 0) issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    vmem_wait_all();
  }
  __syncthreads();

  bf16x8 b_prev[2];
  bool have_prev = false;
  bool pending = false;  // O^T rescale by alpha before the next P^T V^ (see fwd_softmax_pv)
  float alpha = 1.0f;
  auto step = [&](int it, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = it % NB;
    const int pbuf = (it + NB - 1) % NB;
    const int k0 = (t0 + it) * BN;
    if constexpr (!PACKED) {
      if (it + 2 < ntiles) issue_tile(it + 2);
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
      if (it + 1 < ntiles) store_packed((it + 1) % NB);
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
  for (; it < it_hi; ++it) step(it, BoolTag<false>());
  for (; it < ntiles; ++it) step(it, BoolTag<true>());
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

// Merge of the key splits of k_fwd<..., SPLIT>: per query row, with M the
// largest split max and w_s = exp2(m_s - M), O_hp = sum_s w_s O_s / L and
// lse = (M + log2 L) ln 2, L = sum_s w_s l_s.  One thread per 4 columns of a
// row (D/4 threads per row); the splits are visited in order.
template <int D>
__global__ __launch_bounds__(256) void k_fwd_combine(AttnArgs a, int64_t rows) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / TPR;  // bh * nq + q
  if (row >= rows) return;
  const int c4 = (int)(g % TPR);
  const int S = a.kv_splits;
  const int64_t bh = row / a.nq, q = row % a.nq;
  const float* ml = a.ml_part + ((size_t)bh * S * a.nq + q) * 2;
  const size_t sstride = (size_t)a.nq * 2;  // split stride in ml_part
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[s * sstride]);
  const float base = M == -INFINITY ? 0.0f : M;
  const float* op = a.o_part + ((size_t)bh * S * a.nq + q) * D + 4 * c4;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float L = 0.0f;
  for (int s = 0; s < S; ++s) {
    const f32x2 mls = *reinterpret_cast<const f32x2*>(ml + s * sstride);
    const float w = fast_exp2(mls[0] - base);
    L = __builtin_fmaf(w, mls[1], L);
    const f32x4 v = *reinterpret_cast<const f32x4*>(op + (size_t)s * a.nq * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, v[e], acc[e]);
  }
  const float inv = 1.0f / L;
  uint16_t* O = a.o_hp + (size_t)row * D + 4 * c4;
  *reinterpret_cast<u32x2*>(O) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                       pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  if (c4 == 0) a.lse_out[row] = (M + __builtin_log2f(L)) * kLn2;
}

}  // namespace

template <bool PACKED>
hipError_t launch_fwd_t(const AttnArgs& a, int head_dim, hipStream_t stream,
                        const LaunchEvents* ev) {
  const unsigned qtiles = (unsigned)(((a.nq + kFwdBM - 1) / kFwdBM) * a.bh);
  const dim3 block(256);
  if (a.kv_splits > 1 && !a.causal) {
    // split over keys, then the merge (timed as one span: start of the
    // first launch to the end of the second)
    const dim3 grid(qtiles, (unsigned)a.kv_splits);
    const LaunchEvents e0 = {ev ? ev->start : nullptr, nullptr};
    const LaunchEvents e1 = {nullptr, ev ? ev->stop : nullptr};
    const hipError_t st = head_dim == 128
                              ? launch(k_fwd<128, false, PACKED, true>, grid, block, stream,
                                       ev ? &e0 : nullptr, a)
                              : launch(k_fwd<64, false, PACKED, true>, grid, block, stream,
                                       ev ? &e0 : nullptr, a);
    if (st != hipSuccess) return st;
    const int64_t rows = (int64_t)a.bh * a.nq;
    const int64_t threads = rows * (head_dim / 4);
    const dim3 cgrid((unsigned)((threads + 255) / 256));
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
