// QAT backward, key side: dK and dV with the fake-quantized probabilities
// ("NVFP4 Attention QAT Backward", §Overview formula block and the dK/dV
// kernel of its four-kernel split):
//
//   P   = exp(s Q^ K^T - lse)          recomputed per tile, fp32
//   dS  = P * (dO V^T - delta)         delta = rowsum(O_hp * dO)
//   dK  = s dS^T Q^                    straight-through: the unquantized P
//   dV  = fq(P)^T dO                   fq: fake_nvfp4, 16 consecutive keys
//
// gfx950 design (wave64, bf16 MFMA 32x32x16, fp32 accumulation).
//
// A workgroup of 8 waves owns 128 keys, as four pairs of waves that share a
// SIMD (waves w and w+4).  The two waves of a pair split the work on their
// 32 keys by role; per 32-query step:
//  * wave X (w < 4) keeps the pair's K^ and V^ rows (A operands).  At step j
//    it issues the MFMAs of S^T(j+1) = K^ Q^T and dP^T(j+1) = V^ dO^T (one
//    step ahead, with operands read from LDS two MFMAs ahead; the dP^T chain
//    starts from -delta through one extra MFMA) interleaved with the VALU
//    work on S^T(j) and dP^T(j): P = exp2(S s log2e - lse log2e), the group
//    amax and E4M3 scale, dS = P (dP - delta), the quotients P / scale, their
//    E2M1 codes (rounded like the exact quotient, i.e. precise division) and
//    P^F = code * scale (exact in bf16).  It writes the dS and P^F tiles
//    (bf16) to LDS, and stages the Q^/dO sub-tiles two steps ahead.
//  * wave Y (w >= 4) keeps the dV and dK accumulators.  At step j it adds
//    dS^T Q^ and P^F^T dO of sub-tile j-1 (16 MFMAs, operands from LDS
//    transpose reads) and issues no VALU work.
// One barrier per step orders the handover.
//
// In the S^T accumulator each lane holds one query and, because the K^/V^
// rows are loaded in the permuted order pi, 16 *consecutive* keys: exactly
// one P quantization group, so the amax and the scale are per-lane work.
// The Q^/dO sub-tiles (32 queries) sit in a ring of four LDS slots
// (XOR-swizzled rows; row reads for S/dP, transpose reads for dK/dV); X
// waves copy them global -> LDS directly, two steps ahead.  The step loops are
// unrolled by the ring period, so every LDS address is a lane register plus
// an immediate.  P^F and dS reach the A operands of dV and dK through
// [query][key] LDS tiles read back with transpose reads.
//
// Masks: only sub-tiles on a boundary (causal diagonal, query tail, keys past
// nkv) evaluate them, in X (P = 0, hence dS = 0 and P^F = 0); causal
// sub-tiles entirely above the diagonal are skipped by both waves.  Loads
// beyond the ends read zeros and stores stop at the ends.
//
// When the key blocks cannot fill the chip, the query sub-tiles of each
// block are split over blockIdx.y: each split writes its fp32 dK and dV
// partials, and k_sum_parts (launched next, with dQ's sums) adds the splits
// in order (deterministic).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kKeys = 128;     // keys per workgroup
constexpr int kSub = 32;       // queries per sub-tile
constexpr int kThreads = 512;  // 4 X waves + 4 Y waves
constexpr int kStagers = 256;  // the X waves stage the sub-tiles
constexpr int kRing = 4;       // Q^/dO sub-tile slots (also the unroll factor)
#ifndef ATTNQAT_DKDV_AHEAD
#define ATTNQAT_DKDV_AHEAD 2
#endif
#ifndef ATTNQAT_DKDV_AHEAD_Y
#define ATTNQAT_DKDV_AHEAD_Y 6
#endif
#ifndef ATTNQAT_DKDV_SGB
#define ATTNQAT_DKDV_SGB 1
#endif
#ifndef ATTNQAT_DKDV_SGB_VALU
#define ATTNQAT_DKDV_SGB_VALU 8
#endif
constexpr int kAhead = ATTNQAT_DKDV_AHEAD;     // X: MFMA operand reads issued this many MFMAs ahead
constexpr int kAheadY = ATTNQAT_DKDV_AHEAD_Y;  // Y: the same

// Element offset of (row r, column c) in a [query][key] handover tile (32 x 32
// bf16, 64-byte rows): 16-byte chunk c / 8 of row r sits at chunk position
// (c / 8) ^ ((r >> 1) & 3).  gfx950's LDS takes writes at 128 bytes per clock
// (32 banks of 4 bytes: 8 lanes of a 16-byte write) and reads at 256 (64
// banks); a probe of SQ_LDS_BANK_CONFLICT over write patterns fits that model
// exactly.  X writes row l32 in 16-byte pieces, 8 lanes (rows) per clock:
// rows of one parity share a 64-byte half of the 128-byte bank window and
// the swizzle gives each of the 4 a different chunk.  Y's transpose reads
// (lanes 0-31: 4 whole consecutive rows) cover 256 bytes once for any
// permutation within a row.  Both patterns are conflict-free.
__device__ __forceinline__ int hoff(int r, int c) {
  return r * 32 + 8 * ((c >> 3) ^ ((r >> 1) & 3)) + (c & 7);
}

template <int N>
struct IntTag {
  static constexpr int value = N;
};

// LDS map (bytes).  The ring comes first so that its offsets fit the 16-bit
// immediate of LDS instructions.
template <int D>
struct DkdvLds {
  static constexpr int SUBT = kSub * D * 2;             // one Q^ or dO sub-tile (bf16)
  static constexpr int RING = 0;                        // slot r: Q^ at 2r SUBT, dO at (2r+1) SUBT
  static constexpr int PAIR = RING + kRing * 2 * SUBT;  // per-pair buffers start here
  // offsets within the per-pair area
  static constexpr int DS = 0;                       // dS[pair][2] 32x32 bf16 tiles
  static constexpr int PF = DS + 4 * 2 * 2048;       // P^F[pair][2] 32x32 bf16 tiles
  static constexpr int LSE = PF + 4 * 2 * 2048;      // lse[kRing][64] (raw; 32 used)
  static constexpr int DL = LSE + kRing * 64 * 4;    // delta[kRing][64]
  static constexpr int TOTAL = PAIR + DL + kRing * 64 * 4;
};

// X-wave VALU items of one step and their approximate instruction counts:
// 16 elements, the scale, 4 quotient groups, 2 halves of P^F, the dS rows.
constexpr int kXItems = 24;
constexpr int x_item_cost(int i) {
  return i < 16 ? 6 : i == 16 ? 5 : i < 21 ? 12 : i < 23 ? 22 : 10;
}
// MFMA slot (of nslot) in which item i is issued: items in order, spread by cost
constexpr int x_item_slot(int i, int nslot) {
  int before = 0, total = 0;
  for (int t = 0; t < kXItems; ++t) {
    if (t < i) before += x_item_cost(t);
    total += x_item_cost(t);
  }
  return before * nslot / total;
}

template <int D, bool CAUSAL, bool UNIT_P>
__global__ __launch_bounds__(kThreads) void k_dkdv(AttnArgs a) {
  using L = DkdvLds<D>;
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int NCH = kSub * CPR;         // chunks per tensor per sub-tile
  constexpr int CH = 2 * NCH / kStagers;  // chunks per staging thread per sub-tile
  static_assert(CH >= 1 && (2 * NCH) % kStagers == 0 && NCH % 64 == 0,
                "sub-tile staging shape");
  static_assert(2 * kRing * L::SUBT <= 65536, "ring offsets fit LDS immediates");
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::TOTAL];

  const int tid = threadIdx.x;
  // wave index in a scalar register: role and key-block branches are uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const bool is_x = wave < 4;  // role
  const int kk = wave & 3;     // the pair's 32-key block
  const TileId t = xcd_tile((a.nkv + kKeys - 1) / kKeys);
  const int bh = t.bh;
  const int nq = a.nq, nkv = a.nkv;
  const int kblk0 = t.tile * kKeys;
  const int kw0 = kblk0 + 32 * kk;
  const uint16_t* Q = a.q_hat + (size_t)bh * nq * D;
  const uint16_t* dO = a.d_o + (size_t)bh * nq * D;
  const float* LSE = a.lse + (size_t)bh * nq;
  const float* DL = a.delta + (size_t)bh * nq;

  // sub-tiles: queries below the workgroup's first key are masked (causal)
  const int qfirst = CAUSAL ? kblk0 : 0;
  const int nsub_all = qfirst < nq ? (nq - qfirst + kSub - 1) / kSub : 0;
  // this workgroup's sub-tiles: all of them, or run blockIdx.y of the split
  const int QSPL = a.dkdv_splits > 1 ? a.dkdv_splits : 1;
  const int per = (nsub_all + QSPL - 1) / QSPL;
  const int js0 = QSPL > 1 ? (int)blockIdx.y * per : 0;
  const int nsub = QSPL > 1 ? max(0, min(nsub_all - js0, per)) : nsub_all;
  const int qstart = qfirst + kSub * js0;  // first query of sub-tile 0
  const int nsteps = nsub > 0 ? nsub + 1 : 0;
  // a sub-tile entirely above the pair's keys (causal) is skipped by both waves
  auto skipped = [&](int j) __attribute__((always_inline)) {
    return CAUSAL && qstart + kSub * j + kSub - 1 < kw0;
  };

  auto ring = [&](int slot, int tensor) __attribute__((always_inline)) {
    return reinterpret_cast<const uint16_t*>(smem + L::RING + (2 * slot + tensor) * L::SUBT);
  };
  uint8_t* const pair = smem + L::PAIR;
  uint16_t* const dstile = reinterpret_cast<uint16_t*>(pair + L::DS + kk * 2 * 2048);
  uint16_t* const pftile = reinterpret_cast<uint16_t*>(pair + L::PF + kk * 2 * 2048);
  // tile row writes: row l32, columns 16h .. 16h + 15
  const int hw0 = hoff(l32, 16 * h), hw1 = hoff(l32, 16 * h + 8);
  auto write_tile_row = [&](uint16_t* tile, const u32x4& lo, const u32x4& hi)
      __attribute__((always_inline)) {
    *reinterpret_cast<u32x4*>(tile + hw0) = lo;
    *reinterpret_cast<u32x4*>(tile + hw1) = hi;
  };

  if (is_x) {
    // K^ and V^ rows of the pair's keys, in the order pi (A operands)
    bf16x8 kf[KB], vf[KB];
    {
      const size_t base = ((size_t)bh * nkv + kblk0) * D;
      const uint32_t bytes = (uint32_t)(min(nkv - kblk0, kKeys) * D) * 2u;
      const bool fuse = a.k_in != nullptr;  // raw K/V: quantize here
      const auto rk = make_rsrc((fuse ? a.k_in : a.k_hat) + base, bytes);
      const auto rv = make_rsrc((fuse ? a.v_in : a.v_hat) + base, bytes);
      const int row = 32 * kk + key_perm(l32);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t off = (uint32_t)(row * D + 16 * kb + 8 * h) * 2u;
        kf[kb] = __builtin_bit_cast(bf16x8, buf_ld16(rk, off));
        vf[kb] = __builtin_bit_cast(bf16x8, buf_ld16(rv, off));
      }
      if (fuse) {
        // group kb of the row: columns 16 kb .. 16 kb + 15, this lane's half
        // at 8 h (rows past nkv arrived as zeros and are not written)
        const bool wr = blockIdx.y == 0 && kblk0 + row < nkv;
        const size_t r = (size_t)bh * nkv + kblk0 + row;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          uint32_t sk, sv;
          kf[kb] = fq_half_group<32>(kf[kb], sk);
          vf[kb] = fq_half_group<32>(vf[kb], sv);
          if (wr) {
            *reinterpret_cast<bf16x8*>(a.k_hat_out + r * D + 16 * kb + 8 * h) = kf[kb];
            *reinterpret_cast<bf16x8*>(a.v_hat_out + r * D + 16 * kb + 8 * h) = vf[kb];
            if (h == 0) {
              a.k_scale_out[r * KB + kb] = (uint8_t)sk;
              a.v_scale_out[r * KB + kb] = (uint8_t)sv;
            }
          }
        }
      }
    }
    const bool keys_tail = kw0 + 32 > nkv;
    // A operand of the delta MFMA: k = 0, 1, 2 of every key row are -1 (bf16
    // 0xBF80), the other k are 0
    const bf16x8 adl = __builtin_bit_cast(
        bf16x8, h == 0 ? u32x4{0xBF80BF80u, 0x0000BF80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
    const RowOffsets<D> ro(lane);  // row reads (S, dP B operands)

    // ---- staging of sub-tile j (Q^ and dO rows, lse, delta) into slot j % kRing,
    // copied global -> LDS directly.  Copy instruction c of X wave w fills the
    // slot's LDS chunks 64*(CH*w + c) + lane (the Q^ tile, then the dO tile);
    // chunk (row r, position jj) of the XOR-swizzled layout holds column chunk
    // swz(r, jj), so each lane fetches that chunk (the swizzle is an
    // involution).  Waves 0 and 1 copy the sub-tile's lse and delta.
    uint32_t goff[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int pc = (64 * (CH * wave + c) + lane) % NCH;
      goff[c] = (uint32_t)swz<D>(pc / CPR, 8 * (pc % CPR)) * 2u;
    }
    auto issue_sub = [&](int j, auto stag) __attribute__((always_inline)) {
      constexpr int S = decltype(stag)::value;  // ring slot
      const int q0 = qstart + kSub * j;
      const int rows = min(nq - q0, kSub);
      const uint32_t bytes = (uint32_t)(rows * D) * 2u;  // rows past nq arrive as zeros
      const u32x4 dq_ = buf_desc(Q + (size_t)q0 * D, bytes);
      const u32x4 dd_ = buf_desc(dO + (size_t)q0 * D, bytes);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const bool is_q = CH * wave + c < NCH / 64;  // uniform per instruction
        buf_ld16_lds(is_q ? dq_ : dd_, goff[c],
                     __builtin_amdgcn_readfirstlane(lds_addr(
                         smem + L::RING + 2 * S * L::SUBT + 16 * 64 * (CH * wave + c))));
      }
      if (wave < 2)  // lanes past the sub-tile read zeros
        buf_ld4_lds(buf_desc((wave == 0 ? LSE : DL) + q0, (uint32_t)rows * 4u),
                    (uint32_t)lane * 4u,
                    __builtin_amdgcn_readfirstlane(
                        lds_addr(pair + (wave == 0 ? L::LSE : L::DL) + S * 64 * 4)));
    };

    const float sl2 = a.softmax_scale * kLog2e;
    const float psc = a.p_scale;
    const float* const slse = reinterpret_cast<const float*>(pair + L::LSE);
    const float* const sdl = reinterpret_cast<const float*>(pair + L::DL);  // [kRing][64]
    // MFMA k of a sub-tile (slot RN): S^T for even k, dP^T for odd k, over
    // head-dim block k / 2
    auto operand = [&](int k, auto rntag) __attribute__((always_inline)) {
      constexpr int RN = decltype(rntag)::value;
      return ld_bf16x8(ring(RN, k & 1) + ro.o[k >> 1]);
    };

    // One step: MFMAs of sub-tile j+1 (slot RN, when DO_M) interleaved with
    // the VALU work on sub-tile j (slot R, when DO_V) from sc / dc.
    auto x_step_body = [&](int j, auto rtag, auto dom_tag, auto dov_tag, auto mask_tag,
                           const f32x16& sc, const f32x16& dc, f32x16& sn, f32x16& dn)
        __attribute__((always_inline)) {
      constexpr int R = decltype(rtag)::value;
      constexpr int RN = (R + 1) % kRing;
      constexpr bool DO_M = decltype(dom_tag)::value;
      constexpr bool DO_V = decltype(dov_tag)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr int NM = 2 * KB;  // MFMAs per sub-tile
      bf16x8 b[NM];
      bf16x8 bdl;  // -delta of sub-tile j+1 as three bf16 terms (see adl)
      if (DO_M) {
#pragma unroll
        for (int k = 0; k < kAhead; ++k) b[k] = operand(k, IntTag<RN>());
        // delta = d1 + d2 + d3 exactly: d1, d2 take the top 8 significant
        // bits of delta and of its remainder (exact truncations), d3 the
        // last 8 (fits bf16)
        const float dl1 = sdl[RN * 64 + l32];
        const float d1 = __uint_as_float(__float_as_uint(dl1) & 0xFFFF0000u);
        const float r1 = dl1 - d1;
        const float d2 = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
        const float d3 = r1 - d2;
        bdl = __builtin_bit_cast(bf16x8, u32x4{pack_exact_bf16x2(d1, d2),
                                               __float_as_uint(d3) >> 16, 0u, 0u});
      }
      float lse2 = 0.0f;
      int lim = 16;
      if (DO_V) {
        lse2 = slse[R * 64 + l32] * kLog2e;
        // this lane: query qj, keys kw0 + 16h + v; under MASK key v is valid
        // when v < lim (below nkv, not above the query, query below nq)
        if (MASK) {
          const int qj = qstart + kSub * j + l32;
          lim = (CAUSAL ? min(nkv, qj + 1) : nkv) - (kw0 + 16 * h);
          lim = qj < nq ? lim : 0;
        }
      }
      // VALU work items, spread over the MFMA slots by their cost: the 16
      // elements (P, dS, amax), the scale, four groups of refined
      // quotients, P^F = E2M1(quotient) * scale in two halves (-> tile),
      // the dS rows (-> tile)
      float p[16], ds[16];
      float amax = 0.0f, scv = 0.0f;
      FastP fq(1.0f);
      f32x4 q4[4];
      u32x4 pfw[2];
      auto item = [&](int i) __attribute__((always_inline)) {
        if (i < 16) {
          float x = __builtin_fmaf(sc[i], sl2, -lse2);
          if (MASK) x = i < lim ? x : -INFINITY;
          const float pv = fast_exp2(x);
          ds[i] = pv * dc[i];  // dc holds dP - delta
          p[i] = UNIT_P ? pv : pv * psc;
          amax = fmaxf(amax, p[i]);
        } else if (i == 16) {
          scv = e4m3_scale_from_amax(amax);
          // a zero scale divides by 1 instead (its values are then multiplied by 0)
          fq = FastP(scv > 0.0f ? scv : 1.0f);
        } else if (i < 21) {
          const int g = i - 17;
#pragma unroll
          for (int e = 0; e < 4; ++e) q4[g][e] = fq.quotient(p[4 * g + e]);
        } else if (i < 23) {
          // P^F of elements 8h'..8h'+7 (h' = i - 21): E2M1 rounding of the
          // quotients, times the scale (exact in bf16)
          const int hh = i - 21;
          const uint32_t cw = FastP::codes8(q4[2 * hh], q4[2 * hh + 1]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y0, y1;
            FastP::dequant_codes(cw, e, scv, y0, y1);
            pfw[hh][e] = pack_exact_bf16x2(y0, y1);
          }
          if (hh == 1) {
            write_tile_row(pftile + (R & 1) * 1024, pfw[0], pfw[1]);
          }
        } else {
          u32x4 dsb[2];
#pragma unroll
          for (int e = 0; e < 8; ++e) dsb[e >> 2][e & 3] = pack_bf16x2(ds[2 * e], ds[2 * e + 1]);
          write_tile_row(dstile + (R & 1) * 1024, dsb[0], dsb[1]);
        }
      };
      constexpr int NSLOT = NM > 16 ? NM : 16;
#pragma unroll
      for (int k = 0; k < NSLOT; ++k) {
        if (DO_M && k < NM) {
          if (k + kAhead < NM) b[k + kAhead] = operand(k + kAhead, IntTag<RN>());
          if (k & 1) {
            // the dP^T chain starts from -delta: (-1, -1, -1) x (d1, d2, d3)
            if (k == 1) dn = mfma32x32x16(adl, bdl, zero_f32x16());
            dn = mfma32x32x16(vf[k >> 1], b[k], dn);
          } else {
            sn = mfma32x32x16(kf[k >> 1], b[k], k == 0 ? zero_f32x16() : sn);
          }
        }
        if (DO_V) {
#pragma unroll
          for (int i = 0; i < kXItems; ++i)
            if (x_item_slot(i, NSLOT) == k) item(i);
        }
        if (!(ATTNQAT_DKDV_SGB && DO_M && DO_V)) __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (ATTNQAT_DKDV_SGB && DO_M && DO_V) {
        // one scheduling region for the whole step: the compiler fills the
        // VALU groups between consecutive MFMAs with ready instructions
#pragma unroll
        for (int k = 0; k < NM + 1; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x002, ATTNQAT_DKDV_SGB_VALU, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // prologue: sub-tiles 0 and 1 staged, S^T(0) and dP^T(0)
    if (nsub > 0) issue_sub(0, IntTag<0>());
    if (nsub > 1) issue_sub(1, IntTag<1>());
    vmem_wait_all();  // in-loop waits then only track the loop's own copies
    __syncthreads();
    f32x16 s_even, d_even, s_odd, d_odd;  // S^T / dP^T of even and odd sub-tiles
    if (nsub > 0 && !skipped(0))
      x_step_body(-1, IntTag<kRing - 1>(), BoolTag<true>(), BoolTag<false>(),
                  BoolTag<false>(), s_odd, d_odd, s_even, d_even);

    auto x_step = [&](int j, auto rtag) __attribute__((always_inline)) {
      constexpr int R = decltype(rtag)::value;  // j % kRing
      if (j >= nsteps) return;
      f32x16& sc = (R & 1) ? s_odd : s_even;
      f32x16& dc = (R & 1) ? d_odd : d_even;
      f32x16& sn = (R & 1) ? s_even : s_odd;
      f32x16& dn = (R & 1) ? d_even : d_odd;
      // slot (j+2) % kRing last held sub-tile j-2, last used by Y at step j-1
      const bool stage = j + 2 < nsub;
      if (stage) issue_sub(j + 2, IntTag<(R + 2) % kRing>());
      const bool do_m = j + 1 < nsub && !skipped(j + 1);
      const bool do_v = j < nsub && !skipped(j);
      const int q0 = qstart + kSub * j;
      // masks: keys past nkv, the query tail, the causal diagonal
      const bool mask = keys_tail || q0 + kSub > nq || (CAUSAL && q0 < kw0 + 31);
      if (do_m && do_v) {
        if (mask)
          x_step_body(j, rtag, BoolTag<true>(), BoolTag<true>(), BoolTag<true>(), sc, dc, sn, dn);
        else
          x_step_body(j, rtag, BoolTag<true>(), BoolTag<true>(), BoolTag<false>(), sc, dc, sn,
                      dn);
      } else if (do_m) {
        x_step_body(j, rtag, BoolTag<true>(), BoolTag<false>(), BoolTag<false>(), sc, dc, sn, dn);
      } else if (do_v) {
        if (mask)
          x_step_body(j, rtag, BoolTag<false>(), BoolTag<true>(), BoolTag<true>(), sc, dc, sn,
                      dn);
        else
          x_step_body(j, rtag, BoolTag<false>(), BoolTag<true>(), BoolTag<false>(), sc, dc, sn,
                      dn);
      }
      // sub-tile j+2 has landed (this wave's copies; the barrier covers the others')
      if (stage) vmem_wait<0>();
      __syncthreads();
    };
    for (int j0 = 0; j0 < nsteps; j0 += kRing) {
      x_step(j0, IntTag<0>());
      x_step(j0 + 1, IntTag<1>());
      x_step(j0 + 2, IntTag<2>());
      x_step(j0 + 3, IntTag<3>());
    }
  } else {
    // ---- Y, step j: dK += dS^T Q^(j-1), dV += P^F^T dO(j-1), with dS and
    // P^F from X's tiles of the previous step: MFMAs and LDS reads only
    const ColOffsets<D> co(8 * h, 8 * h + 4, lane);   // column reads (dV, dK B operands)
    // key-column (transpose) reads of the P^F / dS tiles: lane l gets key
    // column 16*(l/16 % 2) + 4*(l%4) .. of query rows 16kb + 8h + (l%16)/4
    // (elements 0..3) and 16kb + 8h + 4 + (l%16)/4 (elements 4..7)
    int tro[2][2];
    {
      const int j = lane & 15;
      const int col = ((lane >> 4) & 1) * 16 + 4 * (j & 3);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        tro[kb][0] = hoff(16 * kb + 8 * h + (j >> 2), col);
        tro[kb][1] = hoff(16 * kb + 8 * h + 4 + (j >> 2), col);
      }
    }
    f32x16 dv[DB], dk[DB];  // lane -> d, VGPR -> key
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dv[db] = zero_f32x16();
      dk[db] = zero_f32x16();
    }
    vmem_wait_all();
    __syncthreads();  // the prologue barrier of the X waves

    auto y_step = [&](int j, auto rtag) __attribute__((always_inline)) {
      constexpr int R = decltype(rtag)::value;     // j % kRing
      constexpr int RP = (R + kRing - 1) % kRing;  // slot of sub-tile j-1
      if (j >= nsteps) return;
      if (j >= 1 && !skipped(j - 1)) {  // j - 1 < nsub holds for j < nsteps
        const uint16_t* dt = dstile + (RP & 1) * 1024;
        const uint16_t* pt = pftile + (RP & 1) * 1024;
        constexpr int NH = 2 * DB;  // MFMAs per product (dK, dV)
        // B operand of MFMA k: the dK product (Q^ columns) for k < NH, then
        // the dV product (dO columns); 16-query k-block (k % NH) / DB, d
        // block k % DB
        auto operand = [&](int k) __attribute__((always_inline)) {
          const uint16_t* tile = ring(RP, k < NH ? 0 : 1);
          const int kk2 = k % NH;
          return lds_operand_cols_at(tile + 16 * (kk2 / DB) * D, co.a[kk2 % DB], co.b[kk2 % DB]);
        };
        const bf16x8 as[2] = {lds_operand_cols_at(dt, tro[0][0], tro[0][1]),
                              lds_operand_cols_at(dt, tro[1][0], tro[1][1])};
        bf16x8 b[2 * NH];
#pragma unroll
        for (int k = 0; k < kAheadY; ++k) b[k] = operand(k);
        bf16x8 ap[2];
#pragma unroll
        for (int k = 0; k < 2 * NH; ++k) {
          if (k + kAheadY < 2 * NH) b[k + kAheadY] = operand(k + kAheadY);
          if (k == NH - kAheadY || (NH <= kAheadY && k == 0)) {
            ap[0] = lds_operand_cols_at(pt, tro[0][0], tro[0][1]);
            ap[1] = lds_operand_cols_at(pt, tro[1][0], tro[1][1]);
          }
          if (k < NH)
            dk[k % DB] = mfma32x32x16(as[k / DB], b[k], dk[k % DB]);
          else
            dv[k % DB] = mfma32x32x16(ap[(k - NH) / DB], b[k], dv[k % DB]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
    };
    for (int j0 = 0; j0 < nsteps; j0 += kRing) {
      y_step(j0, IntTag<0>());
      y_step(j0 + 1, IntTag<1>());
      y_step(j0 + 2, IntTag<2>());
      y_step(j0 + 3, IntTag<3>());
    }

    // accumulators: lane -> d = 32*db + l32, VGPR v -> key kw0 + 8*(v/4) + 4h + v%4
    if (QSPL > 1) {
      // this split's unscaled dK and dV rows (a split without queries stores zeros)
      const size_t tstride = (size_t)a.bh * nkv * D;  // one tensor of the split
      float* PK = a.dkdv_part + 2 * (size_t)blockIdx.y * tstride + (size_t)bh * nkv * D;
      float* PV = PK + tstride;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kw0 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (key < nkv) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            PK[(size_t)key * D + 32 * db + l32] = dk[db][v];
            PV[(size_t)key * D + 32 * db + l32] = dv[db][v];
          }
        }
      }
      return;
    }
    const float vsc = UNIT_P ? 1.0f : 1.0f / a.p_scale;
    const float ksc = a.softmax_scale;
    uint16_t* DV = a.dv + (size_t)bh * nkv * D;
    uint16_t* DK = a.dk + (size_t)bh * nkv * D;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kw0 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (key < nkv) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          DV[(size_t)key * D + 32 * db + l32] = (uint16_t)f32_to_bf16_bits(dv[db][v] * vsc);
          DK[(size_t)key * D + 32 * db + l32] = (uint16_t)f32_to_bf16_bits(dk[db][v] * ksc);
        }
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_d(const AttnArgs& a, hipStream_t stream, const LaunchEvents* ev) {
  // split over queries: fp32 partials, summed by the caller's k_sum_parts launch
  const dim3 block(kThreads);
  const dim3 grid((unsigned)(((a.nkv + kKeys - 1) / kKeys) * a.bh),
                  (unsigned)(a.dkdv_splits > 1 ? a.dkdv_splits : 1));
  if (a.p_scale == 1.0f) return launch(k_dkdv<D, CAUSAL, true>, grid, block, stream, ev, a);
  return launch(k_dkdv<D, CAUSAL, false>, grid, block, stream, ev, a);
}

}  // namespace

hipError_t launch_bwd_dkdv(const AttnArgs& a, int head_dim, hipStream_t stream,
                           const LaunchEvents* ev) {
  if (head_dim == 128)
    return a.causal ? launch_dkdv_d<128, true>(a, stream, ev)
                    : launch_dkdv_d<128, false>(a, stream, ev);
  return a.causal ? launch_dkdv_d<64, true>(a, stream, ev) : launch_dkdv_d<64, false>(a, stream, ev);
}

}  // namespace attnqat
