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
// SIMD (waves w and w+4).  The two waves of a pair split the work on their 32
// keys by role, so that each issues the same number of MFMAs and a similar
// VALU load (a lone wave issues VALU at only half of a SIMD's rate):
//  * wave X (w < 4) keeps the pair's K^ rows and the dV accumulator.  Per
//    32-query sub-tile j it computes S^T = K^ Q^T, P = exp2(S * s log2e -
//    lse log2e), the group amax, the E4M3 scale and the refined quotients
//    q = P / scale (q = P when the scale is 0), and hands q and the scale to
//    Y through LDS.  Two steps later it reads P^F(j) back (from Y) and adds
//    P^F^T dO to dV.
//  * wave Y (w >= 4) keeps the V^ rows and the dK accumulator.  It computes
//    dP^T = V^ dO^T for sub-tile j, and one step later (with q and the scale
//    of sub-tile j) P ~ q * scale, dS = P (dP - delta), the E2M1 rounding of
//    q (P^F = code * scale), writes P^F for X, and adds dS^T Q^ to dK.
// One barrier per sub-tile orders the handovers.  P^F is exact: the E2M1
// code comes from the FMA-refined quotient, which rounds like the exact
// quotient (precise division).  P ~ q * scale differs from P by about one
// fp32 ulp and only enters dS, which is rounded to bf16 for its MFMA.
//
// In the S^T accumulator each lane holds one query and, because the K^/V^
// rows are loaded in the permuted order pi, 16 *consecutive* keys: exactly
// one P quantization group, so the amax and the scale are per-lane work.
// The Q^/dO sub-tiles (32 queries) sit in a ring of four LDS slots
// (XOR-swizzled rows; row reads for S/dP, transpose reads for dK/dV),
// prefetched one step ahead through registers.  The step loops are unrolled
// by the ring period, so every LDS address is a lane register plus an
// immediate.  P^F and dS reach the A operands of dV and dK through per-pair
// [query][key] LDS tiles read back with transpose reads.
//
// Masks: only sub-tiles on a boundary (causal diagonal, query tail, keys past
// nkv) evaluate them, in X (P = 0, hence q = 0, dS = 0 and P^F = 0); causal
// sub-tiles entirely above the diagonal are skipped by both waves.  Loads
// beyond the ends read zeros and stores stop at the ends.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kKeys = 128;     // keys per workgroup
constexpr int kSub = 32;       // queries per sub-tile
constexpr int kThreads = 512;  // 4 X waves + 4 Y waves
constexpr int kRing = 4;       // Q^/dO sub-tile slots (also the unroll factor)

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
  static constexpr int QB = 0;                       // q[pair][2][4 KB], [g][lane][4] floats
  static constexpr int PF = QB + 4 * 2 * 4096;       // P^F[pair][2] 32x32 bf16 tiles
  static constexpr int DS = PF + 4 * 2 * 2048;       // dS[pair] 32x32 bf16 tiles
  static constexpr int SB = DS + 4 * 2048;           // scale[pair][2][64] floats
  static constexpr int LSE = SB + 4 * 2 * 256;       // lse[kRing][32] (raw)
  static constexpr int DL = LSE + kRing * kSub * 4;  // delta[kRing][32]
  static constexpr int TOTAL = PAIR + DL + kRing * kSub * 4;
};

// Row r of a wave's 32-row K^/V^ operand holds key pi(r): the S^T
// accumulator row 8*(v/4) + 4h + v%4 of lane half h is then key 16h + v.
__device__ __forceinline__ int key_perm(int r) {
  return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

template <int D, bool CAUSAL, bool UNIT_P>
__global__ __launch_bounds__(kThreads) void k_dkdv(AttnArgs a) {
  using L = DkdvLds<D>;
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int NCH = kSub * CPR;         // chunks per tensor per sub-tile
  constexpr int CH = 2 * NCH / kThreads;  // chunks per thread per sub-tile
  static_assert(CH >= 1 && (2 * NCH) % kThreads == 0 && NCH % 64 == 0,
                "sub-tile staging shape");
  static_assert(2 * kRing * L::SUBT <= 65536, "ring offsets fit LDS immediates");
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::TOTAL];

  const int tid = threadIdx.x;
  // wave index in a scalar register: role and key-block branches are uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const bool is_x = wave < 4;  // role
  const int kk = wave & 3;     // the pair's 32-key block
  const int bh = blockIdx.y;
  const int nq = a.nq, nkv = a.nkv;
  const int kblk0 = blockIdx.x * kKeys;
  const int kw0 = kblk0 + 32 * kk;
  const uint16_t* Q = a.q_hat + (size_t)bh * nq * D;
  const uint16_t* dO = a.d_o + (size_t)bh * nq * D;
  const float* LSE = a.lse + (size_t)bh * nq;
  const float* DL = a.delta + (size_t)bh * nq;

  // X: K^ rows, Y: V^ rows of the pair's keys, in the order pi (A operands)
  bf16x8 frag[KB];
  {
    const uint16_t* src = (is_x ? a.k_hat : a.v_hat) + ((size_t)bh * nkv + kblk0) * D;
    const auto rs = make_rsrc(src, (uint32_t)(min(nkv - kblk0, kKeys) * D) * 2u);
    const int row = 32 * kk + key_perm(l32);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      frag[kb] =
          __builtin_bit_cast(bf16x8, buf_ld16(rs, (uint32_t)(row * D + 16 * kb + 8 * h) * 2u));
  }

  // sub-tiles: queries below the workgroup's first key are masked (causal)
  const int qfirst = CAUSAL ? kblk0 : 0;
  const int nsub = qfirst < nq ? (nq - qfirst + kSub - 1) / kSub : 0;
  const int nsteps = nsub > 0 ? nsub + 2 : 0;
  // a sub-tile entirely above the pair's keys (causal) is skipped by both waves
  auto skipped = [&](int j) __attribute__((always_inline)) {
    return CAUSAL && qfirst + kSub * j + kSub - 1 < kw0;
  };
  const bool keys_tail = kw0 + 32 > nkv;

  // ---- staging of sub-tile j (Q^ and dO rows, lse, delta) into slot j % kRing
  u32x4 rst[CH];
  float rl = 0.0f;
  // this thread's chunk c: tensor (uniform per wave) and swizzled LDS offset
  uint32_t goff[CH];
  int loff[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = tid + kThreads * c;
    const int ch = idx % NCH;
    goff[c] = (uint32_t)((ch / CPR) * D + (ch % CPR) * 8) * 2u;
    loff[c] = 2 * swz<D>(ch / CPR, (ch % CPR) * 8);
  }
  auto load_sub = [&](int j) __attribute__((always_inline)) {
    const int q0 = qfirst + kSub * j;
    const int rows = min(nq - q0, kSub);
    const uint32_t bytes = (uint32_t)(rows * D) * 2u;  // rows past nq read as zeros
    const auto rsq = make_rsrc(Q + (size_t)q0 * D, bytes);
    const auto rsd = make_rsrc(dO + (size_t)q0 * D, bytes);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool is_q = 64 * wave + kThreads * c < NCH;
      rst[c] = buf_ld16(is_q ? rsq : rsd, goff[c]);
    }
    // wave 0 stages lse, wave 1 delta (lanes past the sub-tile read zeros)
    if (wave < 2)
      rl = buf_ldf(make_rsrc((wave == 0 ? LSE : DL) + q0, (uint32_t)rows * 4u),
                   (uint32_t)lane * 4u);
  };
  auto store_sub = [&](auto rtag) __attribute__((always_inline)) {
    constexpr int S = decltype(rtag)::value;  // ring slot
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool is_q = 64 * wave + kThreads * c < NCH;
      *reinterpret_cast<u32x4*>(smem + L::RING + (2 * S + (is_q ? 0 : 1)) * L::SUBT + loff[c]) =
          rst[c];
    }
    if (wave < 2 && lane < kSub)
      reinterpret_cast<float*>(smem + L::PAIR + (wave == 0 ? L::LSE : L::DL))[S * kSub + lane] =
          rl;
  };

  const float sl2 = a.softmax_scale * kLog2e;
  const float psc = a.p_scale;
  const RowOffsets<D> ro(lane);                     // row reads (S, dP B operands)
  const ColOffsets<D> co(8 * h, 8 * h + 4, lane);   // column reads (dV, dK B operands)
  const ColOffsets<32> cp(8 * h, 8 * h + 4, lane);  // key-column reads of P^F / dS tiles
  const int pw0 = swz<32>(l32, 16 * h), pw1 = swz<32>(l32, 16 * h + 8);
  uint8_t* const pair = smem + L::PAIR;
  float* const qbuf = reinterpret_cast<float*>(pair + L::QB + kk * 2 * 4096);
  float* const sbuf = reinterpret_cast<float*>(pair + L::SB + kk * 2 * 256);
  uint16_t* const pftile = reinterpret_cast<uint16_t*>(pair + L::PF + kk * 2 * 2048);
  uint16_t* const dstile = reinterpret_cast<uint16_t*>(pair + L::DS + kk * 2048);
  const float* const slse = reinterpret_cast<const float*>(pair + L::LSE);
  const float* const sdl = reinterpret_cast<const float*>(pair + L::DL);
  auto ring = [&](int slot, int tensor) __attribute__((always_inline)) {
    return reinterpret_cast<const uint16_t*>(smem + L::RING + (2 * slot + tensor) * L::SUBT);
  };

  f32x16 acc[DB];  // X: dV, Y: dK (lane -> d, VGPR -> key)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();

  if (nsub > 0) {
    load_sub(0);
    store_sub(IntTag<0>());
  }
  // the K^/V^ fragments have arrived: waits inside the step loops then only
  // track the loops' own prefetches
  vmem_wait_all();
  __syncthreads();

  // The stage prefetch and the barrier of a step are common to both roles.
  auto step_common_begin = [&](int j) __attribute__((always_inline)) {
    if (j + 1 < nsub) load_sub(j + 1);
  };
  auto step_common_end = [&](int j, auto rtag) __attribute__((always_inline)) {
    constexpr int R = decltype(rtag)::value;
    // slot (j+1) % kRing last held sub-tile j-3, whose last use (X, step
    // j-1) is behind the previous barrier
    if (j + 1 < nsub) store_sub(IntTag<(R + 1) % kRing>());
    __syncthreads();
  };

  if (is_x) {
    // ---- X, step j: S^T(j) -> P -> q(j), scale(j); dV += P^F(j-2)^T dO(j-2)
    auto x_valu = [&](int j, const f32x16& s, auto rtag, auto mask_tag)
        __attribute__((always_inline)) {
      constexpr int R = decltype(rtag)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      // this lane: query qj, keys kw0 + 16h + v; under MASK key v is valid
      // when v < lim (below nkv, not above the query, query below nq)
      const float lse2 = slse[R * kSub + l32] * kLog2e;
      int lim = 16;
      if (MASK) {
        const int qj = qfirst + kSub * j + l32;
        lim = (CAUSAL ? min(nkv, qj + 1) : nkv) - (kw0 + 16 * h);
        lim = qj < nq ? lim : 0;
      }
      float p[16];
      float amax = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = __builtin_fmaf(s[v], sl2, -lse2);
        if (MASK) x = v < lim ? x : -INFINITY;
        p[v] = UNIT_P ? fast_exp2(x) : fast_exp2(x) * psc;
        amax = fmaxf(amax, p[v]);
      }
      // a zero scale (every P of the group underflows) divides by 1 instead:
      // the handed-over value is then P itself, which Y still needs for dS
      const float sc = e4m3_scale_from_amax(amax);
      const FastP fq(sc > 0.0f ? sc : 1.0f);
      float* qd = qbuf + (R & 1) * 1024;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 w = {fq.quotient(p[4 * g]), fq.quotient(p[4 * g + 1]),
                         fq.quotient(p[4 * g + 2]), fq.quotient(p[4 * g + 3])};
        *reinterpret_cast<f32x4*>(qd + (g * 64 + lane) * 4) = w;
      }
      sbuf[(R & 1) * 64 + lane] = sc;
    };
    auto x_step = [&](int j, auto rtag) __attribute__((always_inline)) {
      constexpr int R = decltype(rtag)::value;
      if (j >= nsteps) return;
      step_common_begin(j);
      const bool do_s = j < nsub && !skipped(j);
      const bool do_v = j >= 2 && !skipped(j - 2);
      f32x16 s;
      if (do_s) {
        const uint16_t* sQ = ring(R, 0);
        s = mfma32x32x16(frag[0], ld_bf16x8(sQ + ro.o[0]), zero_f32x16());
#pragma unroll
        for (int kb = 1; kb < KB; ++kb) s = mfma32x32x16(frag[kb], ld_bf16x8(sQ + ro.o[kb]), s);
      }
      if (do_v) {
        // P^F(j-2) was written by Y at step j-1 into tile (j-2) & 1 = R & 1
        const uint16_t* pt = pftile + (R & 1) * 1024;
        const uint16_t* sDO = ring((R + 2) % kRing, 1);
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const bf16x8 ap = lds_operand_cols_at(pt + 16 * kq * 32, cp.a[0], cp.b[0]);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mfma32x32x16(
                ap, lds_operand_cols_at(sDO + 16 * kq * D, co.a[db], co.b[db]), acc[db]);
        }
      }
      if (do_s) {
        const int q0 = qfirst + kSub * j;
        // masks: keys past nkv, the query tail, the causal diagonal
        if (keys_tail || q0 + kSub > nq || (CAUSAL && q0 < kw0 + 31))
          x_valu(j, s, rtag, BoolTag<true>());
        else
          x_valu(j, s, rtag, BoolTag<false>());
      }
      step_common_end(j, rtag);
    };
    for (int j0 = 0; j0 < nsteps; j0 += kRing) {
      x_step(j0, IntTag<0>());
      x_step(j0 + 1, IntTag<1>());
      x_step(j0 + 2, IntTag<2>());
      x_step(j0 + 3, IntTag<3>());
    }
  } else {
    // ---- Y, step j: dS(j-1), P^F(j-1) -> LDS, dK += dS(j-1)^T Q^(j-1); dP^T(j)
    f32x16 dp = zero_f32x16();  // dP^T of the sub-tile handled next step
    auto y_step = [&](int j, auto rtag) __attribute__((always_inline)) {
      constexpr int R = decltype(rtag)::value;
      constexpr int RP = (R + kRing - 1) % kRing;  // slot of sub-tile j-1
      if (j >= nsteps) return;
      step_common_begin(j);
      const bool do_k = j >= 1 && j - 1 < nsub && !skipped(j - 1);
      const bool do_p = j < nsub && !skipped(j);
      if (do_k) {
        const float* qs = qbuf + (RP & 1) * 1024;
        const float sc = sbuf[(RP & 1) * 64 + lane];
        // P = q * divisor / p_scale (the divisor is 1 for a zero scale);
        // P^F = code * scale is then 0 for a zero scale
        const float sdiv = sc > 0.0f ? sc : 1.0f;
        const float sp = UNIT_P ? sdiv : sdiv / psc;
        const float dl = sdl[RP * kSub + l32];
        u32x4 pf[2], dsb[2];
        f32x4 q4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          q4[g] = *reinterpret_cast<const f32x4*>(qs + (g * 64 + lane) * 4);
        // E2M1 codes of the 16 quotients, 8 to a dword
        const uint32_t codes[2] = {FastP::codes8(q4[0], q4[1]), FastP::codes8(q4[2], q4[3])};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float y[4], d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) d[e] = q4[g][e] * sp * (dp[4 * g + e] - dl);
          FastP::dequant_codes(codes[g >> 1], 2 * (g & 1), sc, y[0], y[1]);
          FastP::dequant_codes(codes[g >> 1], 2 * (g & 1) + 1, sc, y[2], y[3]);
          pf[g >> 1][2 * (g & 1)] = pack_bf16x2(y[0], y[1]);
          pf[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(y[2], y[3]);
          dsb[g >> 1][2 * (g & 1)] = pack_bf16x2(d[0], d[1]);
          dsb[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(d[2], d[3]);
        }
        uint16_t* pt = pftile + (RP & 1) * 1024;
        *reinterpret_cast<u32x4*>(pt + pw0) = pf[0];
        *reinterpret_cast<u32x4*>(pt + pw1) = pf[1];
        *reinterpret_cast<u32x4*>(dstile + pw0) = dsb[0];
        *reinterpret_cast<u32x4*>(dstile + pw1) = dsb[1];
        wave_lds_fence();
        const uint16_t* sQ = ring(RP, 0);
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const bf16x8 as = lds_operand_cols_at(dstile + 16 * kq * 32, cp.a[0], cp.b[0]);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mfma32x32x16(
                as, lds_operand_cols_at(sQ + 16 * kq * D, co.a[db], co.b[db]), acc[db]);
        }
        wave_lds_fence();
      }
      if (do_p) {
        const uint16_t* sDO = ring(R, 1);
        dp = mfma32x32x16(frag[0], ld_bf16x8(sDO + ro.o[0]), zero_f32x16());
#pragma unroll
        for (int kb = 1; kb < KB; ++kb) dp = mfma32x32x16(frag[kb], ld_bf16x8(sDO + ro.o[kb]), dp);
      }
      step_common_end(j, rtag);
    };
    for (int j0 = 0; j0 < nsteps; j0 += kRing) {
      y_step(j0, IntTag<0>());
      y_step(j0 + 1, IntTag<1>());
      y_step(j0 + 2, IntTag<2>());
      y_step(j0 + 3, IntTag<3>());
    }
  }

  // accumulators: lane -> d = 32*db + l32, VGPR v -> key kw0 + 8*(v/4) + 4h + v%4
  const float osc = is_x ? (UNIT_P ? 1.0f : 1.0f / psc) : a.softmax_scale;
  uint16_t* OUT = (is_x ? a.dv : a.dk) + (size_t)bh * nkv * D;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = kw0 + 8 * (v >> 2) + 4 * h + (v & 3);
    if (key < nkv) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        OUT[(size_t)key * D + 32 * db + l32] = (uint16_t)f32_to_bf16_bits(acc[db][v] * osc);
    }
  }
}

template <int D, bool CAUSAL>
void launch_dkdv_d(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((a.nkv + kKeys - 1) / kKeys, a.bh);
  if (a.p_scale == 1.0f)
    hipLaunchKernelGGL((k_dkdv<D, CAUSAL, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((k_dkdv<D, CAUSAL, false>), grid, dim3(kThreads), 0, stream, a);
}

}  // namespace

hipError_t launch_bwd_dkdv(const AttnArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 128) {
    if (a.causal)
      launch_dkdv_d<128, true>(a, stream);
    else
      launch_dkdv_d<128, false>(a, stream);
  } else {
    if (a.causal)
      launch_dkdv_d<64, true>(a, stream);
    else
      launch_dkdv_d<64, false>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace attnqat
