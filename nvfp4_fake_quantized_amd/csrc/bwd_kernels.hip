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
//    feeds the B operand of dQ^T = K^T dS^T from registers; K^ is staged in
//    LDS both row-major (A operand of S^T) and transposed (A of dQ^T).
//  * k_dkdv: each wave owns 32 keys.  Its K^ and V^ rows sit in registers as
//    A operands with the row order permuted so that, in the S^T accumulator,
//    each lane holds one query and 16 *consecutive* keys: exactly one P
//    quantization group.  The group amax, the E4M3 scale and the E2M1
//    rounding are then per-lane work with no cross-lane reduction.  P^F and
//    dS go through a per-wave LDS transpose ([key][query]) to become the A
//    operands of dV = P^F^T dO and dK = dS^T Q^; dO and Q^ are staged in LDS
//    both row-major and transposed ([d][query]).
//  * Causal: tiles entirely above the diagonal are skipped per wave; the
//    diagonal tile keeps the elementwise key <= query mask.  Tails: keys >= Nkv
//    and queries >= Nq get P = 0 (so a short last P group is zero-padded),
//    loads beyond the ends read zeros and stores stop at the ends.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kDqBM = 128;    // queries per workgroup (k_dq)
constexpr int kDqBN = 64;     // keys per tile (k_dq)
constexpr int kDkvBN = 128;   // keys per workgroup (k_dkdv)
constexpr int kDkvBM = 32;    // queries per tile (k_dkdv)

__device__ __forceinline__ u32x4 ld_u32x4(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <int D>
__global__ __launch_bounds__(256) void k_dq(AttnArgs a) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int BN = kDqBN;
  constexpr int SK = D + 8;    // row stride of sK / sV
  constexpr int SKT = BN + 4;  // row stride of sKt
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * SK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BN * SK];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * SKT];

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

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();
  const int kend = a.causal ? min(nkv, qblk0 + kDqBM) : nkv;

  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int c = tid; c < BN * D / 8; c += 256) {
      const int r = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = k0 + r;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < nkv) {
        kv = ld_u32x4(K + (size_t)key * D + col);
        vv = ld_u32x4(V + (size_t)key * D + col);
      }
      *reinterpret_cast<u32x4*>(&sK[r * SK + col]) = kv;
      *reinterpret_cast<u32x4*>(&sV[r * SK + col]) = vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sKt[(col + 2 * e) * SKT + r] = (uint16_t)(kv[e] & 0xFFFFu);
        sKt[(col + 2 * e + 1) * SKT + r] = (uint16_t)(kv[e] >> 16);
      }
    }
    __syncthreads();
    if (a.causal && qw0 + 31 < k0) continue;

    f32x16 s[2], dp[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      s[nb] = zero_f32x16();
      dp[nb] = zero_f32x16();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int off = (32 * nb + l32) * SK + 16 * kb + 8 * h;
        s[nb] = mfma32x32x16(ld_bf16x8(&sK[off]), qf[kb], s[nb]);
        dp[nb] = mfma32x32x16(ld_bf16x8(&sV[off]), df[kb], dp[nb]);
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = k0 + 32 * nb + 8 * (v >> 2) + 4 * h + (v & 3);
        const bool ok = qok && key < nkv && (!a.causal || key <= qi);
        const float p = ok ? fast_exp2(s[nb][v] * sl2 - lse2) : 0.0f;
        s[nb][v] = p * (dp[nb][v] - dl);  // dS
      }
    }
    // dQ^T += K^T dS^T over four 16-key k-blocks (key mapping as in the
    // forward: lane half h, element e -> 16*kblk + 8*(e/4) + 4h + e%4).
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) dsv[e] = s[nb][8 * kh + e];
        const bf16x8 b = pack_bf16x8(dsv);
        const int kb0 = 32 * nb + 16 * kh + 4 * h;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* row = &sKt[(32 * db + l32) * SKT];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(row + kb0);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(row + kb0 + 8);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, av), b, acc[db]);
        }
      }
    }
  }

  if (qok) {
    const float sc = a.softmax_scale;
    uint16_t* out = a.dq + (size_t)bh * nq * D + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t w0 = f32_to_bf16_bits(acc[db][4 * g4] * sc) |
                            (f32_to_bf16_bits(acc[db][4 * g4 + 1] * sc) << 16);
        const uint32_t w1 = f32_to_bf16_bits(acc[db][4 * g4 + 2] * sc) |
                            (f32_to_bf16_bits(acc[db][4 * g4 + 3] * sc) << 16);
        const u32x2 w = {w0, w1};
        *reinterpret_cast<u32x2*>(out + 32 * db + 8 * g4 + 4 * h) = w;
      }
    }
  }
}

// Row r of a wave's 32-key MFMA A operand holds key pi(r) so that the S^T
// accumulator (rows 8*(v/4) + 4h + v%4 in VGPR v of lane half h) holds key
// 16h + v: one contiguous 16-key group per lane.
__device__ __forceinline__ int key_perm(int r) {
  return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

template <int D>
__global__ __launch_bounds__(256) void k_dkdv(AttnArgs a) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int BM = kDkvBM;
  constexpr int SQ = D + 8;    // row stride of sQ / sdO
  constexpr int SQT = BM + 8;  // row stride of sQt / sdOt
  constexpr int SP = BM + 8;   // row stride of the per-wave transpose buffers
  __shared__ __attribute__((aligned(16))) uint16_t sQ[BM * SQ];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[BM * SQ];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[D * SQT];
  __shared__ __attribute__((aligned(16))) uint16_t sdOt[D * SQT];
  __shared__ __attribute__((aligned(16))) uint16_t sPt[4 * 32 * SP];
  __shared__ __attribute__((aligned(16))) uint16_t sSt[4 * 32 * SP];
  __shared__ float sLse[BM];
  __shared__ float sDl[BM];

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
  uint16_t* myPt = &sPt[wave * 32 * SP];
  uint16_t* mySt = &sSt[wave * 32 * SP];
  // queries below the workgroup's first key are fully masked when causal
  const int qstart = a.causal ? (kblk0 / BM) * BM : 0;

  for (int q0 = qstart; q0 < nq; q0 += BM) {
    __syncthreads();
    for (int c = tid; c < BM * D / 8; c += 256) {
      const int r = c / (D / 8), col = (c % (D / 8)) * 8;
      const int qq = q0 + r;
      u32x4 qv = {0u, 0u, 0u, 0u}, dv4 = {0u, 0u, 0u, 0u};
      if (qq < nq) {
        qv = ld_u32x4(Q + (size_t)qq * D + col);
        dv4 = ld_u32x4(dO + (size_t)qq * D + col);
      }
      *reinterpret_cast<u32x4*>(&sQ[r * SQ + col]) = qv;
      *reinterpret_cast<u32x4*>(&sdO[r * SQ + col]) = dv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sQt[(col + 2 * e) * SQT + r] = (uint16_t)(qv[e] & 0xFFFFu);
        sQt[(col + 2 * e + 1) * SQT + r] = (uint16_t)(qv[e] >> 16);
        sdOt[(col + 2 * e) * SQT + r] = (uint16_t)(dv4[e] & 0xFFFFu);
        sdOt[(col + 2 * e + 1) * SQT + r] = (uint16_t)(dv4[e] >> 16);
      }
    }
    if (tid < BM) {
      const int qq = q0 + tid;
      sLse[tid] = qq < nq ? LSE[qq] * kLog2e : 0.0f;
      sDl[tid] = qq < nq ? DL[qq] : 0.0f;
    }
    __syncthreads();
    // every query of the tile is below this wave's first key: fully masked
    const bool active = !(a.causal && q0 + BM - 1 < kw0);
    if (active) {
      f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int off = l32 * SQ + 16 * kb + 8 * h;
        s = mfma32x32x16(kf[kb], ld_bf16x8(&sQ[off]), s);
        dp = mfma32x32x16(vf[kb], ld_bf16x8(&sdO[off]), dp);
      }
      // this lane: query q0 + l32, keys kw0 + 16h + v (v = 0..15)
      const int qj = q0 + l32;
      const float lse2 = sLse[l32];
      const float dl = sDl[l32];
      float pq[16];
      float amax = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kw0 + 16 * h + v;
        const bool ok = qj < nq && key < nkv && (!a.causal || key <= qj);
        const float p = ok ? fast_exp2(s[v] * sl2 - lse2) : 0.0f;
        s[v] = p * (dp[v] - dl);  // dS
        pq[v] = p * psc;
        amax = fmaxf(amax, pq[v]);
      }
      const float sc = e4m3_scale_from_amax(amax);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kr = (16 * h + v) * SP + l32;
        myPt[kr] = (uint16_t)f32_to_bf16_bits(e2m1_dequant(pq[v], sc));
        mySt[kr] = (uint16_t)f32_to_bf16_bits(s[v]);
      }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int kq = 0; kq < BM / 16; ++kq) {
        const bf16x8 ap = ld_bf16x8(&myPt[l32 * SP + 16 * kq + 8 * h]);
        const bf16x8 as = ld_bf16x8(&mySt[l32 * SP + 16 * kq + 8 * h]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = (32 * db + l32) * SQT + 16 * kq + 8 * h;
          dv[db] = mfma32x32x16(ap, ld_bf16x8(&sdOt[off]), dv[db]);
          dk[db] = mfma32x32x16(as, ld_bf16x8(&sQt[off]), dk[db]);
        }
      }
    }
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
  if (head_dim == 128)
    hipLaunchKernelGGL(k_dq<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_dq<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((a.nkv + kDkvBN - 1) / kDkvBN, a.bh);
  if (head_dim == 128)
    hipLaunchKernelGGL(k_dkdv<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_dkdv<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attnqat
