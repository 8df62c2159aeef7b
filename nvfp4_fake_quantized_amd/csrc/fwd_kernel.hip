// QAT forward on the fake-quantized Q^, K^, V^: O_hp = softmax(s Q^ K^T) V^
// and the natural-log lse ("NVFP4 Attention QAT Backward", §High-level
// wrapper: O_hp is the value saved before probability quantization; the
// Attn-QAT summary, fix 1, gives its reason).
//
// Work decomposition (gfx950, wave64, bf16 MFMA 32x32x16, fp32 accumulate):
//  * a workgroup of 4 waves owns 128 queries; each wave owns 32 queries and
//    keeps its Q^ rows in registers as the B operand of S^T = K^ Q^T;
//  * the key loop stages 64-key tiles of K^ (row-major) and V^ (transposed,
//    [d][key]) in LDS;
//  * S^T's accumulator layout puts one query per lane (and 16 of its keys in
//    VGPRs), so the online-softmax row statistics are per lane (plus one
//    exchange with the lane 32 away), and P^T feeds the B operand of
//    O^T = V^T P^T straight from registers;
//  * causal: tiles with every key above the wave's last query are skipped
//    (and the key loop ends at the workgroup's last query); the diagonal
//    tile keeps the elementwise key <= query mask; keys >= Nkv are masked
//    and rows >= Nq are never stored (non-aligned tails).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attnqat {

namespace {

constexpr int kFwdBM = 128;  // queries per workgroup
constexpr int kFwdBN = 64;   // keys per tile

template <int D>
__global__ __launch_bounds__(256) void k_fwd(AttnArgs a) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int BN = kFwdBN;
  constexpr int SK = D + 8;    // row stride of sK (elements)
  constexpr int SVT = BN + 4;  // row stride of sVt
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * SK];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * SVT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y;
  const int nq = a.nq, nkv = a.nkv;
  const int qblk0 = blockIdx.x * kFwdBM;
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
  const int kend = a.causal ? min(nkv, qblk0 + kFwdBM) : nkv;

  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int c = tid; c < BN * D / 8; c += 256) {
      const int r = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = k0 + r;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < nkv) {
        kv = *reinterpret_cast<const u32x4*>(K + (size_t)key * D + col);
        vv = *reinterpret_cast<const u32x4*>(V + (size_t)key * D + col);
      }
      *reinterpret_cast<u32x4*>(&sK[r * SK + col]) = kv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sVt[(col + 2 * e) * SVT + r] = (uint16_t)(vv[e] & 0xFFFFu);
        sVt[(col + 2 * e + 1) * SVT + r] = (uint16_t)(vv[e] >> 16);
      }
    }
    __syncthreads();
    if (a.causal && qw0 + 31 < k0) continue;  // every key of the tile is above this wave's rows

    f32x16 s[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      s[nb] = zero_f32x16();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        s[nb] = mfma32x32x16(ld_bf16x8(&sK[(32 * nb + l32) * SK + 16 * kb + 8 * h]), qf[kb],
                             s[nb]);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = k0 + 32 * nb + 8 * (v >> 2) + 4 * h + (v & 3);
        const bool ok = key < nkv && (!a.causal || key <= qi);
        const float x = ok ? s[nb][v] * sl2 : -INFINITY;
        s[nb][v] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, xor32(tmax));
    const float mnew = fmaxf(m, tmax);
    const float base = (mnew == -INFINITY) ? 0.0f : mnew;
    const float alpha = fast_exp2(m - base);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(s[nb][v] - base);
        s[nb][v] = p;
        l += p;
      }
    }
    // O^T += V^T P^T over four 16-key k-blocks.  Lane half h, element e of a
    // k-block holds key 16*kblk + 8*(e/4) + 4h + e%4 in both operands.
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[nb][8 * kh + e];
        const bf16x8 b = pack_bf16x8(pv);
        const int kb0 = 32 * nb + 16 * kh + 4 * h;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* row = &sVt[(32 * db + l32) * SVT];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(row + kb0);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(row + kb0 + 8);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, av), b, o[db]);
        }
      }
    }
  }

  const float lt = l + xor32(l);
  if (qi < nq) {
    const float inv = 1.0f / lt;
    uint16_t* O = a.o_hp + (size_t)bh * nq * D + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t w0 = f32_to_bf16_bits(o[db][4 * g4] * inv) |
                            (f32_to_bf16_bits(o[db][4 * g4 + 1] * inv) << 16);
        const uint32_t w1 = f32_to_bf16_bits(o[db][4 * g4 + 2] * inv) |
                            (f32_to_bf16_bits(o[db][4 * g4 + 3] * inv) << 16);
        const u32x2 w = {w0, w1};
        *reinterpret_cast<u32x2*>(O + 32 * db + 8 * g4 + 4 * h) = w;
      }
    }
    if (h == 0) a.lse_out[(size_t)bh * nq + qi] = (m + __builtin_log2f(lt)) * kLn2;
  }
}

}  // namespace

hipError_t launch_fwd(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((a.nq + kFwdBM - 1) / kFwdBM, a.bh);
  if (head_dim == 128)
    hipLaunchKernelGGL(k_fwd<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_fwd<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attnqat
