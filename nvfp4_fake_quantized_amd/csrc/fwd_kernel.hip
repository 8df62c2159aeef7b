// QAT forward on the fake-quantized Q^, K^, V^: O_hp = softmax(s Q^ K^T) V^
// and the natural-log lse ("NVFP4 Attention QAT Backward", §High-level
// wrapper: O_hp is the value saved before probability quantization; the
// Attn-QAT summary, fix 1, gives its reason).
//
// Work decomposition (gfx950, wave64, bf16 MFMA 32x32x16, fp32 accumulate):
//  * a workgroup of 4 waves owns 128 queries; each wave owns 32 queries and
//    keeps its Q^ rows in registers as the B operand of S^T = K^ Q^T;
//  * the key loop stages 32-key tiles of K^ and V^ row-major (XOR-swizzled
//    16-byte chunks) in double-buffered LDS, prefetched one tile ahead
//    through registers; the V^T operand is read with LDS transpose reads;
//  * S^T's accumulator layout puts one query per lane (and 16 of its keys in
//    VGPRs), so the online-softmax row statistics are per lane (plus one
//    exchange with the lane 32 away), and P^T feeds the B operand of
//    O^T = V^T P^T straight from registers;
//  * the running max only triggers a rescale of the accumulator when it
//    moved for some row of the wave (otherwise the factor is exactly 1);
//  * only boundary tiles (the last key tiles: tail, causal diagonal) evaluate
//    masks; the leading tiles run a branch-free loop;
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
constexpr int kFwdBN = ATTNQAT_FWD_BN;  // keys per staged tile (32-key sub-tiles)

// One 32-key tile for one wave (32 queries): online-softmax update of
// (m, l, O^T).  m is the running row max in log2 units.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void fwd_tile(const bf16x8* qf, f32x16* o, float& m, float& l,
                                         const uint16_t* sKb, const uint16_t* sVb,
                                         const RowOffsets<D>& ro, const ColOffsets<D>& co, int k0,
                                         int qi, int nkv, float sl2, int lane) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  const int h = lane >> 5, l32 = lane & 31;
  f32x16 s = zero_f32x16();
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    s = mfma32x32x16(ld_bf16x8(sKb + ro.o[kb]), qf[kb], s);
  float tmax = -INFINITY;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float x = s[v] * sl2;
    if (MASK) {
      const int key = k0 + 8 * (v >> 2) + 4 * h + (v & 3);
      const bool ok = key < nkv && (!CAUSAL || key <= qi);
      x = ok ? x : -INFINITY;
    }
    s[v] = x;
    tmax = fmaxf(tmax, x);
  }
  tmax = fmaxf(tmax, xor32(tmax));
  const float mnew = fmaxf(m, tmax);
  // rescale only when some row's max moved; otherwise alpha would be exactly 1
  if (__any(mnew > m)) {
    const float alpha = fast_exp2(m - (mnew == -INFINITY ? 0.0f : mnew));
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
  }
  m = mnew;
  const float base = (mnew == -INFINITY) ? 0.0f : mnew;
  float pv[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    pv[v] = fast_exp2(s[v] - base);
    l += pv[v];
  }
  // O^T += V^T P^T over two 16-key k-blocks: lane half h, element e of
  // k-block kh holds key 16*kh + 8*(e/4) + 4h + e%4 in both operands.
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const u32x4 bw = {pack_bf16x2(pv[8 * kh], pv[8 * kh + 1]),
                      pack_bf16x2(pv[8 * kh + 2], pv[8 * kh + 3]),
                      pack_bf16x2(pv[8 * kh + 4], pv[8 * kh + 5]),
                      pack_bf16x2(pv[8 * kh + 6], pv[8 * kh + 7])};
    const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      o[db] = mfma32x32x16(lds_operand_cols_at(sVb + 16 * kh * D, co.a[db], co.b[db]), b, o[db]);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ATTNQAT_FWD_WAVES, 8)))
void k_fwd(AttnArgs a) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int BN = kFwdBN;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CH = BN * CPR / 256;  // chunks per thread per tensor per tile
  static_assert(BN % 32 == 0 && CH >= 1, "key tile must be whole 32-key sub-tiles");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * D];  // swizzled rows
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const TileId t = xcd_tile((a.nq + kFwdBM - 1) / kFwdBM);
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
  auto store_tile = [&](int buf) {
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
        fwd_tile<D, CAUSAL, MASK>(qf, o, m, l, kb, vb, ro, co, ks, qi, nkv, sl2, lane);
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

  const float lt = l + xor32(l);
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

}  // namespace

hipError_t launch_fwd(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)(((a.nq + kFwdBM - 1) / kFwdBM) * a.bh));
  if (head_dim == 128) {
    if (a.causal)
      hipLaunchKernelGGL((k_fwd<128, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_fwd<128, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.causal)
      hipLaunchKernelGGL((k_fwd<64, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_fwd<64, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attnqat
