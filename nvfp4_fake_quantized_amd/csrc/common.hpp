// Device-side building blocks shared by the attnqat kernels (gfx950 / CDNA4).
//
// NVFP4 fake quantization follows "NVFP4 Attention QAT Backward" (cuDNN
// frontend docs), §Overview: one E4M3FN scale per 16 values, s = RNE(amax/6)
// saturating at 448, E2M1 codes c = RNE(|x|/s) with precise division (exact
// midpoints round to even), x^ = sign(x) * c * s.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace attnqat {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Build-time knobs (defaults are the tuned values): waves per SIMD that the
// register allocation of the forward and dQ kernels targets (the dK/dV
// kernel's 512-thread workgroup fixes its own: two waves per SIMD).
#ifndef ATTNQAT_FWD_WAVES
#define ATTNQAT_FWD_WAVES 2
#endif
#ifndef ATTNQAT_DQ_WAVES
#define ATTNQAT_DQ_WAVES 2
#endif
// Steps by which the dK/dV pipeline reads its LDS MFMA operands ahead.
#ifndef ATTNQAT_DKDV_PREFETCH
#define ATTNQAT_DKDV_PREFETCH 2
#endif

constexpr float kLog2e = 1.4426950408889634f;

#ifndef ATTNQAT_XCD_GROUP
#define ATTNQAT_XCD_GROUP 1
#endif
constexpr int kNumXcd = 8;  // XCDs of an MI355X

// Tile of a 1-D launch over (tiles per head) x (batch*heads). The dispatcher
// deals workgroup ids out to the XCDs round-robin, so ids are renumbered to
// give every XCD a contiguous run of logical ids, i.e. whole heads: the K/V
// (or Q/dO) tiles that the workgroups of one head stream then hit that XCD's
// own L2 instead of eight L2s each holding every head.
struct TileId {
  int tile, bh;
};
// last_first: hand out each head's tiles from the last one down (causal
// query tiles: the last one has the most keys, so the heavy work starts
// first and the light tiles fill the tail).
__device__ __forceinline__ TileId xcd_tile(int tiles_per_head, bool last_first = false) {
  const int w = blockIdx.x;
  int l = w;
  if (ATTNQAT_XCD_GROUP) {
    const int total = gridDim.x;
    const int per = total / kNumXcd, rem = total % kNumXcd;
    const int x = w % kNumXcd, slot = w / kNumXcd;
    l = x < rem ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
  }
  const int tile = l % tiles_per_head;
  return {last_first ? tiles_per_head - 1 - tile : tile, l / tiles_per_head};
}

// Compile-time boolean carried through generic lambdas.
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Compile-time integer carried through generic lambdas, and a loop whose
// body sees its index as one (f(IntTag<0>()), ..., f(IntTag<N-1>())).
template <int N>
struct IntTag {
  static constexpr int value = N;
};
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(IntTag<I>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// NVFP4 scalar math (bit-exact).

// E4M3FN block scale of a group with max magnitude `amax` (finite, >= 0):
// the E4M3FN value nearest to amax/6, ties to the even mantissa, saturating
// at 448.  y approximates amax/6 by a product with the fp32 reciprocal of 6
// and one FMA residual correction; rounding y to E4M3 gives the exact
// rounding of amax/6 for every finite non-negative fp32 amax (checked
// exhaustively over all such values against exact comparisons with 6 times
// the E4M3 midpoints).  The plain product alone does not.
__device__ __forceinline__ float e4m3_quotient(float amax) {
  constexpr float kSixth = 1.0f / 6.0f;
  const float y0 = amax * kSixth;
  return __builtin_fmaf(__builtin_fmaf(-y0, 6.0f, amax), kSixth, y0);
}

// The E4M3FN byte (e << 3 | m, bias 7) nearest to y >= 0, ties to even,
// saturating at 448: the gfx950 FP8 conversion rounds to nearest even on
// the OCP E4M3FN grid (subnormals included) and yields NaN above 464, hence
// the clamp.
__device__ __forceinline__ uint32_t e4m3_rne_byte(float y) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(y, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// The value of an E4M3FN byte (no NaN codes are produced above).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

__device__ __forceinline__ float e4m3_scale_from_amax(float amax) {
  return e4m3_value(e4m3_rne_byte(e4m3_quotient(amax)));
}

// The E4M3FN byte of a scale produced above (an exact conversion).
__device__ __forceinline__ uint32_t e4m3_byte(float s) { return e4m3_rne_byte(s); }

// Dequantized E2M1 value c * s (with the sign of x) for c = RNE(|x| / s).
// Comparing |x| with the exact products m * s of the E2M1 midpoints m is the
// same decision as rounding the exact quotient |x| / s: every m * s has at
// most 7 significant bits and is exact in fp32.  At a tie the comparison
// direction picks the even code: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1,
// 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4.  Above 5*s the code saturates at 6.
// s == 0 yields a signed zero (c * 0).
__device__ __forceinline__ float e2m1_dequant(float x, float s) {
  const float a = fabsf(x);
  float c = (a > 0.25f * s) ? 0.5f : 0.0f;
  c += (a >= 0.75f * s) ? 0.5f : 0.0f;
  c += (a > 1.25f * s) ? 0.5f : 0.0f;
  c += (a >= 1.75f * s) ? 0.5f : 0.0f;
  c += (a > 2.5f * s) ? 1.0f : 0.0f;
  c += (a >= 3.5f * s) ? 1.0f : 0.0f;
  c += (a > 5.0f * s) ? 2.0f : 0.0f;
  return __builtin_copysignf(c * s, x);
}

// The 4-bit E2M1 code of the same rounding (bit 3: the sign of x, bits 0-2:
// the magnitude index into 0, 0.5, 1, 1.5, 2, 3, 4, 6; the layout of the
// gfx950 FP4 conversions).  s == 0 yields a signed zero code.
__device__ __forceinline__ uint32_t e2m1_code(float x, float s) {
  const float a = fabsf(x);
  uint32_t k = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) +
               (a > 2.5f * s) + (a >= 3.5f * s) + (a > 5.0f * s);
  k = s > 0.0f ? k : 0u;
  return k | ((__float_as_uint(x) >> 31) << 3);
}

// 16 bf16 values (two 16-byte words) as floats, and back (values exact in
// bf16, so the low halves are dropped exactly).
__device__ __forceinline__ void unpack_bf16x16(u32x4 lo, u32x4 hi, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(lo[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(lo[i] >> 16);
    x[8 + 2 * i] = bf16_bits_to_f32(hi[i] & 0xFFFFu);
    x[8 + 2 * i + 1] = bf16_bits_to_f32(hi[i] >> 16);
  }
}

__device__ __forceinline__ void pack_bf16x16(const float* x, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // values are exact in bf16: truncation of the low half is exact
    lo[i] = (__float_as_uint(x[2 * i]) >> 16) | (__float_as_uint(x[2 * i + 1]) & 0xFFFF0000u);
    hi[i] = (__float_as_uint(x[8 + 2 * i]) >> 16) |
            (__float_as_uint(x[8 + 2 * i + 1]) & 0xFFFF0000u);
  }
}

// Quantizes 16 floats in place; returns the scale.
__device__ __forceinline__ float fq16(float* x) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float s = e4m3_scale_from_amax(amax);
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = e2m1_dequant(x[i], s);
  return s;
}

// Faster exact path for non-negative fp32 values (the probabilities P), used
// where the scale is shared by the 16 values one lane holds:
//   q  = |x|/s from a two-term reciprocal: r_hi = rcp(s) and
//        r_lo = (1 - r_hi*s) * r_hi (one FMA residual step), then
//        q = fma(x, r_hi, x * r_lo), which is x/s within a relative 2^-46
//        before its final rounding,
//   c  = RNE_E2M1(q) by the hardware FP4 conversion (scale 1: no scaling;
//        ties to even, saturating at 6), converted back to fp32,
//   x^ = c * s.
// An exact tie x = m*s (m an E2M1 midpoint) yields q = m exactly and the
// conversion rounds it to even; otherwise x/s lies more than 1.06 half-ulps
// of m away from m (x and m*s are distinct fp32 values and m*s has at most
// 7 significant bits), so q falls on the same side of m as x/s.  Hence c is
// the code of the exact quotient for every fp32 x >= 0 (checked
// exhaustively on the CPU for every fp32 x in [0.125 s, 8 s) and every E4M3
// mantissa of s, with rcp within 1 ulp; below 0.125 s both give 0).  s == 0
// uses rcp 0 and yields 0.
struct FastP {
  float s, r, rl;
  __device__ __forceinline__ explicit FastP(float scale)
      : s(scale), r(scale > 0.0f ? __builtin_amdgcn_rcpf(scale) : 0.0f) {
    rl = __builtin_fmaf(-r, scale, 1.0f) * r;
  }
  // x / s for x >= 0 (see above)
  __device__ __forceinline__ float quotient(float x) const {
    return __builtin_fmaf(x, r, x * rl);
  }
  // E2M1-rounded quotients q0, q1 times the scale s
  __device__ __forceinline__ static void dequant_pair(float q0, float q1, float s, float& y0,
                                                      float& y1) {
    const uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q0, q1, 1.0f, 0);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 0);
    y0 = c[0] * s;
    y1 = c[1] * s;
  }
  // E2M1 codes (RNE, saturating) of 8 quotients, packed 4 bits each: byte b
  // holds the codes of elements 2b and 2b+1
  __device__ __forceinline__ static uint32_t codes8(f32x4 lo, f32x4 hi) {
    uint32_t p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, lo[0], lo[1], 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, lo[2], lo[3], 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, hi[0], hi[1], 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, hi[2], hi[3], 1.0f, 3);
  }
  // values of the two codes in byte `sel` of `codes`, times the scale s
  __device__ __forceinline__ static void dequant_codes(uint32_t codes, int sel, float s,
                                                       float& y0, float& y1) {
    f32x2 c;
    switch (sel) {  // the byte select is an instruction immediate
      case 0: c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0); break;
      case 1: c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1); break;
      case 2: c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2); break;
      default: c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3); break;
    }
    y0 = c[0] * s;
    y1 = c[1] * s;
  }
  // quantize-dequantize a pair (x0, x1 >= 0)
  __device__ __forceinline__ void pair(float x0, float x1, float& y0, float& y1) const {
    dequant_pair(quotient(x0), quotient(x1), s, y0, y1);
  }
};

// fake_nvfp4 of the 8 values a lane holds of a 16-value group whose other 8
// the lane XOR positions away holds: one exchange of the amax, the codec's
// E4M3 scale, and the exact E2M1 rounding of FastP applied to |x| (the sign
// copied back; code * scale is exact in bf16).  Returns the quantized values;
// sb receives the scale byte.
template <int XOR>
__device__ __forceinline__ bf16x8 fq_half_group(bf16x8 v, uint32_t& sb) {
  const u32x4 w = __builtin_bit_cast(u32x4, v);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
  am = fmaxf(am, __shfl_xor(am, XOR, 64));
  const float s = e4m3_scale_from_amax(am);
  const FastP fq(s);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y0, y1;
    fq.pair(fabsf(x[2 * i]), fabsf(x[2 * i + 1]), y0, y1);
    o[i] = __builtin_amdgcn_perm(__float_as_uint(__builtin_copysignf(y1, x[2 * i + 1])),
                                 __float_as_uint(__builtin_copysignf(y0, x[2 * i])),
                                 0x07060302u);
  }
  sb = e4m3_byte(s);
  return __builtin_bit_cast(bf16x8, o);
}

// ---------------------------------------------------------------------------
// LDS transpose reads (ds_read_b64_tr_b16).
//
// Within each group of 16 lanes, source lane j supplies the address of 4
// consecutive 16-bit elements; result lane i receives element (i % 4) of
// source lanes 4e + i/4 for e = 0..3.  When source lane j points at row
// r0 + j/4, columns c0 + 4*(j%4) .. +3 of a row-major tile, lane i receives
// column c0 + i of rows r0 .. r0+3: a column read.
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles.
//
// Tiles of bf16 rows of W elements are stored unpadded; the 16-byte chunk c
// of row r sits at chunk position c ^ f(r).  The two access patterns of the
// kernels are (a) 16-byte row reads by 32 lanes over 32 consecutive rows and
// (b) transpose reads of 4 consecutive rows by each 16-lane group.  On
// gfx950's 64-bank LDS, f below makes both conflict-free (measured with all
// waves of a CU streaming one pattern: both reach 170-230 B per CU per clock,
// against 60-70 for transpose reads of an unswizzled tile; splitting a
// 16-byte row read into two 8-byte reads drops it to 120-135):
//   W = 128: f(r) = ((r >> 2) & 3) ^ ((r & 3) << 2)
//   W = 64:  f(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
//   W = 32:  f(r) = (r >> 2) & 3
template <int W>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  if constexpr (W == 128) return c ^ (((r >> 2) & 3) ^ ((r & 3) << 2));
  else if constexpr (W == 64) return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  else return c ^ ((r >> 2) & 3);
}

// Element offset of (row r, column col) in a swizzled tile of width W.
template <int W>
__device__ __forceinline__ int swz(int r, int col) {
  return r * W + 8 * swz_chunk<W>(r, col >> 3) + (col & 7);
}

// A 32x32x16 MFMA operand whose lanes index columns of a swizzled tile:
// lane l gets column col0 + l%32 of rows r0 + 0..3 (elements 0..3) and
// r1 + 0..3 (elements 4..7), where r0, r1 may depend on h = l/32.
template <int W>
__device__ __forceinline__ bf16x8 lds_operand_cols(const uint16_t* tile, int col0, int r0, int r1,
                                                   int lane) {
  const int j = lane & 15;
  const int col = col0 + ((lane >> 4) & 1) * 16 + 4 * (j & 3);
  const u32x2 lo = lds_read_tr16(tile + swz<W>(r0 + (j >> 2), col));
  const u32x2 hi = lds_read_tr16(tile + swz<W>(r1 + (j >> 2), col));
  const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// The same read from two precomputed per-lane element offsets (see
// ColOffsets); `tile` may carry compile-time row offsets.
__device__ __forceinline__ bf16x8 lds_operand_cols_at(const uint16_t* tile, int off0, int off1) {
  const u32x2 lo = lds_read_tr16(tile + off0);
  const u32x2 hi = lds_read_tr16(tile + off1);
  const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// Per-lane offsets of the column reads of lds_operand_cols<W> for the
// column blocks col0 = 32*db and first rows r0 = RA(h), r1 = RB(h).  The
// swizzle phase of a row depends only on bits of the row index that a
// k-block shift by a multiple of 16 rows does not change, so the offsets for
// k-block kb are these plus 16*kb*W (a compile-time constant).
template <int W>
struct ColOffsets {
  int a[W / 32], b[W / 32];
  __device__ __forceinline__ ColOffsets(int ra, int rb, int lane) {
    const int j = lane & 15;
#pragma unroll
    for (int db = 0; db < W / 32; ++db) {
      const int col = 32 * db + ((lane >> 4) & 1) * 16 + 4 * (j & 3);
      a[db] = swz<W>(ra + (j >> 2), col);
      b[db] = swz<W>(rb + (j >> 2), col);
    }
  }
};

// Per-lane offsets of the 16-byte row reads (row l32, or the given row,
// column 16*kb + 8h).
template <int W>
struct RowOffsets {
  int o[W / 16];
  __device__ __forceinline__ explicit RowOffsets(int lane) : RowOffsets(lane, lane & 31) {}
  __device__ __forceinline__ RowOffsets(int lane, int row) {
    const int h = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < W / 16; ++kb) o[kb] = swz<W>(row, 16 * kb + 8 * h);
  }
};

// Row r of a 32-row A operand taken from key pi(r) of a 32-key block: the
// 32x32 accumulator row 8*(v/4) + 4h + v%4 of lane half h (VGPR v) is then
// key 16h + v, so each lane holds 16 consecutive keys -- one P quantization
// group -- of its column.
__device__ __forceinline__ int key_perm(int r) {
  return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// bf16 pair from two floats (round to nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// bf16 pair of two floats that are exactly representable in bf16 (their low
// 16 bits are zero): a byte permute instead of a rounding conversion.
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Returns x unchanged but makes the compiler materialize it here: the value
// is computed before this point and not sunk towards its later uses (keeps a
// hand-interleaved VALU stream where it was placed between scheduling fences).
__device__ __forceinline__ uint32_t pin_vgpr(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Waits for every outstanding vector-memory load of this wave (s_waitcnt
// vmcnt(0); expcnt and lgkmcnt left at their maximum).  Used once before a
// main loop whose MFMAs read registers loaded earlier, so that the compiler's
// wait placement inside the loop only has to track the loop's own prefetches.
__device__ __forceinline__ void vmem_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations left
// outstanding (they complete in issue order for loads).
template <int N>
__device__ __forceinline__ void vmem_wait() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Compiler-level ordering point for LDS traffic exchanged between the lanes
// of one wave (LDS operations of a wave complete in issue order).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// MFMA (bf16 in, fp32 accumulate).
//
// v_mfma_f32_32x32x16_bf16, operands per lane l (h = l / 32, i = l % 32):
//   A (32 x 16): row i, k = 8h .. 8h+7
//   B (16 x 32): col i, k = 8h .. 8h+7
//   C (32 x 32): col i, rows 8*(v/4) + 4h + (v%4) for v = 0..15
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Pack 8 floats (already exact or to be rounded) into bf16x8, RNE.
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)f[e];
  return r;
}

// Buffer resource over `bytes` bytes starting at p (raw, unswizzled, 32-bit
// dword format).  Buffer loads past `bytes` return zeros (hardware range
// check), so a tile that runs past the end of a tensor is zero-filled without
// a select on the loaded data, and the per-lane offsets stay loop-invariant.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// Asynchronous copy of 16 bytes per lane straight into LDS
// (buffer_load_dwordx4 ... lds): lane l's bytes land at LDS byte address
// lds + 16*l, and lanes whose offset falls outside the descriptor's
// num_records bytes write zeros.  `lds` must be wave-uniform.  Completion is
// counted by vmcnt like any vector-memory load; the caller waits
// (vmem_wait) and synchronizes before reading the destination.  Issued as
// inline assembly so that the compiler does not add its own conservative
// vmcnt waits in front of every later LDS read.
// (The descriptor must live in SGPRs: its fields are read as wave-uniform.)
__device__ __forceinline__ u32x4 buf_desc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu),
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p);
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; it is set right here
__device__ __forceinline__ void buf_ld16_lds(const u32x4& desc, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(desc)
      : "memory", "m0");
}
// The same for 4 bytes per lane (buffer_load_dword ... lds): lane l's dword
// lands at lds + 4*l.
__device__ __forceinline__ void buf_ld4_lds(const u32x4& desc, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(desc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ float buf_ldf(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const void* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ void st_bf16x8(void* p, bf16x8 v) {
  *reinterpret_cast<bf16x8*>(p) = v;
}

// Exchange with the lane 32 positions away (lanes 0-31 <-> 32-63).
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

}  // namespace attnqat
