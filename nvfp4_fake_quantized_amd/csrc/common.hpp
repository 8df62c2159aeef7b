// Device-side building blocks shared by the attnqat kernels (gfx950 / CDNA4).
//
// NVFP4 fake quantization follows "NVFP4 Attention QAT Backward" (cuDNN
// frontend docs), §Overview: one E4M3FN scale per 16 values, s = RNE(amax/6)
// saturating at 448, E2M1 codes c = RNE(|x|/s) with precise division (exact
// midpoints round to even), x^ = sign(x) * c * s.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnqat {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
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
// at 448.  amax/6 is the correctly rounded fp32 quotient; for bf16 and fp32
// amax it never lands on an E4M3 midpoint unless the exact quotient is that
// midpoint (E4M3 midpoints have 5 significant bits; a non-exact quotient
// stays more than half an fp32 ulp away from them), so rounding it again is
// the exact rounding of amax/6.
__device__ __forceinline__ float e4m3_scale_from_amax(float amax) {
  const float y = amax / 6.0f;  // IEEE division (no fast-math in this library)
  float s;
  if (y < 0x1p-6f) {
    // subnormal E4M3 range: multiples of 2^-9 (y * 512 is exact)
    s = __builtin_rintf(y * 512.0f) * 0x1p-9f;
  } else {
    // keep 3 mantissa bits, round to nearest even on the fp32 bit pattern
    uint32_t u = __float_as_uint(y);
    u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
    s = __uint_as_float(u);
  }
  return fminf(s, 448.0f);
}

// The E4M3FN byte (e << 3 | m, bias 7) of a scale produced above.
__device__ __forceinline__ uint32_t e4m3_byte(float s) {
  if (s < 0x1p-6f) return (uint32_t)(s * 512.0f);
  const uint32_t u = __float_as_uint(s);
  const uint32_t e = ((u >> 23) & 0xFFu) - 120u;  // -127 + 7
  const uint32_t m = (u >> 20) & 7u;
  return (e << 3) | m;
}

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
