/* Exhaustive check of the E4M3 block-scale arithmetic used by the GPU codec
 * ("NVFP4 Attention QAT Backward", Overview: the per-16 E4M3 scale is the
 * round-to-nearest-even of amax/6).
 *
 * The kernels form the quotient without a divide: y0 = amax * (1/6)f, then
 * one FMA correction y = fma(fma(-y0, 6, amax), (1/6)f, y0), and round y to
 * E4M3 with the hardware FP8 conversion after clamping at 448 (round to
 * nearest even, subnormals included; the GPU codec tests pin that conversion
 * at every E4M3 rounding boundary).  Here that rounding is written out: nearest
 * even on the fp32 bit pattern in the normal range, rint(y*512) / 512 below
 * 2^-6, saturating at 448.  For every finite non-negative fp32
 * amax this program compares that result with the exact rounding of the
 * rational amax/6 onto the E4M3 grid (comparisons against 6*g in double,
 * which are exact), and prints the number of mismatches.  It also counts
 * the mismatches of the uncorrected product y0, which are expected. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float e4m3_from_y(float y) {
  float s;
  if (y < 0x1p-6f) {
    s = rintf(y * 512.0f) * 0x1p-9f;
  } else {
    uint32_t u = u_of(y);
    u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
    s = f_of(u);
  }
  return fminf(s, 448.0f);
}

static double grid[127]; /* non-negative finite E4M3 values, code order */

static double exact_scale(float amax) {
  const double t = amax;
  int lo = 0, hi = 126;
  if (t >= 6.0 * grid[126]) return grid[126];
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (6.0 * grid[mid] <= t) lo = mid; else hi = mid;
  }
  const double d0 = t - 6.0 * grid[lo], d1 = 6.0 * grid[hi] - t;
  if (d0 < d1) return grid[lo];
  if (d1 < d0) return grid[hi];
  return (lo % 2 == 0) ? grid[lo] : grid[hi];
}

int main(void) {
  for (int c = 0; c < 127; ++c) {
    const int e = c >> 3, m = c & 7;
    grid[c] = e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  }
  const float r6 = 1.0f / 6.0f;
  long bad_fma = 0, bad_mul = 0, n = 0;
#pragma omp parallel for reduction(+ : bad_fma, bad_mul, n) schedule(static)
  for (long long v = 0; v < 0x7F800000LL; ++v) {
    const float amax = f_of((uint32_t)v);
    const double ex = exact_scale(amax);
    const float y0 = amax * r6;
    const float y = fmaf(fmaf(-y0, 6.0f, amax), r6, y0);
    if ((double)e4m3_from_y(y) != ex) ++bad_fma;
    if ((double)e4m3_from_y(y0) != ex) ++bad_mul;
    ++n;
  }
  printf("checked %ld fma_mismatches %ld mul_mismatches %ld\n", n, bad_fma, bad_mul);
  return 0;
}
