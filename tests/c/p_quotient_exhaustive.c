/* Exhaustive check of the probability quotient used with the E2M1 rounding of
 * P ("NVFP4 Attention QAT Backward", Overview: the codes are the
 * round-to-nearest-even of x/s with precise division).
 *
 * The kernels form q = fma(x, r_hi, x * r_lo) with r_hi the hardware
 * reciprocal of s (within 1 ulp; all three candidates are tried) and
 * r_lo = fma(-r_hi, s, 1) * r_hi, and round q to E2M1 with the hardware
 * conversion (round to nearest even, saturating at 6).  For every E4M3
 * mantissa of s (the check is invariant under the power-of-two part) and
 * every fp32 x in [s/8, 8s) this program compares that code with the exact
 * rounding of the rational x/s (comparisons of x with m*s in double, which
 * are exact), and prints the number of mismatches.  Below s/8 both codes are
 * 0 (q < 0.126 < 0.25); at or above 8s both saturate at 6. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E2M1 midpoints; at 0.25, 1.25, 2.5 and 5 a tie rounds down (to the even
 * code), at 0.75, 1.75 and 3.5 it rounds up */
static const double MID[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};

static int code_exact(double x, double s) {
  int k = 0;
  for (int i = 0; i < 7; ++i) {
    const double t = MID[i] * s;
    k += (i % 2 == 0) ? (x > t) : (x >= t);
  }
  return k;
}

static int code_of_quotient(float q) {
  int k = 0;
  for (int i = 0; i < 7; ++i) {
    const float t = (float)MID[i];
    k += (i % 2 == 0) ? (q > t) : (q >= t);
  }
  return k;
}

int main(void) {
  long bad = 0, n = 0;
  for (int M = 8; M <= 15; ++M) {
    const float s = M / 8.0f;
    for (int dv = -1; dv <= 1; ++dv) {
      const float r_hi = f_of(u_of(1.0f / s) + dv);
      const float r_lo = fmaf(-r_hi, s, 1.0f) * r_hi;
      const uint32_t u0 = u_of(s / 8.0f), u1 = u_of(8.0f * s);
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
      for (long long u = u0; u < (long long)u1; ++u) {
        const float x = f_of((uint32_t)u);
        const float q = fmaf(x, r_hi, x * r_lo);
        if (code_of_quotient(q) != code_exact((double)x, (double)s)) ++bad;
        ++n;
      }
    }
  }
  printf("checked %ld mismatches %ld\n", n, bad);
  return 0;
}
