/* Exhaustive host check of the division-free quotient used by the GPU
 * per-token quantiser (quant8 in the library's device helpers).
 *
 * For every BF16 row maximum amax (s = fl32(amax / 448), or 1 for a zero row,
 * r = fl32(1 / s)) and every BF16 x with |x| <= amax, both signs, the kernel
 * computes, when s >= 2^-99,
 *     q0 = fl32(x * r),  q = copysign(fma(fma(-q0, s, x), r, q0), x)
 * (Markstein's residual correction) and otherwise q = fl32(x / s). The E4M3
 * code of q must equal that of fl32(x / s): this program checks that q equals
 * fl32(x / s) bit for bit where |x / s| >= 2^-12, and elsewhere has magnitude
 * below 2^-11 (E4M3 code +-0) with the sign of x / s.
 *
 * argv[1] selects the formula: 0 = the kernel's; 1 = without the copysign;
 * 2 = the correction for every scale; 3 = x * r alone. 1..3 are planted
 * mistakes that the check must catch. Prints the failure count; exit status
 * 0 when the count is zero. Build: gcc -O2 -std=c11 -ffp-contract=off
 * -fopenmp (fmaf is the C library's correctly rounded fused multiply-add).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(int argc, char** argv) {
  const int mode = argc > 1 ? atoi(argv[1]) : 0;
  long long pairs = 0, failures = 0;
  int stop = 0; /* set once a planted mistake is caught; OpenMP atomics */
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, failures)
  for (int a = 0; a <= 0x7F7F; ++a) {
    int stopped;
#pragma omp atomic read
    stopped = stop;
    if (stopped) continue;
    const float s = a == 0 ? 1.0f : bf16((uint32_t)a) / 448.0f;
    const float r = 1.0f / s;
    const int corrected = mode == 2 || s >= 0x1p-99f;
    for (uint32_t m = 0; m <= (uint32_t)a; ++m) {
      for (uint32_t sign = 0; sign < 2; ++sign) {
        const float x = bf16(m | (sign << 15));
        const float want = x / s;
        float q;
        if (mode == 3) {
          q = x * r;
        } else if (corrected) {
          const float q0 = x * r;
          q = fmaf(fmaf(-q0, s, x), r, q0);
          if (mode != 1) q = copysignf(q, x);
        } else {
          q = x / s;
        }
        const int ok = fabsf(want) >= 0x1p-12f ? bits(q) == bits(want)
                                                 : (fabsf(q) < 0x1p-11f && signbit(q) == signbit(want));
        ++pairs;
        if (!ok) {
          ++failures;
          if (mode != 0) {
#pragma omp atomic write
            stop = 1;
          }
        }
      }
    }
  }
  printf("mode %d pairs %lld failures %lld\n", mode, pairs, failures);
  return failures != 0;
}
