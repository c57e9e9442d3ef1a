/* Host check of the quotient step of the NVFP4 block-scale computation:
 * q1 = fma(fma(-q0, d, m), rd, q0) with q0 = m * rd and rd = 1 / d (all FP32,
 * round to nearest) must equal the FP32 quotient m / d.  Usage:
 *   fdiv_check <divisors> <random pairs> <seed>
 * Every dividend significand at two exponents for each of the divisors
 * (the first two fixed: 2 - 2^-22 and 3), then random pairs placed near a
 * rounding midpoint of the quotient.  Prints the number of mismatches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static uint64_t st;
static uint64_t next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }

static float quot(float m, float d, float rd) {
  const float q0 = m * rd;
  const float r = fmaf(-q0, d, m);
  const float q1 = fmaf(r, rd, q0);
  return q1 == q1 ? q1 : q0;
}

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const int nd = atoi(argv[1]);
  const long nr = atol(argv[2]);
  st = 0x9E3779B97F4A7C15ull ^ (uint64_t)atol(argv[3]);
  long bad = 0;
  for (int t = 0; t < nd; ++t) {
    float d = u2f((127u << 23) | (uint32_t)(next() & 0x7FFFFF));
    if (t == 0) d = u2f(0x3FFFFFFFu);
    if (t == 1) d = 3.0f;
    const float rd = 1.0f / d;
    for (uint32_t e = 127; e <= 128; ++e)
      for (uint32_t mm = 0; mm < 0x800000u; ++mm) {
        const float m = u2f((e << 23) | mm);
        if (f2u(quot(m, d, rd)) != f2u(m / d)) ++bad;
      }
  }
  for (long i = 0; i < nr; ++i) {
    const uint64_t x = next();
    const int de = (int)((x >> 23) % 41) - 20, qe = (int)((x >> 55) % 22) - 12;
    const float d = u2f(((uint32_t)(de + 127) << 23) | (uint32_t)(x & 0x7FFFFF));
    const float rd = 1.0f / d;
    const double q = (double)u2f(((uint32_t)(qe + 127) << 23) | (uint32_t)((x >> 32) & 0x7FFFFF));
    const float m0 = (float)((q + ldexp(1.0, qe - 24)) * (double)d);
    const float m = u2f(f2u(m0) + (uint32_t)((int)((x >> 60) & 7) - 3));
    if (f2u(quot(m, d, rd)) != f2u(m / d)) ++bad;
  }
  printf("%ld\n", bad);
  return 0;
}
