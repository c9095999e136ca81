/* Checks, on the host, the quotient the quantisation kernels compute:
 * q = copysign(fma(fma(-x*r, s, x), r, x*r), x) with s = max(amax, 1e-8)/448
 * and r = 1/s (both IEEE float32 divisions), against the IEEE quotient x/s.
 *   mode "bf16": every positive bf16 amax and every bf16 x with 0 <= x <= amax
 *                (the whole domain of the activation quantiser, up to the
 *                sign symmetry of IEEE rounding), plus -x for every fourth
 *                amax and -0 for all;
 *   mode "random": N random float32 pairs with |x| <= amax (the
 *                requantisation domain).
 * The sign must agree on every quotient.  Below 2^-12 in magnitude only the
 * sign is compared, since every such value rounds to an e4m3 zero of that
 * sign.  Prints "checked mismatches". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static int check(float x, float amax, unsigned long long* n) {
  volatile float s = fmaxf(amax, 1e-8f) / 448.0f;
  volatile float r = 1.0f / s;
  volatile float ref = x / s;
  volatile float q0 = x * r;
  volatile float rem = fmaf(-q0, s, x);
  volatile float q = copysignf(fmaf(rem, r, q0), x);
  ++*n;
  if (fabsf(ref) < 0x1p-12f) return (u_of(q) >> 31) != (u_of(ref) >> 31);
  return u_of(q) != u_of(ref);
}

static uint64_t st = 88172645463325252ull;
static uint32_t next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)(st >> 16); }

int main(int argc, char** argv) {
  unsigned long long n = 0, bad = 0;
  if (argc > 1 && strcmp(argv[1], "random") == 0) {
    long long N = argc > 2 ? atoll(argv[2]) : 10000000;
    for (long long i = 0; i < N; ++i) {
      float amax = f_of(next() % 0x7F000000u + 0x00800000u);   /* normal, finite */
      float x = amax * (float)((next() & 0xFFFFFF) + 1) * 0x1p-24f;
      if (x > amax) x = amax;
      bad += check(x, amax, &n);
      bad += check(f_of(u_of(amax) - (next() & 0xFFFF)), amax, &n);
    }
  } else {
    for (uint32_t a = 1; a < 0x7F80; ++a) {
      const float amax = f_of(a << 16);
      for (uint32_t b = 0; b <= a; ++b) {
        bad += check(f_of(b << 16), amax, &n);
        if ((a & 3) == 0 || b == 0) bad += check(f_of((b << 16) | 0x80000000u), amax, &n);
      }
    }
  }
  printf("%llu %llu\n", n, bad);
  return bad != 0;
}
