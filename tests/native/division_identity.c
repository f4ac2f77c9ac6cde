/* Checks the arithmetic the GPU quantizer relies on (host C, no GPU):
 *  (1) fl32(w / s) == fma(w, r_hi, fl32(w * r_lo)) with r_hi = fl32(1 / s),
 *      r_lo = fl32(fma(-s, r_hi, 1) * r_hi), for every finite fp16 w and every
 *      STEP-th positive finite fp16 s (STEP = 1 is the exhaustive check);
 *  (2) fl32(d / M) == fma(d, m_hi, fl32(d * m_lo)) for every fp32 significand d
 *      and M = 3, 7, 15, 127, 255 (the min-max divisors 2^b - 1 and the
 *      symmetric divisors 2^(b-1) - 1 of b = 2, 3, 4, 8);
 *  (3) |w| / s < 2^22 for groups whose extrema lie within 8 fp16 steps of
 *      each other (where |w| / s is largest), so v + 1.5 * 2^23 rounds exactly.
 * Usage: division_identity [STEP [PART PARTS]]: with PARTS > 1, check (1)
 * covers only the scales whose index is PART modulo PARTS, so that PARTS
 * processes together cover every STEP-th scale once.
 * Prints one line per check and exits non-zero on any failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float h2f(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v = e == 0 ? ldexp(m, -24) : ldexp(1024 + m, e - 25);
  return (float)(s ? -v : v);
}

static uint16_t f2h(float f) { /* round to nearest even, finite values */
  double a = fabs((double)f);
  uint16_t sg = signbit(f) ? 0x8000 : 0;
  if (a == 0) return sg;
  if (a < ldexp(1, -14)) return sg | (uint16_t)nearbyint(ldexp(a, 24));
  int E;
  frexp(a, &E);
  int e = E - 1;
  double m = nearbyint(ldexp(a, 10 - e));
  if (m == 2048) { m = 1024; e++; }
  if (e > 15) return sg | 0x7c00;
  return sg | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

int main(int argc, char** argv) {
  const int step = argc > 1 ? atoi(argv[1]) : 1;
  const int part = argc > 3 ? atoi(argv[2]) : 0, parts = argc > 3 ? atoi(argv[3]) : 1;
  if (step < 1 || parts < 1 || part < 0 || part >= parts) return 2;
  long bad = 0, n = 0;
  long idx = -1;
  for (uint32_t sb = 1; sb < 0x7c00; sb += (uint32_t)step) {
    if (++idx % parts != part) continue;
    const float s = h2f((uint16_t)sb);
    volatile float one = 1.0f;
    const float r_hi = one / s;
    const float r_lo = fmaf(-s, r_hi, 1.0f) * r_hi;
    for (uint32_t wb = 0; wb < 0x10000; ++wb) {
      if (((wb >> 10) & 31) == 31) continue;
      const float w = h2f((uint16_t)wb);
      const float q = w / s, v = fmaf(w, r_hi, w * r_lo);
      ++n;
      if (memcmp(&q, &v, 4) != 0 && !(q == 0 && v == 0)) ++bad;
    }
  }
  printf("quotient identity: %ld pairs, %ld mismatches\n", n, bad);
  long bad2 = 0;
  const int Ms[5] = {3, 7, 15, 127, 255};
  for (int i = 0; i < 5; ++i) {
    volatile float mv = (float)Ms[i];
    const float m = mv, m_hi = 1.0f / m, m_lo = fmaf(-m, m_hi, 1.0f) * m_hi;
    for (uint32_t f = 0; f < (1u << 23); ++f) {
      uint32_t bits = (127u << 23) | f;
      float d;
      memcpy(&d, &bits, 4);
      const float q = d / m, v = fmaf(d, m_hi, d * m_lo);
      if (memcmp(&q, &v, 4) != 0) ++bad2;
    }
  }
  printf("scale identity: %ld mismatches\n", bad2);
  double worst = 0;
  for (int i = 0; i < 5; ++i) {
    for (uint32_t lb = 0; lb < 0x10000; ++lb) {
      if (((lb >> 10) & 31) == 31) continue;
      const float lo = h2f((uint16_t)lb);
      float hi = lo;
      for (int k = 0; k <= 8; ++k) {
        if (k > 0) hi = nextafterf(hi, INFINITY);
        const uint16_t hh = f2h(hi);
        if (((hh >> 10) & 31) == 31) break;
        hi = h2f(hh);
        const float dd = hi - lo, s32 = dd / (float)Ms[i];
        uint16_t s16 = f2h(s32);
        if ((s16 & 0x7fff) == 0) s16 = 0x3c00;
        const double r = fmax(fabs((double)lo), fabs((double)hi)) / (double)h2f(s16);
        if (r > worst) worst = r;
      }
    }
  }
  printf("largest |w|/s: %.1f\n", worst);
  return (bad || bad2 || !(worst < 4194304.0)) ? 1 : 0;
}
