/* Host check of the reciprocal-and-FMA division the fp8 tiled GEMMs use to
 * requantise h: for s >= 2^-64 and y = 1/s (IEEE), q = |a| y refined twice by
 * q += fma(-q, s, |a|) * y (one FMA each), with a's sign restored, must equal
 * the IEEE quotient a / s bit for bit whenever |a / s| >= 2^-10 (half the
 * smallest e4m3 step); smaller quotients (subnormal numerators) may differ in
 * the last bits but must stay below 2^-10 with the same sign, so that their
 * e4m3 code is the same signed zero.  Inputs: log-uniform block maxima
 * 2^-60 .. 2^60 with s = amax / 448 and a drawn inside +-amax, values whose
 * quotient lands within a few ulps of every e4m3 rounding midpoint, +-0 and
 * subnormal numerators.  Prints the number of mismatches (0 expected). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float div_rn_by(float a, float s, float y) {
  const float m = fabsf(a);
  float q = m * y;
  q = fmaf(fmaf(-q, s, m), y, q);
  q = fmaf(fmaf(-q, s, m), y, q);
  return copysignf(q, a);
}

static uint32_t bits(float v) { uint32_t b; memcpy(&b, &v, 4); return b; }
static float from_bits(uint32_t b) { float v; memcpy(&v, &b, 4); return v; }

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) { rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17; return rs; }
static double unif(void) { return (double)(next() >> 11) * 0x1p-53; }

static long long n_bad = 0, n_cases = 0;
static void check(float a, float s) {
  if (!(s >= 0x1p-64f)) return;
  const float y = 1.f / s;
  const float got = div_rn_by(a, s, y), want = a / s;
  ++n_cases;
  const int small = fabsf(want) < 0x1p-10f;
  const int ok = small ? fabsf(got) < 0x1p-10f && signbit(got) == signbit(want) : bits(got) == bits(want);
  if (!ok) {
    if (n_bad < 10) printf("mismatch a=%a s=%a got=%a want=%a\n", a, s, got, want);
    ++n_bad;
  }
}

int main(int argc, char** argv) {
  const long long n = argc > 1 ? atoll(argv[1]) : 2000000;
  for (long long i = 0; i < n; ++i) {
    const float amax = (float)ldexp(1.0 + unif(), (int)(unif() * 120.0) - 60);
    const float s = amax / 448.f;
    check((float)(amax * (2.0 * unif() - 1.0)), s);
    check(amax, s);
    check(-amax, s);
    /* a quotient near an e4m3 midpoint: m = (2k + 1) 2^(e - 4), e in -10 .. 8 */
    const int e = (int)(unif() * 19.0) - 10;
    const int k = (int)(unif() * 8.0);
    const double mid = (2.0 * k + 1.0) * ldexp(1.0, e - 4) + (e < -6 ? 0.0 : ldexp(1.0, e));
    const float a0 = (float)(mid * s);
    const uint32_t b0 = bits(a0);
    for (int d = -3; d <= 3; ++d) {
      check(from_bits(b0 + d), s);
      check(-from_bits(b0 + d), s);
    }
    check(from_bits((uint32_t)(next() & 0x7FFFFFu)), s);   /* subnormal numerator */
  }
  check(0.f, 1.f);
  check(-0.f, 1.f);
  check(-0.f, 0x1p-60f);
  printf("cases %lld mismatches %lld\n", n_cases, n_bad);
  return n_bad != 0;
}
