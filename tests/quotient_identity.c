/* Host check of the binary32 identities the quantize-on-append kernel uses
 * in place of a divide and a rint per element (see code_word in
 * kvq_quant.hip).  For a group with stored fp16 scale s > 0, r = RN(1/s)
 * and a numerator num = RN(x - z) of fp16 values (0 or at least 2^-24):
 *
 *   q1 = RN(num * r);  e = fma(-q1, s, num);  q = fma(e, r, q1)
 *
 * must equal RN(num / s), the correctly rounded quotient (a zero's sign
 * aside, which no code depends on); and for a value
 * v in [0, 400], RN(v + 2^23) - 2^23 must equal rint(v) (ties to even).
 *
 * Numerators: for every positive finite fp16 scale, the 81 binary32 values
 * around every k*s and (k + 1/2)*s for k = 0..400 (where the rounding of
 * the quotient to an integer code can flip), plus 2000 seeded random ones
 * in [0, 400 s].  The reference quotient is taken in binary64 and rounded
 * to binary32, which is the correctly rounded binary32 quotient (53 >=
 * 2*24 + 2).  Prints the number of cases and mismatches; exit status 1 on
 * any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_value(unsigned h) {         /* positive fp16 bits -> value */
  unsigned e = (h >> 10) & 31u, m = h & 1023u;
  return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024u), (int)e - 25);
}

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

static uint64_t state = 0x9E3779B97F4A7C15ull;  /* xorshift64 */
static double uniform01(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) * 0x1p-53;
}

static long long cases = 0, bad = 0;

static void check(float num, float s, float r) {
  if (num < 0.f || (num != 0.f && num < 0x1p-24f)) return;  /* not reachable */
  const float q1 = num * r;
  const float e = fmaf(-q1, s, num);
  const float q = fmaf(e, r, q1);
  const float ref = (float)((double)num / (double)s);
  ++cases;
  /* compared as values: a numerator of -0 (x = -0 against z = +0) gives
   * +0 here and -0 for the divide, the same code */
  if (!(q == ref)) {
    if (bad < 5) printf("quotient mismatch: s=%a num=%a got %a want %a\n", s, num, q, ref);
    ++bad;
  }
}

int main(void) {
  for (unsigned h = 1; h < 0x7C00u; ++h) {   /* every positive finite fp16 */
    const float s = half_value(h);
    const float r = (float)(1.0 / (double)s);   /* RN(1/s) */
    for (int k = 0; k <= 400; ++k)
      for (int half = 0; half < 2; ++half) {
        float num = (float)(((double)k + 0.5 * half) * (double)s);
        for (int i = 0; i < 40; ++i) num = nextafterf(num, -INFINITY);
        for (int i = 0; i < 81; ++i, num = nextafterf(num, INFINITY)) check(num, s, r);
      }
    for (int i = 0; i < 2000; ++i) check((float)(uniform01() * 400.0 * (double)s), s, r);
  }
  long long rcases = 0;
  for (float v = 0.f; v <= 400.f; v = nextafterf(v, INFINITY)) {  /* rint by 2^23 */
    const float got = (v + 8388608.f) - 8388608.f;
    ++rcases;
    if (bits_of(got) != bits_of(rintf(v))) {
      if (bad < 5) printf("rounding mismatch: v=%a got %a\n", v, got);
      ++bad;
    }
  }
  printf("%lld quotients, %lld roundings, %lld mismatches\n", cases, rcases, bad);
  return bad != 0;
}
