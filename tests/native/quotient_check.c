/* Exhaustive check of the row quantizer's quotient arithmetic (test infrastructure).
 *
 * The GPU kernel computes |x| / s as y = RN(1/s), q0 = RN(|x| * y), r = fma(-q0, s, |x|),
 * q = fma(r, y, q0) (Markstein's correction) with s = RN(max(amax, 2^-24) / 448).  This program
 * replays that sequence in IEEE single precision for every positive FP16 amax (and the zero
 * row's floor) and every FP16 |x| <= amax, and compares it with the correctly rounded
 * quotient RN(|x| / s).  Exit status 0 iff all 5.0e8 pairs agree.  Build with
 * -ffp-contract=off so the only fused operations are the explicit fmaf calls. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

static float fp16_to_float(uint16_t h) {
  const uint32_t e = (h >> 10) & 31, m = h & 1023;
  float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), (int)e - 25);
  return (h >> 15) ? -v : v;
}

int main(void) {
  static float mag[31744];
  int n = 0;
  for (uint32_t h = 0; h < 0x7C00; ++h) mag[n++] = fp16_to_float((uint16_t)h); /* 0 .. 65504 */
  long long pairs = 0, bad = 0;
  for (int ia = 0; ia < n; ++ia) {
    const float floor24 = ldexpf(1.0f, -24);
    const float amax = mag[ia] < floor24 ? floor24 : mag[ia];
    volatile float s = amax / 448.0f;
    volatile float y = 1.0f / s;
    for (int ix = 0; ix <= ia; ++ix) {
      const float x = mag[ix];
      const float q0 = x * y;
      const float r = fmaf(-q0, s, x);
      const float q = fmaf(r, y, q0);
      const float ref = x / s;
      ++pairs;
      if (q != ref) {
        if (bad < 5) printf("mismatch amax=%a x=%a q=%a ref=%a\n", mag[ia], x, q, ref);
        ++bad;
      }
    }
  }
  printf("pairs %lld mismatches %lld\n", pairs, bad);
  return bad != 0;
}
