/*
 * Host check of the kernels' temperature scale (test infrastructure): the
 * fast form fl32(fl64(x) fl64(1/T)) and, for T >= 2, the recomputation of
 * results at or below 2^-126 with the double-double form
 * fl32(fma(x, r_hi, fl64(x r_lo))), r_lo = fl64((1 - r_hi T) r_hi), against
 * IEEE fp32 division, over every positive fp32 with bit pattern in
 * [lo_bits, hi_bits). Built with -ffp-contract=off (plain IEEE operations).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float fast_form(float x, double rh) { return (float)((double)x * rh); }
static float dd_form(float x, double rh, double rl) {
  return (float)fma((double)x, rh, (double)x * rl);
}

/* form: 0 fast, 1 double-double, 2 the kernels' rule */
long scale_mismatches(float t, uint32_t lo_bits, uint32_t hi_bits, int form) {
  const double rh = 1.0 / (double)t;
  const double rl = fma(-rh, (double)t, 1.0) * rh;
  long bad = 0;
  for (uint32_t b = lo_bits; b < hi_bits; ++b) {
    float x;
    memcpy(&x, &b, sizeof x);
    float s;
    if (form == 0) s = fast_form(x, rh);
    else if (form == 1) s = dd_form(x, rh, rl);
    else {
      s = fast_form(x, rh);
      if (t >= 2.0f && fabsf(s) <= 0x1p-126f) s = dd_form(x, rh, rl);
    }
    if (s != x / t) ++bad;
  }
  return bad;
}
