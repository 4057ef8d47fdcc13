/* The packed write computes a group's scale RN(range / levels) for levels =
 * 15 or 255 without a division: q0 = RN(range * RN(1/levels)), then one fma
 * correction with the exact remainder, q1 = RN(q0 + RN(range - q0 * levels) *
 * RN(1/levels)).  This program checks that q1 equals the IEEE quotient for
 * every finite non-negative fp32 range (2^31 - 2^23 values per divisor), and
 * that range = inf needs the separate case the kernel gives it.  Exit status
 * 0 when both hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float corrected(float a, float levels, float inv) {
  const float q0 = a * inv;
  return fmaf(fmaf(-q0, levels, a), inv, q0);
}

int main(void) {
  const float levels[2] = {15.f, 255.f};
  int bad_total = 0;
  for (int k = 0; k < 2; ++k) {
    const float b = levels[k];
    const float inv = 1.f / b;
    long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (long long u = 0; u < 0x7f800000LL; ++u) {
      const float a = from_bits((uint32_t)u);
      if (to_bits(corrected(a, b, inv)) != to_bits(a / b)) ++bad;
    }
    const int inf_special = isnan(corrected(INFINITY, b, inv));  /* the kernel returns a for a = inf */
    printf("levels %g: inverse %a, mismatches %lld over all finite a >= 0; a = inf needs its case: %d\n",
           b, inv, bad, inf_special);
    bad_total += bad != 0 || !inf_special;
  }
  return bad_total ? 1 : 0;
}
