/* Host check of the quotient that the FP8 convert kernel forms.
 *
 * The per-tensor FP8 code of x is defined on fl32(x / s), s = fl32(amax /
 * fmax).  The kernel forms that quotient without a division when s lies in
 * [2^-60, inf): q0 = fl32(x * r) with r = fl32(1 / s), then
 * q = fma(fma(-q0, s, x), r, q0) with the sign of x (the sum in the last
 * step turns x = -0 into +0).  This program compares q with the IEEE
 * quotient for every pair of bf16 values |x| <= amax, amax > 0 finite, for
 * both formats' fmax (448 and 57344), and counts the pairs where the signs
 * differ or the values differ while either magnitude reaches 2^-18 (below
 * 2^-18 both formats round to the code of a signed zero, so such
 * differences cannot change a code).
 *
 * Output: one line "pairs N fast F mismatches M"; exit status 0 iff M == 0.
 * Build: cc -O2 -fopenmp -ffp-contract=off fp8_quotient_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bf16(uint32_t bits) {
  const uint32_t u = bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

int main(void) {
  const float fmax[2] = {448.0f, 57344.0f};
  long long pairs = 0, fast = 0, bad = 0;
  for (int f = 0; f < 2; ++f) {
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, fast, bad)
    for (uint32_t ab = 1; ab < 0x7f80u; ++ab) {  /* positive finite bf16 amax */
      const float amax = from_bf16(ab);
      const float s = amax / fmax[f];
      pairs += 2 * (ab + 1);
      if (!(s >= 0x1p-60f && s < INFINITY)) continue;
      fast += 2 * (ab + 1);
      const float r = 1.0f / s;
      for (uint32_t xb = 0; xb <= ab; ++xb) {  /* bf16 |x| <= amax, both signs */
        for (uint32_t sign = 0; sign < 2; ++sign) {
          const float x = from_bf16(xb | (sign << 15));
          const float ref = x / s;
          const float q0 = x * r;
          const float q = copysignf(fmaf(fmaf(-q0, s, x), r, q0), x);
          const int sign_differs = signbit(q) != signbit(ref);
          const int value_differs = bits_of(q) != bits_of(ref) &&
                                    (fabsf(q) >= 0x1p-18f || fabsf(ref) >= 0x1p-18f);
          if (sign_differs || value_differs) ++bad;
        }
      }
    }
  }
  printf("pairs %lld fast %lld mismatches %lld\n", pairs, fast, bad);
  return bad == 0 ? 0 : 1;
}
