/*
 * Exhaustive host check of the quantizers' division shortcut.
 *
 * For online 1x128 / 128x128 scales the kernels compute fl32(x / s) as
 *     r = fl32(1 / s);  y = fl32(x * r);  e = fma(-y, s, x);
 *     q = copysign(fma(e, r, y), x)
 * instead of a full IEEE division per element.  This program checks that q
 * equals the IEEE quotient for EVERY pair the online path can see: every
 * finite non-negative BF16 tile max a, its scale s = max(fl32(a / 448),
 * fl32(1e-12)), and every BF16 x with |x| <= a (both signs).  Quotients below
 * 2^-11 in magnitude need only agree in sign (both encode to a zero code).
 * It also checks the scale's own division, fl32(a / 448) computed as one
 * correction of y = fl32(a * fl32(1/448)), against the IEEE quotient for
 * every finite non-negative BF16 a.
 * Exit status 0 = all pairs and scales agree; prints the counts.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f(uint32_t b) { float v; memcpy(&v, &b, 4); return v; }
static uint32_t u(float v) { uint32_t b; memcpy(&b, &v, 4); return b; }

int main(void) {
  const float floor_s = f(0x2B8CBCCCu);
  uint64_t pairs = 0, bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad)
  for (uint32_t ab = 0; ab <= 0x7F7Fu; ++ab) {           /* finite non-negative BF16 */
    const float a = f(ab << 16);
    float s = a / 448.0f;
    if (s < floor_s) s = floor_s;
    const float r = 1.0f / s;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      for (int sign = 0; sign < 2; ++sign) {
        const float x = f((xb << 16) | (sign ? 0x80000000u : 0));
        const volatile float ref = x / s;
        const float y = x * r;
        const float e = fmaf(-y, s, x);
        const float q = copysignf(fmaf(e, r, y), x);
        ++pairs;
        if (u(q) != u(ref)) {
          const int tiny = fabsf(q) < 0x1p-11f && fabsf(ref) < 0x1p-11f && signbit(q) == signbit(ref);
          if (!tiny) {
            if (bad < 10)
#pragma omp critical
              printf("mismatch a=%08x x=%08x s=%08x q=%08x ref=%08x\n", u(a), u(x), u(s), u(q), u(ref));
            ++bad;
          }
        }
      }
    }
  }
  printf("pairs=%llu mismatches=%llu\n", (unsigned long long)pairs, (unsigned long long)bad);

  /* The scale itself: fl32(a / 448) through one correction of
   * y = fl32(a * fl32(1/448)), for every finite non-negative BF16 a. */
  const float r448 = 1.0f / 448.0f;
  uint64_t scales = 0, bad_s = 0;
  for (uint32_t ab = 0; ab <= 0x7F7Fu; ++ab) {
    const float a = f(ab << 16);
    const volatile float ref = a / 448.0f;
    const float y = a * r448;
    const float e = fmaf(-y, 448.0f, a);
    const float q = fmaf(e, r448, y);
    ++scales;
    if (u(q) != u(ref)) {
      if (bad_s < 10) printf("scale mismatch a=%08x q=%08x ref=%08x\n", u(a), u(q), u(ref));
      ++bad_s;
    }
  }
  printf("scales=%llu scale_mismatches=%llu\n", (unsigned long long)scales, (unsigned long long)bad_s);
  return bad != 0 || bad_s != 0;
}
