// Host-side check of the forward's epilogue division (csrc/row_divide.h):
// for every row the kernel sends through the reciprocal, the result must be
// the correctly rounded quotient a / l, bit for bit, as the host's IEEE
// division gives it.  Random and boundary operands: significands of l with
// all bits set or clear, l from 1 to 2^100, a at the 2^-100 l threshold, far
// below it, at FLT_MAX and zero, both signs.  The guard itself is checked on
// the rows it must refuse (subnormal, tiny or infinite elements; l outside
// [1, 2^100]) and accept (zeros of either sign, NaN elements).
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "row_divide.h"

using namespace mxattn_internal;

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next() { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main() {
  long checked = 0, wrong = 0;
  for (long it = 0; it < 40000000L; ++it) {
    const uint64_t x = next(), z = next();
    const int k = (int)(it & 31);
    uint32_t le = 127 + (uint32_t)(x % 100);  // l in [1, 2^100)
    uint32_t lm = (uint32_t)(x >> 8) & 0x7FFFFFu;
    if (k == 0) lm = 0x7FFFFFu;
    if (k == 1) lm = 0;
    if (k == 2) le = 227, lm = 0;  // l = 2^100
    const float l = from_bits((le << 23) | lm);
    uint32_t ae = 27 + (uint32_t)(z % 228);
    if (k >= 3 && k < 8) ae = 27 + (le - 127) + (uint32_t)(z % 4);  // at the threshold
    uint32_t am = (uint32_t)(z >> 8) & 0x7FFFFFu;
    if (k == 9) am = 0x7FFFFFu;
    if (k == 10) ae = 254, am = 0x7FFFFFu;  // FLT_MAX
    if (k >= 11 && k < 14) ae = 1 + (uint32_t)(z % 40), le = 127 + (uint32_t)(x % 8);  // tiny a, small l
    if (k == 14) am = 0, ae = 0;  // a zero (either sign)
    const float a = from_bits((uint32_t)((z >> 40) & 1u) << 31 | (ae << 23) | am);
    if (!row_divide_by_reciprocal(l, row_divide_key(a), fabsf(a))) continue;
    ++checked;
    const float q = quotient_from_reciprocal(a, l, 1.0f / l);
    if (to_bits(q) != to_bits(a / l)) {
      if (++wrong < 10) printf("a=%a l=%a: %a, correctly rounded %a\n", a, l, q, a / l);
    }
  }
  // rows the guard must send to the element-by-element division: l, the
  // smallest nonzero |a| (0: none), the largest |a|
  const float refused[][3] = {{2.0f, 0x1p-130f, 1.0f},              // a subnormal element
                              {2.0f, -0x1p-130f, 1.0f},             // (negative)
                              {0x1p20f, 0x1p-81f, 1.0f},            // below 2^-100 l
                              {2.0f, 1.0f, INFINITY},               // an infinite element
                              {0.5f, 1.0f, 2.0f},                   // l < 1
                              {0x1p101f, 0x1p10f, 0x1p20f},         // l > 2^100
                              {INFINITY, 1.0f, 2.0f},               // l infinite
                              {NAN, 1.0f, 2.0f}};                   // l NaN
  int refused_ok = 1;
  for (const auto& c : refused)
    if (row_divide_by_reciprocal(c[0], row_divide_key(c[1]), c[2])) {
      printf("guard accepted l=%a lo=%a hi=%a\n", c[0], c[1], c[2]);
      refused_ok = 0;
    }
  // rows it must accept: zeros of either sign beside normal elements, an
  // all-zero row, a NaN element (NaN on either route)
  const float accepted[][3] = {{2.0f, 0.0f, 1.0f}, {2.0f, -0.0f, 1.0f}, {1.0f, 0.0f, 0.0f}, {3.0f, NAN, 2.0f}};
  for (const auto& c : accepted)
    if (!row_divide_by_reciprocal(c[0], row_divide_key(c[1]), c[2])) {
      printf("guard refused l=%a lo=%a hi=%a\n", c[0], c[1], c[2]);
      refused_ok = 0;
    }
  // signed zeros and exact quotients through the fast route
  for (float l : {1.0f, 1.5f, 3.0f, 0x1.fffffep0f, 1000.0f, 0x1p100f})
    for (float a : {0.0f, -0.0f, 1.0f, -1.0f, 3.0f * l, -7.0f * l}) {
      const float q = quotient_from_reciprocal(a, l, 1.0f / l);
      if (to_bits(q) != to_bits(a / l)) {
        printf("a=%a l=%a: %a, correctly rounded %a\n", a, l, q, a / l);
        refused_ok = 0;
      }
    }
  printf("checked %ld quotients, %ld not correctly rounded\n", checked, wrong);
  if (wrong == 0 && refused_ok && checked > 10000000L) {
    printf("epilogue division correctly rounded\n");
    return 0;
  }
  return 1;
}
