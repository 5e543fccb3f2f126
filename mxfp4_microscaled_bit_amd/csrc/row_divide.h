// The forward's last step, O = O~ / l per query row (MXAttention paper,
// Sec. 4, Eq. 8), rounded once per element without a full division each.
// In one place so that a host-only check (compiled with g++, where __host__
// and __device__ expand to nothing) exercises the very functions the kernels
// call.
//
// With y = RN(1/l), q0 = RN(a y) lies within one ulp of a / l; the fused
// residual s = q0 l - a is then exact, and RN(q0 - s y) is the correctly
// rounded quotient RN(a / l) (Markstein's theorem on division by a correctly
// rounded reciprocal).  Taking the residual as q0 l - a and subtracting it
// leaves q0 unchanged when a is a zero of either sign (-0 + q0 keeps q0's
// sign), so zeros need no special case.  The theorem needs an exact residual
// and a normal quotient: a row takes this route only when l lies in
// [1, 2^100] and every nonzero |a| of the row lies in [2^-100 l, FLT_MAX];
// any other row (a tiny or an infinite element) divides element by element.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace mxattn_internal {

// Guard key of one element: twice its magnitude's bits minus one, unsigned.
// Zeros of either sign map to 0xFFFFFFFF, above every other key, so the
// row's smallest key is that of its smallest nonzero |a|; a NaN maps above
// every finite key (it yields NaN on either route).
__host__ __device__ __forceinline__ uint32_t row_divide_key(float a) {
  return (__builtin_bit_cast(uint32_t, a) << 1) - 1u;
}

// min_key: the smallest row_divide_key of the row; max_abs: its largest |a|
// (a NaN may be skipped)
__host__ __device__ __forceinline__ bool row_divide_by_reciprocal(float l, uint32_t min_key, float max_abs) {
  if (!(l >= 1.0f && l <= 0x1p100f)) return false;
  return min_key >= row_divide_key(0x1p-100f * l) && max_abs <= 0x1.fffffep127f;
}

// RN(a / l) from y = RN(1 / l), for a row that row_divide_by_reciprocal accepts
__host__ __device__ __forceinline__ float quotient_from_reciprocal(float a, float l, float y) {
  const float q0 = a * y;
  const float s = fmaf(q0, l, -a);
  return fmaf(-s, y, q0);
}

}  // namespace mxattn_internal
