// Device code for one 32-element MXFP4 block along the head dimension:
// 16-bit decode, the Hadamard butterflies of a row spread over the lanes of
// a quad, the shared-scale exponent and the E2M1 codes.  Included by the
// standalone quantizer and by the attention kernel's fused Q prologue, so
// both produce the same codes bit for bit.  Floating-point contraction is
// off in every function here: each butterfly is one rounded add or
// subtract and the 1/sqrt(d) multiply is rounded on its own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxattn_internal {
namespace mxblock {

constexpr int kRuleUos = 0;
constexpr int kRuleOcp = 1;
constexpr int kRuleCeilQ = 2;

// Two packed 16-bit inputs -> two binary32 values (exact).
template <int DTYPE>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
  if constexpr (DTYPE == 0) {  // bfloat16: the top half of a binary32
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
  } else {  // IEEE binary16
    lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
    hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
}

// Partner values across the lanes of a quad (DPP quad_perm, no LDS traffic).
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}

// Shared-scale exponent of a block whose max magnitude is M >= 0, from the
// binary32 fields of M = 1.f * 2^(E-127):
//   OCP: floor(log2 M) - 2 = E - 129;
//   UOS: ceil(log2(M / 7.25)) = E - 129 + [1.f > 29/16]  (29/16 = 1.1101b,
//        whose fraction field is 0x680000);
//   ceiling rule with boundary q = 1.g * 2^(Q-127) (bits `qb`):
//        ceil(log2(M / q)) = E - Q + [1.f > 1.g].  M <= q 2^e holds for a
//        binary32 M exactly when it holds for q rounded down to binary32, so
//        the caller passes that rounding.
// A zero block gets 0 (scale 1); a subnormal M needs e <= -127 for every
// boundary >= 2, which the E8M0 range clamps to -127.
template <int RULE>
__device__ __forceinline__ int scale_exponent(float M, uint32_t qb = 0u) {
  const uint32_t b = __float_as_uint(M);
  if (b == 0u) return 0;
  const int E = (int)(b >> 23);
  if (E == 0) return -127;
  int e;
  if constexpr (RULE == kRuleCeilQ) {
    e = E - (int)(qb >> 23) + (((b & 0x7FFFFFu) > (qb & 0x7FFFFFu)) ? 1 : 0);
    e = e > 127 ? 127 : e;
  } else {
    e = E - 129;
    if constexpr (RULE == kRuleUos) e += ((b & 0x7FFFFFu) > 0x680000u) ? 1 : 0;
  }
  return e < -127 ? -127 : e;
}

// 2^k as a binary32 for k in [-126, 127].
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Eight E2M1 codes of y[0..7] / 2^e in one word, element 2k in the low
// nibble of byte k.  The hardware convert divides by the binary32 scale 2^e
// (exact for a power of two), rounds to the nearest E2M1 value with ties to
// the even code, saturates at 6 and keeps the sign of values that round to
// zero.  The first convert's merge input is irrelevant: the four converts
// write all four bytes.
__device__ __forceinline__ uint32_t cvt8(const float* y, float scale) {
  uint32_t w = __float_as_uint(y[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], scale, 3);
  return w;
}

// Codes of a 32-element block y[] with shared exponent e, 16 bytes.  The scale
// 2^e is a normal binary32 for e >= -126; at the clamp e = -127 every element
// is below 2^-124, and ldexp by 127 moves it up exactly before a unit-scale
// convert.
__device__ __forceinline__ uint4 block_codes(float* y, int e) {
#pragma clang fp contract(off)
  float sc = pow2f(e < -126 ? 0 : e);
  if (e < -126) {
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = __builtin_amdgcn_ldexpf(y[i], 127);
  }
  return make_uint4(cvt8(y, sc), cvt8(y + 8, sc), cvt8(y + 16, sc), cvt8(y + 24, sc));
}

template <int DTYPE>
__device__ __forceinline__ void unpack_block(const uint4 (&raw)[4], float (&v)[32]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    unpack2<DTYPE>(raw[k].x, v[8 * k + 0], v[8 * k + 1]);
    unpack2<DTYPE>(raw[k].y, v[8 * k + 2], v[8 * k + 3]);
    unpack2<DTYPE>(raw[k].z, v[8 * k + 4], v[8 * k + 5]);
    unpack2<DTYPE>(raw[k].w, v[8 * k + 6], v[8 * k + 7]);
  }
}

// Unnormalized Hadamard butterflies of one row, for the 32-channel block
// `blk` held by this lane; the row's d/32 blocks sit in consecutive lanes of
// one quad.  Strides 1..16 stay in registers; stride 32 pairs this lane with
// lane^1 and stride 64 with lane^2: the lane holding the first element keeps
// a + b, the other b_partner - own, written as partner + (-own) with the sign
// flipped by XOR.  Every lane of the quad must execute this.
template <int D>
__device__ __forceinline__ void rotate_block(float (&v)[32], int blk) {
#pragma clang fp contract(off)
#pragma unroll
  for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & hs) == 0) {
        const float a = v[i], bb = v[i + hs];
        v[i] = a + bb;
        v[i + hs] = a - bb;
      }
    }
  }
  {
    const uint32_t flip = (blk & 1) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float p = quad_xor1(v[i]);
      v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ flip);
    }
  }
  if constexpr (D == 128) {
    const uint32_t flip = (blk & 2) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float p = quad_xor2(v[i]);
      v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ flip);
    }
  }
}

// Block max of what the quantizer sees, and those values in v: with the
// rotation, y_i = fl(v_i r) for r = fl32(1/sqrt(d)); fl32 rounding is
// monotone, so the max of fl(|v_i| r) is fl(max|v_i| r).
template <int D, bool ROTATE>
__device__ __forceinline__ float finish_block(float (&v)[32]) {
#pragma clang fp contract(off)
  constexpr float kRotScale = (D == 128) ? 0x1.6a09e6p-4f : 0x1p-3f;  // fl32(1/sqrt(d))
  float mraw = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) mraw = fmaxf(mraw, fabsf(v[i]));
  if constexpr (ROTATE) {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] *= kRotScale;
    return mraw * kRotScale;
  }
  return mraw;
}

}  // namespace mxblock
}  // namespace mxattn_internal
