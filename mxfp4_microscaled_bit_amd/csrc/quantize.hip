// MXFP4 quantizers of MXAttention for gfx950 (MI355X).
//
//   k_quantize_headdim: Q and K.  Optional Hadamard rotation along the head
//     dimension (MXAttention paper, Sec. 4.3, Alg. 2 steps 3-4), then UOS or
//     OCP block quantization of every 32 consecutive channels (Alg. 1; Alg. 2
//     steps 5-6).
//   k_quantize_tokens: V.  Block quantization along tokens, 32 consecutive
//     tokens of one channel per block (Alg. 2 step 7, with the block axis that
//     the PV product contracts over, as the MatX leaky-quantization page
//     explains).
//
// Both kernels are HBM-bandwidth bound: 2 bytes read and 0.5 + 1/32 bytes
// written per element.
//
// Numerics follow the bit-exact contract of include/mxattn.h:
//   rotation: binary32 butterflies with strides 1, 2, ..., d/2, then one
//             multiply by fl32(1/sqrt(d));
//   scale:    UOS e = ceil(log2(M / 7.25)), OCP e = floor(log2 M) - 2, read
//             off the binary32 bit pattern of M; clamped to [-127, 127];
//   elements: round to nearest E2M1 value, ties to the even code, saturating
//             at 6, sign bit kept for values that round to zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace mxattn_internal {
namespace {

constexpr int kRuleUos = 0;
constexpr int kRuleOcp = 1;

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
//        whose fraction field is 0x680000).
// A zero block gets 0 (scale 1); a subnormal M needs e <= -129, which the
// E8M0 range clamps to -127.
template <int RULE>
__device__ __forceinline__ int scale_exponent(float M) {
  const uint32_t b = __float_as_uint(M);
  if (b == 0u) return 0;
  const int E = (int)(b >> 23);
  if (E == 0) return -127;
  int e = E - 129;
  if constexpr (RULE == kRuleUos) e += ((b & 0x7FFFFFu) > 0x680000u) ? 1 : 0;
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
  float sc = pow2f(e < -126 ? 0 : e);
  if (e < -126) {
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = __builtin_amdgcn_ldexpf(y[i], 127);
  }
  return make_uint4(cvt8(y, sc), cvt8(y + 8, sc), cvt8(y + 16, sc), cvt8(y + 24, sc));
}

// One lane owns one 32-channel block of one row (d/32 lanes per row, in the
// same quad), so the first five butterfly stages stay in registers and the
// remaining one (d=64) or two (d=128) cross lanes through DPP.  Each thread
// handles two rows-blocks 256 lanes apart so that two 64-byte loads are in
// flight per lane.
template <int D, int DTYPE, bool ROTATE, int RULE>
__global__ __launch_bounds__(256) void k_quantize_headdim(
    const uint16_t* __restrict__ x, int H, int N, int Np, int64_t sB, int64_t sH, int64_t sN,
    int64_t total_units, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int BPR = D / 32;  // blocks (lanes) per row
  constexpr float kRotScale = (D == 128) ? 0x1.6a09e6p-4f : 0x1p-3f;  // fl32(1/sqrt(d))
  static_assert(D == 64 || D == 128, "head dim");

  uint4 raw[2][4];
  int64_t unit[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    unit[it] = (int64_t)blockIdx.x * 512 + it * 256 + threadIdx.x;
    const int64_t row = unit[it] / BPR;
    const int blk = (int)(unit[it] % BPR);
    const int64_t bh = row / Np;
    const int n = (int)(row % Np);
    const bool live = unit[it] < total_units && n < N;
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[it][k] = make_uint4(0, 0, 0, 0);
    if (live) {
      const int64_t b = bh / H, h = bh % H;
      const uint4* p = reinterpret_cast<const uint4*>(x + b * sB + h * sH + (int64_t)n * sN + 32 * blk);
#pragma unroll
      for (int k = 0; k < 4; ++k) raw[it][k] = p[k];
    }
  }

#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int blk = (int)(unit[it] % BPR);
    float v[32];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      unpack2<DTYPE>(raw[it][k].x, v[8 * k + 0], v[8 * k + 1]);
      unpack2<DTYPE>(raw[it][k].y, v[8 * k + 2], v[8 * k + 3]);
      unpack2<DTYPE>(raw[it][k].z, v[8 * k + 4], v[8 * k + 5]);
      unpack2<DTYPE>(raw[it][k].w, v[8 * k + 6], v[8 * k + 7]);
    }
    if constexpr (ROTATE) {
      // butterflies of stride 1, 2, 4, 8, 16 inside the lane
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
      // stride 32 pairs this lane with lane^1, stride 64 with lane^2: the lane
      // holding the first element keeps a + b, the other b_partner - own,
      // written as partner + (-own) with the sign flipped by XOR.
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
    // block max of the (rotated) values; fl32 rounding is monotone, so the
    // max of fl(|v_i| r) is fl(max|v_i| r)
    float mraw = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mraw = fmaxf(mraw, fabsf(v[i]));
    const float M = ROTATE ? mraw * kRotScale : mraw;
    const int e = scale_exponent<RULE>(M);

    // y_i = fl(v_i r), then the exact division by 2^e inside the convert
    if constexpr (ROTATE) {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] *= kRotScale;
    }
    const uint4 packed = block_codes(v, e);
    if (unit[it] < total_units) {
      reinterpret_cast<uint4*>(codes)[unit[it]] = packed;
      scales[unit[it]] = (uint8_t)(e + 127);
    }
  }
}

// One lane owns two adjacent channels of one 32-token block: it reads the 32
// tokens of its channel pair (each wave-wide load is one contiguous row of the
// block), so both block maxima are lane-local, and writes 2 x 16 code bytes
// and 2 scale bytes contiguously.
template <int D, int DTYPE, int RULE>
__global__ __launch_bounds__(256) void k_quantize_tokens(
    const uint16_t* __restrict__ x, int H, int N, int NBp, int64_t sB, int64_t sH, int64_t sN,
    int64_t total_blocks, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int LPB = D / 2;  // lanes per token block
  const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t gblk = gl / LPB;
  const int cp = (int)(gl % LPB);
  if (gblk >= total_blocks) return;
  const int64_t bh = gblk / NBp;
  const int kb = (int)(gblk % NBp);
  const int64_t b = bh / H, h = bh % H;
  const uint16_t* base = x + b * sB + h * sH + (int64_t)(32 * kb) * sN + 2 * cp;

  // all 32 loads are issued before any is used; only a block that crosses N
  // (the last one) takes the guarded path, decided once per wave
  uint32_t w[32];
  if (__all(32 * kb + 31 < N)) {
    const uint16_t* pt = base;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      w[t] = *reinterpret_cast<const uint32_t*>(pt);
      pt += sN;
    }
  } else {
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int tc = min(t, max(N - 1 - 32 * kb, 0));  // an in-range row to read from
      const uint32_t wt = *reinterpret_cast<const uint32_t*>(base + (int64_t)tc * sN);
      w[t] = (32 * kb + t < N) ? wt : 0u;
    }
  }
  float v0[32], v1[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) unpack2<DTYPE>(w[t], v0[t], v1[t]);
  float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    m0 = fmaxf(m0, fabsf(v0[t]));
    m1 = fmaxf(m1, fabsf(v1[t]));
  }
  const int e0 = scale_exponent<RULE>(m0), e1 = scale_exponent<RULE>(m1);
  uint4* dst = reinterpret_cast<uint4*>(codes + (gblk * D + 2 * cp) * 16);
  dst[0] = block_codes(v0, e0);
  dst[1] = block_codes(v1, e1);
  *reinterpret_cast<uint16_t*>(scales + gblk * D + 2 * cp) =
      (uint16_t)((uint32_t)(e0 + 127) | ((uint32_t)(e1 + 127) << 8));
}

template <int D, int DTYPE, bool ROTATE, int RULE>
hipError_t launch_hd(const QuantArgs& a, hipStream_t stream) {
  const int64_t Np = padded_tokens(a.N);
  const int64_t total = (int64_t)a.B * a.H * Np * (D / 32);
  const int64_t grid = (total + 511) / 512;
  hipLaunchKernelGGL((k_quantize_headdim<D, DTYPE, ROTATE, RULE>), dim3((unsigned)grid), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(a.x), a.H, a.N, (int)Np, a.sB, a.sH, a.sN,
                     total, a.codes, a.scales);
  return hipGetLastError();
}

template <int D, int DTYPE, int RULE>
hipError_t launch_tok(const QuantArgs& a, hipStream_t stream) {
  const int64_t NBp = padded_tokens(a.N) / 32;
  const int64_t total_blocks = (int64_t)a.B * a.H * NBp;
  const int64_t lanes = total_blocks * (D / 2);
  const int64_t grid = (lanes + 255) / 256;
  hipLaunchKernelGGL((k_quantize_tokens<D, DTYPE, RULE>), dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.x), a.H, a.N, (int)NBp, a.sB, a.sH, a.sN,
                     total_blocks, a.codes, a.scales);
  return hipGetLastError();
}

template <int D, int DTYPE>
hipError_t dispatch_hd_rule(const QuantArgs& a, hipStream_t s) {
  if (a.rotate) return a.rule == kRuleOcp ? launch_hd<D, DTYPE, true, kRuleOcp>(a, s)
                                          : launch_hd<D, DTYPE, true, kRuleUos>(a, s);
  return a.rule == kRuleOcp ? launch_hd<D, DTYPE, false, kRuleOcp>(a, s)
                            : launch_hd<D, DTYPE, false, kRuleUos>(a, s);
}

template <int D, int DTYPE>
hipError_t dispatch_tok_rule(const QuantArgs& a, hipStream_t s) {
  return a.rule == kRuleOcp ? launch_tok<D, DTYPE, kRuleOcp>(a, s) : launch_tok<D, DTYPE, kRuleUos>(a, s);
}

}  // namespace

hipError_t launch_quantize_headdim(const QuantArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.dtype == 1 ? dispatch_hd_rule<128, 1>(a, stream) : dispatch_hd_rule<128, 0>(a, stream);
  return a.dtype == 1 ? dispatch_hd_rule<64, 1>(a, stream) : dispatch_hd_rule<64, 0>(a, stream);
}

hipError_t launch_quantize_tokens(const QuantArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.dtype == 1 ? dispatch_tok_rule<128, 1>(a, stream) : dispatch_tok_rule<128, 0>(a, stream);
  return a.dtype == 1 ? dispatch_tok_rule<64, 1>(a, stream) : dispatch_tok_rule<64, 0>(a, stream);
}

}  // namespace mxattn_internal
