// In-run throughput probes for the benchmark's roofline figures on gfx950.
// Measurement infrastructure, built into its own library (libmxprobe.so),
// not part of libmxattn's ABI.
//
//   mxprobe_mfma_fp4:  back-to-back scaled-FP4 32x32x64 matrix products, four
//                      independent accumulators per wave, on every SIMD: the
//                      matrix-core rate this GPU reaches at its current clock
//                      and power state.
//   mxprobe_pair_mix:  the fused forward's vector work per (query, key) pair --
//                      one FMA for the exponent argument, one v_exp_f32, half a
//                      v_cvt_scalef32_pk_fp4_f32 and half a v_max3_f32 -- on 16
//                      independent chains per lane, at two waves per SIMD (the
//                      forward's occupancy at d = 128): the vector-unit ceiling
//                      for the forward in pairs per second.
//   mxprobe_stream:    four 16-byte reads and writes per lane over large
//                      buffers: achievable HBM read+write bandwidth.
//   mxprobe_read:      four 16-byte reads per lane (and one 4-byte write):
//                      achievable HBM read bandwidth.
//
// Each call enqueues one launch on `stream` and returns a hipError_t; the
// caller times it with events.  Workgroups: 256 threads (one wave per SIMD
// per workgroup).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Four independent 32x32x64 FP4 accumulators; `iters` rounds of four
// products.  The operands are register constants; the sum of the results is
// written so that nothing is removed.  2 * 32 * 32 * 64 flops per product.
__global__ __launch_bounds__(256) void k_mfma_fp4(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const v8i a = {lane * 0x01010101, lane * 0x02020202, 0x11111111, 0x22222222, 0, 0, 0, 0};
  const v8i b = {0x33333333, lane * 0x01020304, 0x44444444, 0x12345678, 0, 0, 0, 0};
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 4, 4, 0, 120, 0, 120);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 4, 4, 0, 120, 0, 120);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 4, 4, 0, 120, 0, 120);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 4, 4, 0, 120, 0, 120);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// 16 chains per lane; per round and chain: two pairs, i.e. two FMAs, two
// exponentials, one FP4 convert of the two results and one max3 over the two
// arguments.  Each exponential feeds the next round's FMA of its pair, so the
// chains carry no other instruction.
__global__ __launch_bounds__(256, 2) void k_pair_mix(int iters, float c, float* __restrict__ out) {
  float y0[16], y1[16], m[16];
  uint32_t w[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    y0[k] = 0.001f * (float)(threadIdx.x + 7 * k);
    y1[k] = 0.002f * (float)(threadIdx.x + 5 * k);
    m[k] = -1.0f;
    w[k] = 0u;
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float a0 = fmaf(y0[k], c, -0.25f);
      const float a1 = fmaf(y1[k], c, -0.5f);
      y0[k] = __builtin_amdgcn_exp2f(a0);
      y1[k] = __builtin_amdgcn_exp2f(a1);
      w[k] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[k], y0[k], y1[k], 1.0f, 0);
      m[k] = __builtin_fmaxf(__builtin_fmaxf(m[k], a0), a1);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += y0[k] + y1[k] + m[k] + (float)(w[k] & 0xFu);
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Four 16-byte elements per lane, each read and written (one bit flipped);
// one pass, the grid covering the buffer.
__global__ __launch_bounds__(256) void k_stream(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  const int64_t i0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (i0 + 256 * u < n) v[u] = src[i0 + 256 * u];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (i0 + 256 * u < n) {
      v[u].x ^= 1u;
      dst[i0 + 256 * u] = v[u];
    }
}

// Reads four 16-byte elements per lane and writes one 4-byte word per lane:
// read bandwidth (the written bytes are 1/64 of the read ones).
__global__ __launch_bounds__(256) void k_read(const uint4* __restrict__ src, uint32_t* __restrict__ dst, int64_t n) {
  const int64_t i0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  uint32_t acc = 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (i0 + 256 * u < n) {
      const uint4 v = src[i0 + 256 * u];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  dst[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// `groups` workgroups of 256 threads, `iters` rounds; out: groups * 256 floats.
hipError_t mxprobe_mfma_fp4(int groups, int iters, float* out, hipStream_t stream) {
  if (groups < 1 || iters < 1 || !out) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_fp4, dim3(groups), dim3(256), 0, stream, iters, out);
  return hipGetLastError();
}

// `groups` workgroups of 256 threads at two waves per SIMD, `iters` rounds of
// 32 pairs per lane; out: groups * 256 floats.
hipError_t mxprobe_pair_mix(int groups, int iters, float* out, hipStream_t stream) {
  if (groups < 1 || iters < 1 || !out) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_pair_mix, dim3(groups), dim3(256), 0, stream, iters, 0x1.0527dcp-3f, out);
  return hipGetLastError();
}

// n16 16-byte elements of src copied (with one bit flipped) to dst.
hipError_t mxprobe_stream(const void* src, void* dst, int64_t n16, hipStream_t stream) {
  if (!src || !dst || n16 < 1) return hipErrorInvalidValue;
  const int64_t groups = (n16 + 1023) / 1024;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream, dim3((unsigned)groups), dim3(256), 0, stream, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

// n16 16-byte elements of src read; dst receives ceil(n16 / 1024) * 256 words.
hipError_t mxprobe_read(const void* src, void* dst, int64_t n16, hipStream_t stream) {
  if (!src || !dst || n16 < 1) return hipErrorInvalidValue;
  const int64_t groups = (n16 + 1023) / 1024;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read, dim3((unsigned)groups), dim3(256), 0, stream, static_cast<const uint4*>(src),
                     static_cast<uint32_t*>(dst), n16);
  return hipGetLastError();
}

}  // extern "C"
