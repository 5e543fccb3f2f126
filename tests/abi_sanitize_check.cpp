// abi_sanitize_check.cpp -- test infrastructure for the C-ABI layer (api.cpp).
//
// Host-only driver: links api.cpp against stub kernel launchers that abort
// if reached, then calls every entry point with arguments that validation
// must reject (null, misaligned and overlarge arguments, bad enums,
// mismatched descriptors, short workspaces) and the size helpers with
// extreme shapes.  tests/ builds it with the host sanitizers
// (AddressSanitizer + UndefinedBehaviorSanitizer) and runs it on the CPU: no
// call may reach a launcher, and no validation path may overflow or read out
// of bounds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "internal.h"
#include "mxattn.h"

namespace mxattn_internal {
static hipError_t reached(const char* what) {
  fprintf(stderr, "validation let a call through to %s\n", what);
  abort();
}
hipError_t launch_quantize_headdim(const QuantArgs&, hipStream_t) { return reached("launch_quantize_headdim"); }
hipError_t launch_quantize_tokens(const QuantArgs&, hipStream_t) { return reached("launch_quantize_tokens"); }
hipError_t launch_quantize_qkv(const QuantArgs&, const QuantArgs&, const QuantArgs&, hipStream_t) {
  return reached("launch_quantize_qkv");
}
int sweep_chunks(int axis, int N, int d) {
  const int64_t units = axis == 1 ? (int64_t)((N + 31) / 32) * (d / 2) : (int64_t)N * (d / 32);
  return (int)((units + 1023) / 1024);
}
hipError_t launch_scale_sweep(const SweepArgs&, hipStream_t) { return reached("launch_scale_sweep"); }
hipError_t launch_scale_sweep_static(const SweepArgs&, hipStream_t) { return reached("launch_scale_sweep_static"); }
hipError_t launch_attention(const AttnArgs&, hipStream_t) { return reached("launch_attention"); }
}  // namespace mxattn_internal

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  uint8_t* const F = reinterpret_cast<uint8_t*>(static_cast<uintptr_t>(0x100000));  // never dereferenced
  const mxattn_shape ok = {1, 2, 64, 64};
  const int32_t big = 0x7FFFFFFF;
  const mxattn_shape extremes[] = {{big, big, big, 128}, {1, 1, big, 64}, {big, 1, 1, 128}, {1, big, 128, 64},
                                   {-1, 1, 1, 64},       {1, 1, -5, 128}, {0, 0, 0, 0},       {1, 1, 1, 96}};
  for (const mxattn_shape& s : extremes) {
    for (int axis = 0; axis < 3; ++axis) {
      expect((int)mxattn_mx_codes_bytes(s, axis), 0, "codes_bytes of an invalid shape");
      expect((int)mxattn_mx_scales_bytes(s, axis), 0, "scales_bytes of an invalid shape");
      expect((int)mxattn_scale_sweep_workspace_bytes(s, axis, 3), 0, "sweep workspace of an invalid shape");
    }
    for (int pm = 0; pm < 3; ++pm)
      expect((int)mxattn_reference_modes_workspace_bytes(s, pm), 0, "reference workspace of an invalid shape");
    expect((int)mxattn_p_diagnostics_workspace_bytes(s), 0, "diagnostics workspace of an invalid shape");
  }

  // the element limit: B H Np d = 2^36 is accepted, one more head is not
  const mxattn_shape at_limit = {1, 8192, 65536, 128}, past_limit = {1, 8193, 65536, 128};
  if (mxattn_mx_codes_bytes(at_limit, 0) != ((size_t)1 << 35)) {
    fprintf(stderr, "codes_bytes at the 2^36-element limit: %zu\n", mxattn_mx_codes_bytes(at_limit, 0));
    ++failures;
  }
  expect((int)mxattn_mx_codes_bytes(past_limit, 0), 0, "codes_bytes past the element limit");

  mxattn_mx_tensor out = {F, F + 4096, {0, 0, 0, 0}, 5, 5, 5};
  expect(mxattn_rotate_quantize(nullptr, 0, ok, nullptr, 0, 1, 0, &out, nullptr), MXATTN_ERR_NULL, "rq null x");
  expect(mxattn_rotate_quantize(F, 0, extremes[0], nullptr, 0, 1, 0, &out, nullptr), MXATTN_ERR_SHAPE, "rq shape");
  expect(mxattn_rotate_quantize(F + 8, 0, ok, nullptr, 0, 1, 0, &out, nullptr), MXATTN_ERR_ALIGN, "rq align");
  const int64_t bad_strides[3] = {INT64_MAX, -8, 12};
  expect(mxattn_rotate_quantize(F, 0, ok, bad_strides, 0, 1, 0, &out, nullptr), MXATTN_ERR_STRIDE, "rq strides");
  expect(mxattn_rotate_quantize(F, 0, ok, nullptr, 1, 1, 0, &out, nullptr), MXATTN_ERR_ENUM, "rq rotate tokens");
  expect(mxattn_rotate_quantize(F, 0, ok, nullptr, 0, 1, 9, &out, nullptr), MXATTN_ERR_ENUM, "rq rule");
  expect(mxattn_rotate_quantize_q(F, 0, ok, nullptr, 0, 1, 1e308, &out, nullptr), MXATTN_ERR_ENUM, "rq_q q");
  expect(mxattn_rotate_quantize_q(F, 0, ok, nullptr, 0, 1, -0.0, &out, nullptr), MXATTN_ERR_ENUM, "rq_q q<0");
  if (out.axis != 5 || out.rule != 5 || out.rotated != 5) {
    fprintf(stderr, "a rejected call wrote the descriptor\n");
    ++failures;
  }

  mxattn_mx_tensor o3[3] = {out, out, out};
  expect(mxattn_rotate_quantize_qkv(F, F, F, 0, ok, ok, nullptr, nullptr, nullptr, 1, 2, &o3[0], &o3[1], &o3[2],
                                    nullptr),
         MXATTN_ERR_ENUM, "qkv rule");
  const mxattn_shape other = {2, 2, 64, 64};
  expect(mxattn_rotate_quantize_qkv(F, F, F, 0, ok, other, nullptr, nullptr, nullptr, 1, 0, &o3[0], &o3[1], &o3[2],
                                    nullptr),
         MXATTN_ERR_MISMATCH, "qkv shapes");

  const double qs[3] = {6.0, 7.25, 13.0};  // 13 > 2 * 6: rejected
  double* sse = reinterpret_cast<double*>(F);
  expect(mxattn_scale_sweep(F, 0, ok, nullptr, 0, 1, qs, 3, sse, F, 1 << 20, nullptr), MXATTN_ERR_ENUM,
         "sweep boundary spread");
  expect(mxattn_scale_sweep(F, 0, ok, nullptr, 0, 1, qs, 2, sse, F, 0, nullptr), MXATTN_ERR_WORKSPACE,
         "sweep workspace");
  expect(mxattn_scale_sweep(F, 0, ok, nullptr, 0, 1, qs, 1000, sse, F, 1 << 20, nullptr), MXATTN_ERR_ENUM,
         "sweep count");
  // the allocation-free sweep: the same validation, then the static scratch limit
  expect(mxattn_scale_sweep_noalloc(F, 0, ok, nullptr, 0, 1, qs, 3, sse, nullptr), MXATTN_ERR_ENUM,
         "noalloc sweep boundary spread");
  expect(mxattn_scale_sweep_noalloc(F, 0, ok, nullptr, 0, 1, qs, 1000, sse, nullptr), MXATTN_ERR_ENUM,
         "noalloc sweep count");
  expect(mxattn_scale_sweep_noalloc(nullptr, 0, ok, nullptr, 0, 1, qs, 2, sse, nullptr), MXATTN_ERR_NULL,
         "noalloc sweep input");
  expect(mxattn_scale_sweep_noalloc(F, 7, ok, nullptr, 0, 1, qs, 2, sse, nullptr), MXATTN_ERR_DTYPE,
         "noalloc sweep dtype");
  expect(mxattn_scale_sweep_noalloc(F, 0, ok, nullptr, 1, 1, qs, 2, sse, nullptr), MXATTN_ERR_ENUM,
         "noalloc sweep rotation along tokens");
  {
    const mxattn_shape big = {64, 64, 118800, 128};  // 731 MB of partial sums with 48 boundaries
    double q48[48];
    for (int j = 0; j < 48; ++j) q48[j] = 6.0 + 0.04 * j;
    expect(mxattn_scale_sweep_noalloc(F, 0, big, nullptr, 0, 1, q48, 48, sse, nullptr), MXATTN_ERR_SCRATCH,
           "noalloc sweep beyond the static scratch");
    if (mxattn_scale_sweep_workspace_bytes(big, 0, 48) <= (size_t)MXATTN_SWEEP_SCRATCH_BYTES) {
      fprintf(stderr, "the oversize case fits the scratch\n");
      ++failures;
    }
  }
  expect(mxattn_scale_sweep_noalloc(F + 1, 0, ok, nullptr, 0, 1, qs, 2, sse, nullptr), MXATTN_ERR_ALIGN,
         "noalloc sweep alignment");

  mxattn_mx_tensor q = {F, F, ok, MXATTN_AXIS_HEAD_DIM, 0, 1}, k = q, v = q;
  v.axis = MXATTN_AXIS_TOKEN;
  float* o = reinterpret_cast<float*>(F);
  expect(mxattn_forward(&q, &k, &q, 0, o, nullptr, nullptr), MXATTN_ERR_MISMATCH, "forward v axis");
  k.rotated = 0;
  expect(mxattn_forward(&q, &k, &v, 0, o, nullptr, nullptr), MXATTN_ERR_MISMATCH, "forward rotation");
  k.rotated = 1;
  expect(mxattn_forward(&q, &k, &v, 3, o, nullptr, nullptr), MXATTN_ERR_ENUM, "forward causal flag");
  expect(mxattn_forward(&q, &k, &v, 0, reinterpret_cast<float*>(F + 4), nullptr, nullptr), MXATTN_ERR_ALIGN,
         "forward out align");
  mxattn_mx_tensor kc = k;
  kc.shape.N = 65;
  mxattn_mx_tensor vc = v;
  vc.shape.N = 65;
  expect(mxattn_forward(&q, &kc, &vc, 1, o, nullptr, nullptr), MXATTN_ERR_MISMATCH, "forward causal cross");
  expect(mxattn_forward_fused_q(F, 3, ok, nullptr, &k, &v, 0, o, nullptr, nullptr), MXATTN_ERR_DTYPE,
         "fused dtype");
  kc = k;
  kc.rule = MXATTN_SCALE_CEIL_Q;
  expect(mxattn_forward_fused_q(F, 0, ok, nullptr, &kc, &v, 0, o, nullptr, nullptr), MXATTN_ERR_ENUM, "fused rule");

  expect(mxattn_quantize_reference_modes(F, F, F, 0, ok, nullptr, 0, 7, 1, 0, o, nullptr, F, 1 << 30, nullptr),
         MXATTN_ERR_ENUM, "reference mode");
  expect(mxattn_quantize_reference_modes(F, F, F, 0, ok, nullptr, 0, 2, 1, 0, o, nullptr, F, 16, nullptr),
         MXATTN_ERR_WORKSPACE, "reference workspace");
  expect(mxattn_p_diagnostics(F, F, 0, ok, nullptr, 0, 1, 0, 0x1p30f, o, F, 1 << 30, nullptr), MXATTN_ERR_ENUM,
         "diagnostics gamma");
  expect(mxattn_p_diagnostics(F, F, 0, ok, nullptr, 0, 1, 0, 1.0f, o, F, 8, nullptr), MXATTN_ERR_WORKSPACE,
         "diagnostics workspace");
  for (int st = 0; st < 16; ++st)
    if (!mxattn_status_string(static_cast<mxattn_status>(st))) ++failures;

  if (failures) {
    fprintf(stderr, "%d unexpected results\n", failures);
    return 1;
  }
  printf("ABI sanitizer run: ok\n");
  return 0;
}
