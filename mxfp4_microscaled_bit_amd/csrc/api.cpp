// C ABI of libmxattn (include/mxattn.h): argument validation, buffer sizes
// and dispatch to the HIP kernels.  Nothing here allocates device memory or
// keeps state between calls.
#include "mxattn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "internal.h"

using namespace mxattn_internal;

static_assert(kSweepMax == MXATTN_SWEEP_MAX, "sweep capacity of the kernels and the header");

namespace {

// At most 2^36 elements per tensor (B H Np d): every launch then stays within
// the 32-bit work-item count of a dispatch (the forward launches B H Np / 128
// workgroups of 256 threads, at most 2^31 work-items; the head-dim quantizer
// one thread per 32 elements), and 64-bit indexes have ample room.
constexpr int64_t kMaxElems = (int64_t)1 << 36;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mxattn_status check_shape(const mxattn_shape& s) {
  if (s.B < 1 || s.H < 1 || s.N < 1) return MXATTN_ERR_SHAPE;
  if (s.d != 64 && s.d != 128) return MXATTN_ERR_SHAPE;
  const int64_t Np = padded_tokens(s.N);
  if ((int64_t)s.B * s.H > ((int64_t)1 << 30) / (Np / kTokenAlign)) return MXATTN_ERR_SHAPE;
  if ((int64_t)s.B * s.H * Np * s.d > kMaxElems) return MXATTN_ERR_SHAPE;
  return MXATTN_OK;
}

bool same_shape(const mxattn_shape& a, const mxattn_shape& b) {
  return a.B == b.B && a.H == b.H && a.N == b.N && a.d == b.d;
}

// element strides of the B, H, N dimensions (d is contiguous)
mxattn_status resolve_strides(const mxattn_shape& s, const int64_t* strides, int64_t out[3]) {
  if (!strides) {
    out[2] = s.d;
    out[1] = (int64_t)s.N * s.d;
    out[0] = (int64_t)s.H * s.N * s.d;
    return MXATTN_OK;
  }
  for (int i = 0; i < 3; ++i) {
    if (strides[i] < 0 || (strides[i] & 7) != 0) return MXATTN_ERR_STRIDE;
    out[i] = strides[i];
  }
  // rows of one (b, h) must not overlap inside a row
  if (s.N > 1 && out[2] < s.d) return MXATTN_ERR_STRIDE;
  return MXATTN_OK;
}

size_t codes_bytes(const mxattn_shape& s, int axis) {
  const int64_t Np = padded_tokens(s.N);
  (void)axis;  // both axes: d/2 bytes per padded token
  return (size_t)((int64_t)s.B * s.H * Np * (s.d / 2));
}

size_t scales_bytes(const mxattn_shape& s, int axis) {
  const int64_t Np = padded_tokens(s.N);
  (void)axis;  // both axes: d/32 bytes per padded token
  return (size_t)((int64_t)s.B * s.H * Np * (s.d / 32));
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

mxattn_status hip_status(hipError_t e) { return e == hipSuccess ? MXATTN_OK : MXATTN_ERR_HIP; }

// a ceiling-rule boundary: finite, in [MXATTN_Q_MIN, MXATTN_Q_MAX]
bool boundary_ok(double q) { return isfinite(q) && q >= MXATTN_Q_MIN && q <= MXATTN_Q_MAX; }

// binary32 bits of the largest binary32 number <= q: for a binary32 M,
// M <= q 2^e holds exactly when it holds with this number in place of q
uint32_t boundary_bits(double q) {
  float f = (float)q;
  if ((double)f > q) f = nextafterf(f, 0.0f);
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  return b;
}

// validation and arguments of one quantizer tensor; launches nothing and
// writes nothing
mxattn_status prepare_quantize(const void* x, int32_t dtype, mxattn_shape shape, const int64_t* strides,
                               int32_t axis, int32_t rotate, int32_t rule, uint32_t qbits,
                               const mxattn_mx_tensor* out, QuantArgs& a) {
  if (!x || !out || !out->codes || !out->scales) return MXATTN_ERR_NULL;
  if (dtype != MXATTN_BF16 && dtype != MXATTN_FP16) return MXATTN_ERR_DTYPE;
  if (axis != MXATTN_AXIS_HEAD_DIM && axis != MXATTN_AXIS_TOKEN) return MXATTN_ERR_ENUM;
  if (rotate != 0 && rotate != 1) return MXATTN_ERR_ENUM;
  if (rotate && axis != MXATTN_AXIS_HEAD_DIM) return MXATTN_ERR_ENUM;
  mxattn_status st = check_shape(shape);
  if (st != MXATTN_OK) return st;
  int64_t s[3];
  st = resolve_strides(shape, strides, s);
  if (st != MXATTN_OK) return st;
  if (!aligned16(x) || !aligned16(out->codes) || !aligned16(out->scales)) return MXATTN_ERR_ALIGN;

  a.x = x;
  a.dtype = dtype;
  a.B = shape.B; a.H = shape.H; a.N = shape.N; a.d = shape.d;
  a.sB = s[0]; a.sH = s[1]; a.sN = s[2];
  a.rotate = rotate;
  a.rule = rule;
  a.qbits = qbits;
  a.codes = out->codes;
  a.scales = out->scales;
  return MXATTN_OK;
}

void describe(mxattn_mx_tensor* out, const mxattn_shape& shape, int32_t axis, int32_t rule, int32_t rotate) {
  out->shape = shape;
  out->axis = axis;
  out->rule = rule;
  out->rotated = rotate;
}

mxattn_status quantize_common(const void* x, int32_t dtype, mxattn_shape shape, const int64_t* strides,
                              int32_t axis, int32_t rotate, int32_t rule, uint32_t qbits,
                              mxattn_mx_tensor* out, hipStream_t stream) {
  QuantArgs a;
  const mxattn_status st = prepare_quantize(x, dtype, shape, strides, axis, rotate, rule, qbits, out, a);
  if (st != MXATTN_OK) return st;
  describe(out, shape, axis, rule, rotate);
  return hip_status(axis == MXATTN_AXIS_HEAD_DIM ? launch_quantize_headdim(a, stream)
                                                 : launch_quantize_tokens(a, stream));
}

mxattn_status check_mx(const mxattn_mx_tensor* t, int axis) {
  if (!t || !t->codes || !t->scales) return MXATTN_ERR_NULL;
  if (t->axis != axis) return MXATTN_ERR_MISMATCH;
  mxattn_status st = check_shape(t->shape);
  if (st != MXATTN_OK) return st;
  if (!aligned16(t->codes) || !aligned16(t->scales)) return MXATTN_ERR_ALIGN;
  return MXATTN_OK;
}

// checks shared by the two forward entry points; q_shape / q_rotated
// describe Q^ (or, fused, the Q it is made from)
mxattn_status check_forward(const mxattn_shape& q_shape, int32_t q_rotated, const mxattn_mx_tensor* k,
                            const mxattn_mx_tensor* v, int32_t causal, const float* out, const float* row_stats) {
  if (!out) return MXATTN_ERR_NULL;
  mxattn_status st = check_mx(k, MXATTN_AXIS_HEAD_DIM);
  if (st != MXATTN_OK) return st;
  st = check_mx(v, MXATTN_AXIS_TOKEN);
  if (st != MXATTN_OK) return st;
  // K^ and V^ share one shape; Q may have another token count
  // (cross-attention) but the same B, H and d
  if (!same_shape(k->shape, v->shape)) return MXATTN_ERR_MISMATCH;
  if (q_shape.B != k->shape.B || q_shape.H != k->shape.H || q_shape.d != k->shape.d) return MXATTN_ERR_MISMATCH;
  if ((q_rotated != 0) != (k->rotated != 0)) return MXATTN_ERR_MISMATCH;
  if (causal != 0 && causal != 1) return MXATTN_ERR_ENUM;
  if (causal && q_shape.N != k->shape.N) return MXATTN_ERR_MISMATCH;
  if (!aligned16(out) || (row_stats && !aligned16(row_stats))) return MXATTN_ERR_ALIGN;
  return MXATTN_OK;
}

AttnArgs forward_args(const mxattn_shape& q_shape, const mxattn_mx_tensor* k, const mxattn_mx_tensor* v,
                      int32_t causal, float* out, float* row_stats) {
  AttnArgs a;
  a.qc = nullptr; a.qs = nullptr;
  a.kc = k->codes; a.ks = k->scales;
  a.vc = v->codes; a.vs = v->scales;
  a.B = q_shape.B; a.H = q_shape.H; a.N = q_shape.N; a.d = q_shape.d;
  a.Nk = k->shape.N;
  a.causal = causal;
  a.mode = kModePnq;
  a.rule = MXATTN_SCALE_UOS;
  a.out = out;
  a.row_stats = row_stats;
  a.row_sums = nullptr;
  a.stats_ws = nullptr;
  a.diag = nullptr;
  a.gamma = 1.0f;
  return a;
}

}  // namespace

extern "C" {

size_t mxattn_mx_codes_bytes(mxattn_shape shape, int32_t axis) {
  if (check_shape(shape) != MXATTN_OK || (axis != MXATTN_AXIS_HEAD_DIM && axis != MXATTN_AXIS_TOKEN)) return 0;
  return codes_bytes(shape, axis);
}

size_t mxattn_mx_scales_bytes(mxattn_shape shape, int32_t axis) {
  if (check_shape(shape) != MXATTN_OK || (axis != MXATTN_AXIS_HEAD_DIM && axis != MXATTN_AXIS_TOKEN)) return 0;
  return scales_bytes(shape, axis);
}

int32_t mxattn_forward_kv_tile(int32_t d, int32_t causal) {
  (void)causal;
  return (d == 64 || d == 128) ? kKvTile : 0;
}

mxattn_status mxattn_rotate_quantize(const void* x, int32_t dtype, mxattn_shape shape,
                                     const int64_t* strides, int32_t axis, int32_t rotate,
                                     int32_t rule, mxattn_mx_tensor* out, hipStream_t stream) {
  if (x && out && out->codes && out->scales && dtype >= 0 && dtype <= 1 &&
      rule != MXATTN_SCALE_UOS && rule != MXATTN_SCALE_OCP)
    return MXATTN_ERR_ENUM;
  return quantize_common(x, dtype, shape, strides, axis, rotate, rule, 0u, out, stream);
}

mxattn_status mxattn_rotate_quantize_q(const void* x, int32_t dtype, mxattn_shape shape,
                                       const int64_t* strides, int32_t axis, int32_t rotate,
                                       double q_max, mxattn_mx_tensor* out, hipStream_t stream) {
  if (x && out && out->codes && out->scales && dtype >= 0 && dtype <= 1 && !boundary_ok(q_max))
    return MXATTN_ERR_ENUM;
  return quantize_common(x, dtype, shape, strides, axis, rotate, MXATTN_SCALE_CEIL_Q, boundary_bits(q_max), out,
                         stream);
}

mxattn_status mxattn_rotate_quantize_qkv(const void* q, const void* k, const void* v, int32_t dtype,
                                         mxattn_shape q_shape, mxattn_shape kv_shape, const int64_t* q_strides,
                                         const int64_t* k_strides, const int64_t* v_strides, int32_t rotate,
                                         int32_t rule, mxattn_mx_tensor* q_out, mxattn_mx_tensor* k_out,
                                         mxattn_mx_tensor* v_out, hipStream_t stream) {
  if (!q_out || !k_out || !v_out) return MXATTN_ERR_NULL;
  QuantArgs aq, ak, av;
  mxattn_status st =
      prepare_quantize(q, dtype, q_shape, q_strides, MXATTN_AXIS_HEAD_DIM, rotate, rule, 0u, q_out, aq);
  if (st != MXATTN_OK) return st;
  st = prepare_quantize(k, dtype, kv_shape, k_strides, MXATTN_AXIS_HEAD_DIM, rotate, rule, 0u, k_out, ak);
  if (st != MXATTN_OK) return st;
  st = prepare_quantize(v, dtype, kv_shape, v_strides, MXATTN_AXIS_TOKEN, 0, rule, 0u, v_out, av);
  if (st != MXATTN_OK) return st;
  if (rule != MXATTN_SCALE_UOS && rule != MXATTN_SCALE_OCP) return MXATTN_ERR_ENUM;
  if (q_shape.B != kv_shape.B || q_shape.H != kv_shape.H || q_shape.d != kv_shape.d) return MXATTN_ERR_MISMATCH;
  describe(q_out, q_shape, MXATTN_AXIS_HEAD_DIM, rule, rotate);
  describe(k_out, kv_shape, MXATTN_AXIS_HEAD_DIM, rule, rotate);
  describe(v_out, kv_shape, MXATTN_AXIS_TOKEN, rule, 0);
  return hip_status(launch_quantize_qkv(aq, ak, av, stream));
}

size_t mxattn_scale_sweep_workspace_bytes(mxattn_shape shape, int32_t axis, int32_t n_q) {
  if (check_shape(shape) != MXATTN_OK || (axis != MXATTN_AXIS_HEAD_DIM && axis != MXATTN_AXIS_TOKEN)) return 0;
  if (n_q < 1 || n_q > MXATTN_SWEEP_MAX) return 0;
  return round256((size_t)shape.B * shape.H * sweep_chunks(axis, shape.N, shape.d) * n_q * sizeof(double));
}

// Validation shared by the two sweep entry points; fills everything of `a`
// but the partial-sum buffer.
static mxattn_status sweep_args(const void* x, int32_t dtype, mxattn_shape shape, const int64_t* strides,
                                int32_t axis, int32_t rotate, const double* q_values, int32_t n_q, double* sse,
                                SweepArgs& a) {
  if (!x || !q_values || !sse) return MXATTN_ERR_NULL;
  if (dtype != MXATTN_BF16 && dtype != MXATTN_FP16) return MXATTN_ERR_DTYPE;
  if (axis != MXATTN_AXIS_HEAD_DIM && axis != MXATTN_AXIS_TOKEN) return MXATTN_ERR_ENUM;
  if ((rotate != 0 && rotate != 1) || (rotate && axis != MXATTN_AXIS_HEAD_DIM)) return MXATTN_ERR_ENUM;
  if (n_q < 1 || n_q > MXATTN_SWEEP_MAX) return MXATTN_ERR_ENUM;
  double qmin = q_values[0], qmax = q_values[0];
  for (int j = 0; j < n_q; ++j) {
    if (!boundary_ok(q_values[j])) return MXATTN_ERR_ENUM;
    qmin = q_values[j] < qmin ? q_values[j] : qmin;
    qmax = q_values[j] > qmax ? q_values[j] : qmax;
  }
  if (qmax > 2.0 * qmin) return MXATTN_ERR_ENUM;
  mxattn_status st = check_shape(shape);
  if (st != MXATTN_OK) return st;
  int64_t s[3];
  st = resolve_strides(shape, strides, s);
  if (st != MXATTN_OK) return st;
  a.x = x;
  a.dtype = dtype;
  a.B = shape.B; a.H = shape.H; a.N = shape.N; a.d = shape.d;
  a.sB = s[0]; a.sH = s[1]; a.sN = s[2];
  a.axis = axis;
  a.rotate = rotate;
  a.nq = n_q;
  for (int j = 0; j < n_q; ++j) a.qbits[j] = boundary_bits(q_values[j]);
  a.qmin_bits = boundary_bits(qmin);
  a.chunks = sweep_chunks(axis, shape.N, shape.d);
  a.partial = nullptr;
  a.sse = sse;
  return MXATTN_OK;
}

mxattn_status mxattn_scale_sweep(const void* x, int32_t dtype, mxattn_shape shape,
                                 const int64_t* strides, int32_t axis, int32_t rotate,
                                 const double* q_values, int32_t n_q, double* sse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  SweepArgs a;
  mxattn_status st = sweep_args(x, dtype, shape, strides, axis, rotate, q_values, n_q, sse, a);
  if (st != MXATTN_OK) return st;
  const size_t need = mxattn_scale_sweep_workspace_bytes(shape, axis, n_q);
  if (!workspace || workspace_bytes < need) return MXATTN_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(sse) || !aligned16(workspace)) return MXATTN_ERR_ALIGN;
  a.partial = static_cast<double*>(workspace);
  return hip_status(launch_scale_sweep(a, stream));
}

mxattn_status mxattn_scale_sweep_noalloc(const void* x, int32_t dtype, mxattn_shape shape,
                                         const int64_t* strides, int32_t axis, int32_t rotate,
                                         const double* q_values, int32_t n_q, double* sse,
                                         hipStream_t stream) {
  SweepArgs a;
  mxattn_status st = sweep_args(x, dtype, shape, strides, axis, rotate, q_values, n_q, sse, a);
  if (st != MXATTN_OK) return st;
  if (mxattn_scale_sweep_workspace_bytes(shape, axis, n_q) > (size_t)MXATTN_SWEEP_SCRATCH_BYTES)
    return MXATTN_ERR_SCRATCH;
  if (!aligned16(x) || !aligned16(sse)) return MXATTN_ERR_ALIGN;
  return hip_status(launch_scale_sweep_static(a, stream));
}


mxattn_status mxattn_forward(const mxattn_mx_tensor* q, const mxattn_mx_tensor* k,
                             const mxattn_mx_tensor* v, int32_t causal, float* out,
                             float* row_stats, hipStream_t stream) {
  mxattn_status st = check_mx(q, MXATTN_AXIS_HEAD_DIM);
  if (st != MXATTN_OK) return st;
  st = check_forward(q->shape, q->rotated, k, v, causal, out, row_stats);
  if (st != MXATTN_OK) return st;
  AttnArgs a = forward_args(q->shape, k, v, causal, out, row_stats);
  a.qc = q->codes; a.qs = q->scales;
  a.resident_ok = 1;
  return hip_status(launch_attention(a, stream));
}

mxattn_status mxattn_forward_fused_q(const void* q, int32_t dtype, mxattn_shape q_shape,
                                     const int64_t* q_strides, const mxattn_mx_tensor* k,
                                     const mxattn_mx_tensor* v, int32_t causal, float* out,
                                     float* row_stats, hipStream_t stream) {
  if (!q) return MXATTN_ERR_NULL;
  if (dtype != MXATTN_BF16 && dtype != MXATTN_FP16) return MXATTN_ERR_DTYPE;
  mxattn_status st = check_shape(q_shape);
  if (st != MXATTN_OK) return st;
  int64_t s[3];
  st = resolve_strides(q_shape, q_strides, s);
  if (st != MXATTN_OK) return st;
  if (!aligned16(q)) return MXATTN_ERR_ALIGN;
  if (k && k->rule != MXATTN_SCALE_UOS && k->rule != MXATTN_SCALE_OCP) return MXATTN_ERR_ENUM;
  st = check_forward(q_shape, k ? k->rotated : 0, k, v, causal, out, row_stats);
  if (st != MXATTN_OK) return st;
  AttnArgs a = forward_args(q_shape, k, v, causal, out, row_stats);
  a.qx = q;
  a.qdtype = dtype;
  a.qsB = s[0]; a.qsH = s[1]; a.qsN = s[2];
  a.qrotate = k->rotated != 0;
  a.qrule = k->rule;
  return hip_status(launch_attention(a, stream));
}

size_t mxattn_reference_modes_workspace_bytes(mxattn_shape shape, int32_t p_mode) {
  if (check_shape(shape) != MXATTN_OK) return 0;
  if (p_mode != MXATTN_P_PNQ && p_mode != MXATTN_P_DIRECT && p_mode != MXATTN_P_POSTNORM) return 0;
  size_t total = 3 * (round256(codes_bytes(shape, 0)) + round256(scales_bytes(shape, 0)));
  if (p_mode == MXATTN_P_POSTNORM)
    total += round256((size_t)shape.B * shape.H * padded_tokens(shape.N) * 4 * sizeof(float));
  return total;
}

mxattn_status mxattn_quantize_reference_modes(const void* q, const void* k, const void* v,
                                              int32_t dtype, mxattn_shape shape,
                                              const int64_t* strides, int32_t rule,
                                              int32_t p_mode, int32_t rotate, int32_t causal,
                                              float* out, float* row_sums, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out) return MXATTN_ERR_NULL;
  if (dtype != MXATTN_BF16 && dtype != MXATTN_FP16) return MXATTN_ERR_DTYPE;
  if (rule != MXATTN_SCALE_UOS && rule != MXATTN_SCALE_OCP) return MXATTN_ERR_ENUM;
  if (p_mode != MXATTN_P_PNQ && p_mode != MXATTN_P_DIRECT && p_mode != MXATTN_P_POSTNORM) return MXATTN_ERR_ENUM;
  if ((rotate != 0 && rotate != 1) || (causal != 0 && causal != 1)) return MXATTN_ERR_ENUM;
  mxattn_status st = check_shape(shape);
  if (st != MXATTN_OK) return st;
  int64_t s[3];
  st = resolve_strides(shape, strides, s);
  if (st != MXATTN_OK) return st;
  const size_t need = mxattn_reference_modes_workspace_bytes(shape, p_mode);
  if (!workspace || workspace_bytes < need) return MXATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace) ||
      (row_sums && !aligned16(row_sums)))
    return MXATTN_ERR_ALIGN;

  uint8_t* w = static_cast<uint8_t*>(workspace);
  const size_t cb = round256(codes_bytes(shape, 0)), sb = round256(scales_bytes(shape, 0));
  mxattn_mx_tensor tq = {w, w + cb, shape, 0, 0, 0};
  mxattn_mx_tensor tk = {w + cb + sb, w + 2 * cb + sb, shape, 0, 0, 0};
  mxattn_mx_tensor tv = {w + 2 * (cb + sb), w + 3 * cb + 2 * sb, shape, 0, 0, 0};
  float* stats = reinterpret_cast<float*>(w + 3 * (cb + sb));

  st = mxattn_rotate_quantize(q, dtype, shape, strides, MXATTN_AXIS_HEAD_DIM, rotate, rule, &tq, stream);
  if (st != MXATTN_OK) return st;
  st = mxattn_rotate_quantize(k, dtype, shape, strides, MXATTN_AXIS_HEAD_DIM, rotate, rule, &tk, stream);
  if (st != MXATTN_OK) return st;
  st = mxattn_rotate_quantize(v, dtype, shape, strides, MXATTN_AXIS_TOKEN, 0, rule, &tv, stream);
  if (st != MXATTN_OK) return st;

  AttnArgs a;
  a.qc = tq.codes; a.qs = tq.scales;
  a.kc = tk.codes; a.ks = tk.scales;
  a.vc = tv.codes; a.vs = tv.scales;
  a.B = shape.B; a.H = shape.H; a.N = shape.N; a.d = shape.d;
  a.Nk = shape.N;
  a.causal = causal;
  a.mode = p_mode == MXATTN_P_PNQ ? kModePnq : (p_mode == MXATTN_P_DIRECT ? kModeDirect : kModePostnorm);
  a.rule = rule;
  a.out = out;
  a.row_stats = nullptr;
  a.row_sums = row_sums;
  a.stats_ws = p_mode == MXATTN_P_POSTNORM ? stats : nullptr;
  a.diag = nullptr;
  a.gamma = 1.0f;
  return hip_status(launch_attention(a, stream));
}

size_t mxattn_p_diagnostics_workspace_bytes(mxattn_shape shape) {
  if (check_shape(shape) != MXATTN_OK) return 0;
  return 2 * (round256(codes_bytes(shape, 0)) + round256(scales_bytes(shape, 0))) +
         round256((size_t)shape.B * shape.H * padded_tokens(shape.N) * 4 * sizeof(float));
}

mxattn_status mxattn_p_diagnostics(const void* q, const void* k, int32_t dtype, mxattn_shape shape,
                                   const int64_t* strides, int32_t rule, int32_t rotate, int32_t causal,
                                   float gamma, float* diag, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  if (!q || !k || !diag) return MXATTN_ERR_NULL;
  if (dtype != MXATTN_BF16 && dtype != MXATTN_FP16) return MXATTN_ERR_DTYPE;
  if (rule != MXATTN_SCALE_UOS && rule != MXATTN_SCALE_OCP) return MXATTN_ERR_ENUM;
  if ((rotate != 0 && rotate != 1) || (causal != 0 && causal != 1)) return MXATTN_ERR_ENUM;
  if (!(gamma >= 0x1p-20f && gamma <= 0x1p20f)) return MXATTN_ERR_ENUM;  // also rejects NaN
  mxattn_status st = check_shape(shape);
  if (st != MXATTN_OK) return st;
  int64_t s[3];
  st = resolve_strides(shape, strides, s);
  if (st != MXATTN_OK) return st;
  const size_t need = mxattn_p_diagnostics_workspace_bytes(shape);
  if (!workspace || workspace_bytes < need) return MXATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(diag) || !aligned16(workspace)) return MXATTN_ERR_ALIGN;

  uint8_t* w = static_cast<uint8_t*>(workspace);
  const size_t cb = round256(codes_bytes(shape, 0)), sb = round256(scales_bytes(shape, 0));
  mxattn_mx_tensor tq = {w, w + cb, shape, 0, 0, 0};
  mxattn_mx_tensor tk = {w + cb + sb, w + 2 * cb + sb, shape, 0, 0, 0};
  float* stats = reinterpret_cast<float*>(w + 2 * (cb + sb));
  st = mxattn_rotate_quantize(q, dtype, shape, strides, MXATTN_AXIS_HEAD_DIM, rotate, rule, &tq, stream);
  if (st != MXATTN_OK) return st;
  st = mxattn_rotate_quantize(k, dtype, shape, strides, MXATTN_AXIS_HEAD_DIM, rotate, rule, &tk, stream);
  if (st != MXATTN_OK) return st;

  AttnArgs a;
  a.qc = tq.codes; a.qs = tq.scales;
  a.kc = tk.codes; a.ks = tk.scales;
  // no PV product: the value tiles the kernel stages are never read, so K^
  // (a buffer of the same size) stands in for them
  a.vc = tk.codes; a.vs = tk.scales;
  a.B = shape.B; a.H = shape.H; a.N = shape.N; a.d = shape.d;
  a.Nk = shape.N;
  a.causal = causal;
  a.mode = kModeDiag;
  a.rule = rule;
  a.out = nullptr;
  a.row_stats = nullptr;
  a.row_sums = nullptr;
  a.stats_ws = stats;
  a.diag = diag;
  a.gamma = gamma;
  return hip_status(launch_attention(a, stream));
}

const char* mxattn_status_string(mxattn_status status) {
  switch (status) {
    case MXATTN_OK: return "ok";
    case MXATTN_ERR_NULL: return "a required pointer is NULL";
    case MXATTN_ERR_SHAPE: return "unsupported shape (B, H, N >= 1; d in {64, 128})";
    case MXATTN_ERR_DTYPE: return "unknown input dtype";
    case MXATTN_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MXATTN_ERR_STRIDE: return "strides must be non-negative multiples of 8 elements";
    case MXATTN_ERR_MISMATCH: return "MXFP4 tensor descriptors disagree";
    case MXATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case MXATTN_ERR_ENUM: return "unknown axis, rule, placement or flag value";
    case MXATTN_ERR_HIP: return "HIP runtime error";
    case MXATTN_ERR_SCRATCH: return "problem exceeds the library's static scratch (MXATTN_SWEEP_SCRATCH_BYTES)";
  }
  return "unknown status";
}

}  // extern "C"
