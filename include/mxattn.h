/*
 * mxattn.h -- C ABI of libmxattn: MXAttention's MXFP4 attention forward for
 * AMD Instinct MI355X (CDNA4, gfx950).
 *
 * The method (MXAttention, "Data-Free Optimal Scaling and Pre-Normalization
 * Quantization for MXFP4 Attention"):
 *   1. a fixed Hadamard rotation of Q and K (Sec. 4.3, Alg. 2);
 *   2. MXFP4 quantization of Q, K and V -- 32-element blocks of E2M1 values
 *      sharing one E8M0 scale chosen by Universal Optimal Scaling,
 *      e = ceil(log2(M / 7.25)) (Sec. 4.1, Alg. 1; Alg. 2);
 *   3. block-scaled FP4 matrix products QK^T and PV inside a tiled online
 *      softmax (Sec. 2, Eqs. 2-8; Alg. 2);
 *   4. Pre-Normalization Quantization: the unnormalized exponential tile
 *      exp(S - m) is quantized once, and that same quantized tile updates both
 *      the row sum l and the output accumulator (Sec. 4.2, Eqs. 44-48).
 *
 * Conventions shared by every call
 *   - Memory: the caller allocates every buffer (device memory unless noted)
 *     and keeps ownership; the library allocates nothing and keeps no state
 *     between calls.  Calls are thread-safe.
 *   - Streams: work is enqueued on `stream` (0 = the null stream) and returns
 *     without synchronizing; results are valid once the stream has reached
 *     that point.  Kernels run on the calling thread's current HIP device:
 *     every pointer, and the stream, must belong to that device.  The library
 *     cannot check this; memory of another device or host memory makes the
 *     kernels fault.
 *   - Errors: every argument is validated before anything is enqueued; on an
 *     error nothing is written and nothing is launched.  A launch failure
 *     after validation returns MXATTN_ERR_HIP.
 *   - Inputs must be finite.  Outputs for non-finite inputs are unspecified.
 *   - Output and workspace buffers must not overlap each other or any input
 *     of the same call (the library cannot check this).
 *   - Alignment: every device pointer must be 16-byte aligned.
 *
 * Layouts
 *   Input tensors Q, K, V: 16-bit elements (bfloat16 or IEEE half), logical
 *   shape [B, H, N, d].  `strides` gives the element strides of the B, H and N
 *   dimensions (NULL = contiguous); the d dimension is contiguous.  Every
 *   stride must be a multiple of 8 elements (16-byte aligned rows).
 *
 *   Let Np = N rounded up to a multiple of MXATTN_TOKEN_ALIGN (128).
 *
 *   MXFP4, head-dimension axis (Q^, K^):
 *     codes  uint8 [B, H, Np, d/2]: byte k of a row holds element 2k in
 *            bits 0-3 and element 2k+1 in bits 4-7; a 4-bit code is the
 *            E2M1 value with the sign in bit 3 (magnitudes 0, .5, 1, 1.5, 2,
 *            3, 4, 6 are codes 0..7);
 *     scales uint8 [B, H, Np, d/32]: E8M0 byte, value 2^(byte - 127), of
 *            elements 32j .. 32j+31 of the row.
 *     Rows n >= N are written as zeros (codes 0, scale byte 127).
 *   MXFP4, token axis (V^):
 *     codes  uint8 [B, H, Np/32, d, 16]: for token block kb and channel c,
 *            byte t holds token 32kb+2t in bits 0-3 and 32kb+2t+1 in 4-7;
 *     scales uint8 [B, H, Np/32, d]: scale of tokens 32kb .. 32kb+31 of
 *            channel c.
 *     Tokens n >= N count as +0 (code 0); blocks with no token below N get
 *     scale byte 127.
 *
 * Numerics of the quantizers (bit-exact contract)
 *   - Rotation (Q, K): x <- x H_d / sqrt(d) with H_d the Sylvester Hadamard
 *     matrix in natural order, computed in binary32 as butterflies of stride
 *     1, 2, 4, ..., d/2 (each output one correctly rounded add/subtract),
 *     then one multiply by fl32(1/sqrt(d)).
 *   - Block scale: M = max |x_i|; an all-zero block gets 2^0.  Otherwise UOS
 *     e = ceil(log2(M / 7.25)), OCP e = floor(log2 M) - 2, or (the ceiling
 *     family, mxattn_rotate_quantize_q) e = ceil(log2(M / q)), i.e. the
 *     smallest e with M <= q 2^e, clamped to [-127, 127].
 *   - Elements: x_i / 2^e rounded to the nearest E2M1 value, ties to the even
 *     code, magnitudes above 6 saturating at 6; a value that rounds to zero
 *     keeps its sign bit.
 */
#ifndef MXATTN_H
#define MXATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXATTN_OK = 0,
  MXATTN_ERR_NULL = 1,      /* a required pointer is NULL                          */
  MXATTN_ERR_SHAPE = 2,     /* B, H or N < 1, d not 64 or 128, or B*H*Np*d > 2^36   */
  MXATTN_ERR_DTYPE = 3,     /* unknown dtype                                        */
  MXATTN_ERR_ALIGN = 4,     /* a device pointer is not 16-byte aligned              */
  MXATTN_ERR_STRIDE = 5,    /* a stride is negative or not a multiple of 8 elements */
  MXATTN_ERR_MISMATCH = 6,  /* MXFP4 tensor descriptors disagree                    */
  MXATTN_ERR_WORKSPACE = 7, /* workspace missing or smaller than required           */
  MXATTN_ERR_ENUM = 8,      /* unknown axis, rule or P placement                    */
  MXATTN_ERR_HIP = 9,       /* a HIP runtime call or kernel launch failed           */
  MXATTN_ERR_SCRATCH = 10   /* the call needs more than the library's static scratch */
} mxattn_status;

typedef enum { MXATTN_BF16 = 0, MXATTN_FP16 = 1 } mxattn_dtype;
typedef enum { MXATTN_AXIS_HEAD_DIM = 0, MXATTN_AXIS_TOKEN = 1 } mxattn_axis;
/* Shared-scale rule: UOS (Sec. 4.1, Eq. 19 with q* = 7.25), the OCP floor
 * rule used by the vanilla baseline (Sec. 2, Eq. 11; App. G Eq. 97), or the
 * ceiling family e = ceil(log2(M / q)) with a caller-chosen boundary q
 * (Eq. 13; q = 6 is TFS, Eq. 14; q = 7 the OAS-equivalent rule, App. G; UOS
 * is q = 7.25).  CEIL_Q tensors come from mxattn_rotate_quantize_q. */
typedef enum { MXATTN_SCALE_UOS = 0, MXATTN_SCALE_OCP = 1, MXATTN_SCALE_CEIL_Q = 2 } mxattn_scale_rule;
/* Placement of the softmax-path quantizer (Sec. 4.2; Sec. 5.5.2):
 *   PNQ      l and O both updated from Q(P~)            (Eqs. 44-48)
 *   DIRECT   l from P~, O from Q(P~)                     (Eq. 42 / Eqs. 16-17)
 *   POSTNORM P = softmax(S) computed exactly first, then O = Q(P) V^ with no
 *            renormalization (the materialized-P diagnostic of Sec. 5.5.2). */
typedef enum { MXATTN_P_PNQ = 0, MXATTN_P_DIRECT = 1, MXATTN_P_POSTNORM = 2 } mxattn_p_mode;

#define MXATTN_TOKEN_ALIGN 128
#define MXATTN_SWEEP_MAX 48   /* boundaries per mxattn_scale_sweep call     */
#define MXATTN_Q_MIN 2.0      /* range of a ceiling-rule boundary q          */
#define MXATTN_Q_MAX 64.0

typedef struct {
  int32_t B, H, N, d;
} mxattn_shape;

/* Descriptor of a caller-owned MXFP4 tensor in one of the layouts above. */
typedef struct {
  uint8_t* codes;
  uint8_t* scales;
  mxattn_shape shape;
  int32_t axis;    /* mxattn_axis       */
  int32_t rule;    /* mxattn_scale_rule */
  int32_t rotated; /* 1 if Hadamard-rotated before quantization */
} mxattn_mx_tensor;

/* Bytes of the codes / scales buffers of an MXFP4 tensor of `shape` blocked
 * along `axis` (Np-padded layouts above).  0 for an invalid shape or axis. */
size_t mxattn_mx_codes_bytes(mxattn_shape shape, int32_t axis);
size_t mxattn_mx_scales_bytes(mxattn_shape shape, int32_t axis);

/* Width B_c of the key/value tiles of the online-softmax loop of
 * mxattn_forward (Alg. 2).  PNQ quantizes each exponential tile
 * against the running maximum reached after that tile, so the result depends
 * on B_c: it is part of the definition of the output.  Tiles are visited in
 * ascending key order; the exponentials are quantized in 32-key blocks
 * aligned to key 0.  Returns 128 for d in {64, 128}, 0 otherwise. */
int32_t mxattn_forward_kv_tile(int32_t d, int32_t causal);

/* Rotate (optionally) and quantize one tensor to MXFP4.
 *   x        device pointer to the [B, H, N, d] 16-bit input
 *   dtype    mxattn_dtype
 *   strides  host array of 3 element strides (B, H, N) or NULL (contiguous)
 *   axis     MXATTN_AXIS_HEAD_DIM (Q, K; Alg. 2, blocks along d)
 *            or MXATTN_AXIS_TOKEN (V; Alg. 2, blocks along tokens --
 *            the block axis of the PV product's contraction, as the MatX
 *            "leaky quantization" page describes)
 *   rotate   1: apply the Hadamard rotation first (Alg. 2); only
 *            allowed with MXATTN_AXIS_HEAD_DIM
 *   rule     mxattn_scale_rule
 *   out      host descriptor: the caller sets out->codes and out->scales to
 *            buffers of mxattn_mx_codes_bytes / mxattn_mx_scales_bytes; the
 *            call fills shape, axis, rule and rotated.
 * The padded rows/blocks are written too (see Layouts). */
mxattn_status mxattn_rotate_quantize(const void* x, int32_t dtype, mxattn_shape shape,
                                     const int64_t* strides, int32_t axis, int32_t rotate,
                                     int32_t rule, mxattn_mx_tensor* out, hipStream_t stream);

/* mxattn_rotate_quantize with the ceiling rule e = ceil(log2(M / q_max))
 * (Eq. 13) for a boundary q_max in [MXATTN_Q_MIN, MXATTN_Q_MAX]
 * (MXATTN_ERR_ENUM otherwise, or if it is not finite).  The comparison
 * M <= q_max 2^e is exact: q_max is taken as a binary64 number.  Same
 * layouts, arguments and padding as mxattn_rotate_quantize; out->rule is set
 * to MXATTN_SCALE_CEIL_Q.  q_max = 7.25 reproduces the UOS codes bit for bit. */
mxattn_status mxattn_rotate_quantize_q(const void* x, int32_t dtype, mxattn_shape shape,
                                       const int64_t* strides, int32_t axis, int32_t rotate,
                                       double q_max, mxattn_mx_tensor* out, hipStream_t stream);

/* Q, K and V of one attention call quantized in a single launch (Alg. 2's
 * preprocessing of all three inputs): Q and K along the head dimension,
 * rotated first if `rotate`, V along tokens, all with `rule`.  The outputs
 * equal those of three mxattn_rotate_quantize calls bit for bit; one launch
 * saves the two kernel boundaries between them.
 *   q, k, v    16-bit device inputs, one dtype
 *   q_shape    [B, H, Nq, d]; kv_shape [B, H, Nk, d] for K and V (same B, H,
 *              d as Q, else MXATTN_ERR_MISMATCH)
 *   q_strides, k_strides, v_strides   as in mxattn_rotate_quantize
 *   rotate     0 or 1 (Q and K)
 *   rule       MXATTN_SCALE_UOS or MXATTN_SCALE_OCP (else MXATTN_ERR_ENUM)
 *   q_out, k_out, v_out   host descriptors with caller buffers, as `out` of
 *              mxattn_rotate_quantize; the call fills their shape, axis,
 *              rule and rotated fields
 * Errors: those of mxattn_rotate_quantize for each tensor, then
 * MXATTN_ERR_ENUM and MXATTN_ERR_MISMATCH; nothing is enqueued on an error. */
mxattn_status mxattn_rotate_quantize_qkv(const void* q, const void* k, const void* v, int32_t dtype,
                                         mxattn_shape q_shape, mxattn_shape kv_shape, const int64_t* q_strides,
                                         const int64_t* k_strides, const int64_t* v_strides, int32_t rotate,
                                         int32_t rule, mxattn_mx_tensor* q_out, mxattn_mx_tensor* k_out,
                                         mxattn_mx_tensor* v_out, hipStream_t stream);

/* Workspace needed by mxattn_scale_sweep for `shape`, `axis` and n_q
 * boundaries.  0 for an invalid shape, axis or count. */
size_t mxattn_scale_sweep_workspace_bytes(mxattn_shape shape, int32_t axis, int32_t n_q);

/* The Q_max sweep of Sec. 5.5.1 (Table 4): for every head (b, h) and every
 * boundary q_j, the sum over the head's MXFP4 blocks of sum_i (x_i - x^_i)^2,
 * where x is exactly what mxattn_rotate_quantize sees (the decoded input,
 * Hadamard-rotated in binary32 if `rotate`) and x^ its MXFP4 reconstruction
 * under e = ceil(log2(M / q_j)).  Summed over the heads of a tensor and
 * divided by its element count it is the tensor MSE whose argmin over q is
 * the per-attention-block optimum of Table 4.
 *   x, dtype, shape, strides, axis, rotate   as in mxattn_rotate_quantize
 *   q_values  host array of n_q boundaries, 1 <= n_q <= MXATTN_SWEEP_MAX,
 *             each in [MXATTN_Q_MIN, MXATTN_Q_MAX], with max <= 2 min (so a
 *             block has at most two candidate exponents); any order
 *   sse       device double [B*H][n_q] (head-major)
 *   workspace device buffer of at least
 *             mxattn_scale_sweep_workspace_bytes(shape, axis, n_q) bytes
 * Errors: MXATTN_ERR_ENUM for a bad boundary list, MXATTN_ERR_WORKSPACE for
 * a missing or short workspace.  The sums are accumulated in binary64 in a
 * fixed order: the result is identical on every run, and two boundaries that
 * select the same exponent for every block give bit-identical sums. */
mxattn_status mxattn_scale_sweep(const void* x, int32_t dtype, mxattn_shape shape,
                                 const int64_t* strides, int32_t axis, int32_t rotate,
                                 const double* q_values, int32_t n_q, double* sse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the device array, allocated once per GPU with the library's code
 * and kept until the process ends, that mxattn_scale_sweep_noalloc uses in
 * place of a workspace. */
#define MXATTN_SWEEP_SCRATCH_BYTES (16u << 20)

/* mxattn_scale_sweep without a workspace argument, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The per-workgroup
 * partial sums go to a static device array of MXATTN_SWEEP_SCRATCH_BYTES
 * (one per GPU, resolved on the call's current device at its first call
 * there); the call itself allocates nothing.  Arguments, results and the
 * other errors are those of mxattn_scale_sweep; the result is bit-identical
 * to it.  MXATTN_ERR_SCRATCH if mxattn_scale_sweep_workspace_bytes(shape,
 * axis, n_q) exceeds MXATTN_SWEEP_SCRATCH_BYTES (e.g. B*H = 40, N = 32760,
 * d = 128 with 48 boundaries needs 0.49 MB; the limit admits about 34x that),
 * and nothing is enqueued.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * give undefined sums; order them.  Nothing in the array needs clearing:
 * every partial sum is written before it is read. */
mxattn_status mxattn_scale_sweep_noalloc(const void* x, int32_t dtype, mxattn_shape shape,
                                         const int64_t* strides, int32_t axis, int32_t rotate,
                                         const double* q_values, int32_t n_q, double* sse,
                                         hipStream_t stream);

/* Fused MXFP4 attention forward with PNQ (Alg. 2).
 *   q        head-dimension MXFP4 tensor, shape [B, H, Nq, d]
 *   k        head-dimension MXFP4 tensor, shape [B, H, Nk, d]; both q and k
 *            rotated or both not (Q K^T is unchanged by the rotation only if
 *            both are)
 *   v        token-axis MXFP4 tensor of the shape of k
 *            Nk != Nq is cross-attention, as in the separate text
 *            cross-attention of the video models the pages evaluate
 *            (Sec. 5.1); the key loop then runs over the Nk tokens
 *   causal   1: key j is visible to query i iff j <= i (needs Nk = Nq,
 *            else MXATTN_ERR_MISMATCH)
 *   out      device float [B, H, Nq, d], contiguous: O = diag(l)^-1 O~
 *            (Eq. 8)
 *   row_stats device float [B, H, Nq, 2] or NULL: (m, l) per row, with m
 *            the final running maximum of S = Q^ K^T / sqrt(d) and l the
 *            final PNQ row sum (l >= 1, App. J)
 * S, l and O~ accumulate in binary32; O = O~ / l is correctly rounded.  The
 * exponential tile is quantized with the UOS rule whatever the rule of the
 * inputs.  Without the causal mask, when every key tile of a head fits in
 * LDS (Nk <= 512 at d = 128, <= 1024 at d = 64) the call runs a kernel that
 * keeps each head's K^, V^ resident while it walks that head's query tiles;
 * the result is the same, bit for bit, as the streaming kernel's. */
mxattn_status mxattn_forward(const mxattn_mx_tensor* q, const mxattn_mx_tensor* k,
                             const mxattn_mx_tensor* v, int32_t causal, float* out,
                             float* row_stats, hipStream_t stream);

/* mxattn_forward with the Q preprocessing fused into its prologue: the
 * paper puts the Hadamard rotation inside the Q/K preprocessing stage at
 * negligible cost (Sec. 4.3; Alg. 2).  Each workgroup rotates (if
 * k->rotated) and quantizes its own query rows with k's rule, exactly as
 * mxattn_rotate_quantize would (bit for bit), and keeps Q^ on chip: no Q^
 * buffer, no separate launch.  The output equals that of
 * mxattn_rotate_quantize + mxattn_forward bit for bit.
 *   q, dtype   16-bit Q (MXATTN_BF16 or MXATTN_FP16), device, 16-byte aligned
 *   q_shape    [B, H, Nq, d]
 *   q_strides  as in mxattn_rotate_quantize (NULL: contiguous)
 *   k, v, causal, out, row_stats   as in mxattn_forward; k->rule must be
 *              MXATTN_SCALE_UOS or MXATTN_SCALE_OCP (else MXATTN_ERR_ENUM)
 * Errors: those of mxattn_forward (with q_shape in place of q->shape), and
 * MXATTN_ERR_NULL, MXATTN_ERR_DTYPE, MXATTN_ERR_SHAPE, MXATTN_ERR_STRIDE,
 * MXATTN_ERR_ALIGN for q; nothing is enqueued on an error. */
mxattn_status mxattn_forward_fused_q(const void* q, int32_t dtype, mxattn_shape q_shape,
                                     const int64_t* q_strides, const mxattn_mx_tensor* k,
                                     const mxattn_mx_tensor* v, int32_t causal, float* out,
                                     float* row_stats, hipStream_t stream);

/* Workspace needed by mxattn_quantize_reference_modes for `shape`/`p_mode`
 * (the three MXFP4 tensors, plus per-row statistics for POSTNORM).
 * 0 for an invalid shape or mode. */
size_t mxattn_reference_modes_workspace_bytes(mxattn_shape shape, int32_t p_mode);

/* The compared configurations of the ablation (Sec. 5.2, Sec. 5.4) and the
 * materialized-P diagnostic (Sec. 5.5.2), end to end from 16-bit Q, K, V:
 * quantize all three with `rule` (rotating Q and K if `rotate`), then run the
 * forward with the softmax-path placement `p_mode`, quantizing the
 * exponential (or probability) tiles with the same `rule`.
 *   rule=OCP, p_mode=DIRECT, rotate=0 is the vanilla OCP MXFP4 baseline;
 *   rule=UOS, p_mode=PNQ, rotate=1 equals rotate_quantize x3 + forward.
 *   out       device float [B, H, N, d], contiguous
 *   row_sums  device float [B, H, N] or NULL: the induced sum of the
 *             normalized attention weights of each row -- PNQ: 1 up to
 *             rounding (Prop. 1); DIRECT: (sum beta P^ 1) / l (App. I,
 *             Eq. 110); POSTNORM: sum_j Q(P)_ij
 *   workspace device buffer of at least
 *             mxattn_reference_modes_workspace_bytes(shape, p_mode) bytes */
mxattn_status mxattn_quantize_reference_modes(const void* q, const void* k, const void* v,
                                              int32_t dtype, mxattn_shape shape,
                                              const int64_t* strides, int32_t rule,
                                              int32_t p_mode, int32_t rotate, int32_t causal,
                                              float* out, float* row_sums, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream);

/* Workspace needed by mxattn_p_diagnostics for `shape` (Q^, K^ and the
 * per-row statistics).  0 for an invalid shape. */
size_t mxattn_p_diagnostics_workspace_bytes(mxattn_shape shape);

/* Row-sum diagnostics of quantizing the materialized probabilities
 * (Sec. 5.5.2, Fig. 7), from 16-bit Q and K: quantize Q and K with `rule`
 * (rotating them if `rotate`), compute the exact softmax P = softmax(S) of
 * every row (a first pass finds m and l), and quantize gamma P in aligned
 * 32-key blocks with `rule`: P^ = Q(gamma P) / gamma.  gamma is the
 * pre-quantization global scale of Fig. 7 (C); 1 gives the plain
 * diagnostic.  (With the factor kept, Q(gamma P), a row sum is gamma times
 * diag[.., 0].)  Writes, per query row, 6 floats:
 *   diag[.., 0]  sum_j P^_ij, the induced row sum (Fig. 7 (A));
 *   diag[.., 1..4]  the row-sum error sum_j (P^_ij - P_ij) split by the
 *                outcome of each element (Fig. 7 (B)): zeroing (P > 0 but
 *                P^ = 0), saturation (gamma P / 2^e above the largest E2M1
 *                value 6), downward and upward rounding of the rest;
 *   diag[.., 5]  the row's entropy -sum_j P_ij ln P_ij in nats (Fig. 7 (D)).
 * No value tensor and no PV product are involved.
 *   q, k, dtype, shape, strides   as in mxattn_quantize_reference_modes
 *   rule      MXATTN_SCALE_UOS or MXATTN_SCALE_OCP (Q, K and P)
 *   causal    1: key j is visible to query i iff j <= i
 *   gamma     in [2^-20, 2^20]
 *   diag      device float [B, H, N, 6], contiguous
 *   workspace device buffer of at least
 *             mxattn_p_diagnostics_workspace_bytes(shape) bytes
 * P is evaluated in binary32 (exp2 of (s - m) c - log2 l); sums accumulate
 * in binary32.  gamma enters only through gamma_f in gamma = 2^k gamma_f,
 * 1 <= gamma_f < 2: a power-of-two factor moves every block exponent by k
 * and cancels, so such gammas give bit-identical results.  Errors:
 * MXATTN_ERR_NULL, MXATTN_ERR_DTYPE, MXATTN_ERR_ENUM (rule, rotate, causal,
 * gamma outside its range or NaN), the shape and stride errors of
 * mxattn_rotate_quantize, MXATTN_ERR_WORKSPACE, MXATTN_ERR_ALIGN (a pointer
 * not 16-byte aligned); nothing is enqueued on an error. */
mxattn_status mxattn_p_diagnostics(const void* q, const void* k, int32_t dtype, mxattn_shape shape,
                                   const int64_t* strides, int32_t rule, int32_t rotate, int32_t causal,
                                   float gamma, float* diag, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* mxattn_status_string(mxattn_status status);

#ifdef __cplusplus
}
#endif
#endif /* MXATTN_H */
