/*
 * oracle.h -- plain, slow CPU reference ("oracle") for MXAttention's MXFP4
 * attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may call it.  The product path (the HIP kernels
 * and the C-ABI library) never does, and shares no code, header, table or
 * constant generator with it.
 *
 * Sources (the three pages this method is described on):
 *   [P1] "MXAttention: Data-Free Optimal Scaling and Pre-Normalization
 *        Quantization for MXFP4 Attention" (arXiv 2607.24377).
 *   [P2] "MXAttention core idea" explainer with glossary (the page that
 *        carries the UOS worked example, block max 14.5).
 *   [P3] MatX, "Leaky quantization" (block quantization and causal leakage).
 *
 * Precision: every quantity is IEEE binary64, with one exception.  The
 * Hadamard rotation of Q and K is evaluated in binary32 with a fixed butterfly
 * order, because its outputs decide the 4-bit codes bit for bit and the
 * pages fix no precision for it (see oracle_hadamard_rotate_f32).
 *
 * Threads are used only across independent units (heads, row ranges).
 */
#ifndef MXATTN_ORACLE_H
#define MXATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* input element encodings (raw 16-bit patterns) */
#define ORACLE_BF16 0
#define ORACLE_FP16 1

/* block axes: along the head dimension (Q, K) or along tokens (V) [P3, Block
 * quantization / Quantizing attention] */
#define ORACLE_AXIS_HEAD_DIM 0
#define ORACLE_AXIS_TOKEN 1

/* shared-scale rules [P1 Sec. 2, Eqs. 11-13; Sec. 4.1, Eq. 19] */
#define ORACLE_RULE_UOS 0       /* e = ceil(log2(M / 7.25))                 */
#define ORACLE_RULE_OCP 1       /* e = floor(log2 M) - 2      (Eq. 11 / 97) */
#define ORACLE_RULE_CEIL_Q 2    /* e = ceil(log2(M / q)), any q (Eq. 13)    */
#define ORACLE_RULE_FLOOR_Q 3   /* e = floor(log2(M / q)) + 1   (Eq. 12)    */

/* placement of the softmax-path quantizer [P1 Sec. 4.2; Sec. 5.5.2] */
#define ORACLE_P_PNQ 0          /* l and O both from Q(P~)      (Eqs. 44-48) */
#define ORACLE_P_DIRECT 1       /* l from P~, O from Q(P~)      (Eq. 42)     */
#define ORACLE_P_POSTNORM 2     /* quantize the normalized P    (Sec. 5.5.2) */
#define ORACLE_P_EXACT 3        /* P~ enters both updates unquantized        */

/* The E2M1 element grid, magnitude codes 0..7 [P1 Eq. 9 / Eq. 67]. */
double oracle_e2m1_magnitude(int code);

/* Signed value of a 4-bit code: bit 3 is the sign, bits 0..2 the magnitude. */
double oracle_e2m1_value(int code);

/* The E2M1 grid point nearest to y >= 0, with every y above the largest
 * grid value mapped to 6 [P1 Eq. 10]; an exact tie goes to the even code.
 * Returns the magnitude code 0..7. */
int oracle_e2m1_project(double y);

/* Shared-scale exponent for block maximum M > 0 under `rule` (q is read by
 * the *_Q rules only).  Returned unclamped.  M <= 0, a non-finite M, or (for
 * the *_Q rules) q <= 0 or non-finite return 0. */
int oracle_scale_exponent(double M, int rule, double q);

/* oracle_scale_exponent over an array: out[i] for M[i] > 0. */
void oracle_scale_exponents(const double* M, int64_t n, int rule, double q, int32_t* out);

/* Quantize one block of n <= 32 values (missing tail values count as +0)
 * [P1 Alg. 1].  Writes the E8M0 scale byte (exponent + 127, clamped to
 * 0..254) and n 4-bit codes.  An all-zero block gets scale 1 (byte 127).
 * Returns the clamped exponent. */
int oracle_quantize_block(const double* x, int n, int rule, double q,
                          uint8_t* scale_byte, uint8_t* codes);

/* One 32-key block of the softmax-path quantizer [P1 Alg. 1 on P~, Eq. 44]
 * with its decision allowance: ph[t] = the dequantized P^, and (dp non-NULL)
 * dp[t] = the largest change of P^_t that a decision within relative margin
 * delta of its threshold could make -- an element near a rounding midpoint,
 * or a block maximum near an end of the rule's range (then every element is
 * re-projected at the neighbouring exponent).  exact_ref > 0 says the block's
 * maximum is the row maximum's element, known exactly relative to exact_ref
 * (P~ = exp(0) = 1 online; gamma / l* < gamma after normalization): a scale
 * boundary equal to exact_ref then offers no alternative.  Returns the
 * clamped block exponent. */
int oracle_p_block_allowance(const double* p, int rule, double q, double delta, double exact_ref, double* ph,
                             double* dp);

/* Exact decode of a 16-bit element to binary32. */
float oracle_decode_half(uint16_t bits, int dtype);

/* x <- x * H_d / sqrt(d) for one row of length d (a power of two), where H_d
 * is the Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i & j)
 * [P1 Sec. 4.3, Alg. 2; P2 "Rotate Q and K"].  Evaluated in
 * binary32: butterflies with strides 1, 2, 4, ..., d/2, each output one
 * correctly rounded add or subtract, then one multiply by fl32(1/sqrt(d)). */
void oracle_hadamard_rotate_f32(float* x, int d);

/* Quantize selected Q/K rows along the head dimension.  `x` holds B*H*N*d
 * 16-bit elements addressed with element strides `strides` (B, H, N; the d
 * stride is 1; NULL = contiguous).  `rows` lists global row indices
 * (b*H + h)*N + n; NULL with n_rows = B*H*N means every row in order.
 * Outputs: codes [n_rows][d] (one 4-bit code per byte), scales
 * [n_rows][d/32].  Returns 0, or -1 on a bad argument. */
int oracle_quantize_rows(const uint16_t* x, int dtype, int B, int H, int N, int d,
                         const int64_t* strides, int rotate, int rule, double q,
                         const int64_t* rows, int64_t n_rows,
                         uint8_t* codes, uint8_t* scales, int nthreads);

/* Quantize selected V token blocks: block index (b*H + h)*NB + kb with
 * NB = ceil(N/32); NULL with n_blocks = B*H*NB means all blocks in order.
 * Block kb covers tokens 32*kb .. 32*kb+31 of one channel, tokens past N
 * counting as +0 [P3, Quantizing attention].  Outputs: codes
 * [n_blocks][d][32] (token-minor), scales [n_blocks][d]. */
int oracle_quantize_token_blocks(const uint16_t* x, int dtype, int B, int H, int N, int d,
                                 const int64_t* strides, int rule, double q,
                                 const int64_t* blocks, int64_t n_blocks,
                                 uint8_t* codes, uint8_t* scales, int nthreads);

/* Scale-boundary sweep [P1 Sec. 5.5.1, Table 4; Eq. 13]: for each listed
 * head (`heads`: indices b*H + h; NULL with n_heads = B*H means all in order)
 * and each boundary q_j, the sum over the head's MXFP4 blocks of
 * sum_i (x_i - x^_i)^2, where x is what the quantizer sees (the decoded input,
 * Hadamard-rotated in binary32 if `rotate`) and x^ its MXFP4 reconstruction
 * with e = ceil(log2(M / q_j)).  axis HEAD_DIM: 32-channel blocks of a row;
 * axis TOKEN: 32-token blocks of a channel, tokens past N counting as +0.
 * sse: [n_heads][n_q] binary64.  Returns 0, or -1 on a bad argument. */
int oracle_scale_sweep(const uint16_t* x, int dtype, int B, int H, int N, int d,
                       const int64_t* strides, int axis, int rotate, const double* qs, int n_q,
                       const int64_t* heads, int64_t n_heads, double* sse, int nthreads);

typedef struct {
  int32_t B, H, N, d;
  int32_t dtype;
  int32_t causal;      /* key j visible to query i iff j <= i              */
  int32_t rotate;      /* Hadamard-rotate Q and K before quantizing them    */
  int32_t quant;       /* 1: MXFP4 Q, K, V; 0: no quantization anywhere     */
  int32_t rule;        /* ORACLE_RULE_* for every quantizer                 */
  int32_t p_mode;      /* ORACLE_P_*                                        */
  int32_t kv_tile;     /* B_c, a positive multiple of 32                    */
  int32_t nthreads;
  double q;            /* boundary for the *_Q rules                        */
  double amb_delta;    /* relative decision margin for the allowance; 0=off */
  int32_t Nk;          /* key/value tokens (cross-attention); 0 means N.
                          Nk != N needs causal = 0 and contiguous inputs   */
} oracle_attn_cfg;

/* Attention forward [P1 Alg. 2; Eqs. 2-8 and 44-48].  Q holds N query rows
 * per head; K and V hold cfg->Nk (or N) tokens.  For every head and every
 * listed query row (`rows`, n_rows indices shared by all heads; NULL means
 * all N rows) it writes
 *   out      [B][H][n_rows][d]  the output row O_i
 *   m_out    [B][H][n_rows]     final running max (in S units), nullable
 *   l_out    [B][H][n_rows]     final l (for POSTNORM: the exact softmax
 *                               normalizer of pass 1), nullable
 *   rowsum   [B][H][n_rows]     induced row sum of the normalized weights:
 *                               PNQ/EXACT (sum_t beta_t P^_t 1)/l
 *                               [App. H Eqs. 99-105; Prop. 1], DIRECT
 *                               (sum beta P^ 1)/(sum beta P~ 1) [App. I
 *                               Eq. 110], POSTNORM sum_j Q(P)_ij; nullable
 *   amb      [B][H][n_rows][d]  first-order bound on how far O_i moves when
 *                               every P-quantizer decision lying within
 *                               relative margin amb_delta of its threshold
 *                               goes the other way; nullable
 *   absmass  [B][H][n_rows][d]  the output computed with |V^| in place of V^
 *                               (sum_j beta_j P^_j |v^_j| / l), the scale of
 *                               rounding errors of any accumulation order;
 *                               nullable
 *   amb_rowsum [B][H][n_rows]   how far `rowsum` moves when those decisions
 *                               go the other way (it is linear in P^: exact,
 *                               not first-order): POSTNORM the sum of their
 *                               changes, DIRECT the beta-weighted sum over
 *                               (sum beta P~ 1), PNQ 0 (its row sum is 1
 *                               whatever they decide); nullable
 * Returns 0, or -1 on a bad argument. */
int oracle_attention(const oracle_attn_cfg* cfg,
                     const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const int64_t* strides, const int32_t* rows, int32_t n_rows,
                     double* out, double* m_out, double* l_out, double* rowsum,
                     double* amb, double* absmass, double* amb_rowsum);

/* Row-sum diagnostics of quantizing the materialized probabilities
 * [P1 Sec. 5.5.2, Fig. 7]: for each listed query row (rows / n_rows as in
 * oracle_attention; cfg->rule UOS or OCP, cfg->quant = 1, cfg->kv_tile
 * ignored), P = softmax(S) over the visible keys exactly, P^ = Q(gamma P) /
 * gamma with aligned 32-key blocks.  diag [B][H][n_rows][6]:
 *   0  sum_j P^_ij                     (the induced row sum)
 *   1  zeroing: sum of P^ - P over elements with P > 0, P^ = 0
 *   2  saturation: over elements with gamma P / 2^e > 6
 *   3  downward rounding: over the remaining elements with P^ < P
 *   4  upward rounding: over elements with P^ > P
 *   5  entropy -sum_j P_ij ln P_ij (nats)
 * so that diag[0] - 1 = diag[1] + diag[2] + diag[3] + diag[4].
 * amb [B][H][n_rows] (nullable): sum over the row of the largest change of
 * P^_ij that a decision within relative margin cfg->amb_delta of a
 * threshold could make.  Returns 0, or -1 on a bad argument. */
int oracle_p_diagnostics(const oracle_attn_cfg* cfg, const uint16_t* q, const uint16_t* k,
                         const int64_t* strides, const int32_t* rows, int32_t n_rows, double gamma,
                         double* diag, double* amb);

#ifdef __cplusplus
}
#endif
#endif
