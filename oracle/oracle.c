/*
 * oracle.c -- plain, slow CPU reference for MXAttention's MXFP4 attention
 * forward.  TEST INFRASTRUCTURE ONLY (see oracle.h for who may call it).
 *
 * Every function follows the pages step by step; the citations name the page
 * ([P1] the MXAttention paper, [P2] the explainer page, [P3] the MatX
 * leaky-quantization page) and the section, equation or algorithm.
 *
 * Readings of points the pages leave open (each is also listed in the design
 * notes of the repository):
 *   - Rotation: Sylvester Hadamard H_d/sqrt(d) in natural order, no random
 *     signs, evaluated in binary32 with butterfly strides 1,2,..,d/2 and one
 *     final multiply by fl32(1/sqrt(d)).
 *   - Element rounding: nearest grid point, exact ties to the even code;
 *     a value that rounds to zero keeps its sign bit (code 8).
 *   - E8M0 exponent clamped to [-127, 127]; byte 255 is never produced.
 *   - Blocks: Q/K along the head dimension; V and P along tokens/keys, in
 *     32-element blocks aligned to token/key 0, tails padded with +0.
 *   - The softmax tile loop visits key tiles of width B_c in ascending order;
 *     a tile with no visible key for a row is skipped for that row.
 *   - alpha = 0 while the running max is still -infinity.
 *   - Causal: key j is visible to query i iff j <= i.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdlib.h>
#include <string.h>

/* E2M1 magnitudes in code order 0..7 [P1 Eq. 9, Eq. 67]. */
static const double GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_magnitude(int code) { return GRID[code & 7]; }

double oracle_e2m1_value(int code) {
  double v = GRID[code & 7];
  return (code & 8) ? -v : v;
}

/* Nearest E2M1 grid point of y >= 0 [P1 Eq. 10].  The nearest
 * neighbour is decided by comparing with the midpoint of two adjacent grid
 * points (the decision boundaries of Eq. 68), which is exact in binary64.
 * Above the last midpoint every value maps to the largest element, 6: this is
 * the saturation of Eq. 10. */
int oracle_e2m1_project(double y) {
  for (int c = 0; c < 7; ++c) {
    double mid = 0.5 * (GRID[c] + GRID[c + 1]);
    if (y < mid) return c;
    if (y == mid) return (c % 2 == 0) ? c : c + 1; /* tie: even code */
  }
  return 7;
}

/* Smallest integer e with M <= q * 2^e, i.e. ceil(log2(M/q)) [P1 Eq. 13].
 * The frexp estimate is corrected with exact power-of-two comparisons. */
static int ceil_log2_ratio(double M, double q) {
  int E;
  (void)frexp(M / q, &E);
  int e = E;
  while (M <= ldexp(q, e - 1)) --e;
  while (M > ldexp(q, e)) ++e;
  return e;
}

/* Largest integer k with q * 2^k <= M, i.e. floor(log2(M/q)). */
static int floor_log2_ratio(double M, double q) {
  int E;
  (void)frexp(M / q, &E);
  int k = E - 1;
  while (ldexp(q, k) > M) --k;
  while (ldexp(q, k + 1) <= M) ++k;
  return k;
}

int oracle_scale_exponent(double M, int rule, double q) {
  /* outside the precondition (M > 0 finite; q > 0 finite for the *_Q rules)
   * the searches below would not terminate: return 0 instead */
  if (!(M > 0.0) || !isfinite(M)) return 0;
  if ((rule == ORACLE_RULE_CEIL_Q || rule == ORACLE_RULE_FLOOR_Q) && (!(q > 0.0) || !isfinite(q))) return 0;
  switch (rule) {
    case ORACLE_RULE_UOS: /* UOS boundary q* = 29/4 [P1 Eq. 38-39, Alg. 1] */
      return ceil_log2_ratio(M, 7.25);
    case ORACLE_RULE_OCP: /* floor(log2 M) - e_max^elem, e_max^elem = 2 [P1 Eq. 11] */
      return floor_log2_ratio(M, 1.0) - 2;
    case ORACLE_RULE_CEIL_Q: /* [P1 Eq. 13] */
      return ceil_log2_ratio(M, q);
    case ORACLE_RULE_FLOOR_Q: /* [P1 Eq. 12] */
      return floor_log2_ratio(M, q) + 1;
    default:
      return 0;
  }
}

void oracle_scale_exponents(const double* M, int64_t n, int rule, double q, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_scale_exponent(M[i], rule, q);
}

/* [P1 Alg. 1]: block max M; an all-zero block gets sigma = 1 and zero
 * elements; otherwise sigma = 2^e from the rule, and each element is
 * sigma * Pi(v / sigma). */
int oracle_quantize_block(const double* x, int n, int rule, double q,
                          uint8_t* scale_byte, uint8_t* codes) {
  double M = 0.0;
  for (int i = 0; i < n; ++i)
    if (fabs(x[i]) > M) M = fabs(x[i]);
  int e = 0;
  if (M > 0.0) {
    e = oracle_scale_exponent(M, rule, q);
    if (e < -127) e = -127;
    if (e > 127) e = 127;
  }
  *scale_byte = (uint8_t)(e + 127);
  for (int i = 0; i < n; ++i) {
    int c = oracle_e2m1_project(ldexp(fabs(x[i]), -e));
    codes[i] = (uint8_t)(c | (signbit(x[i]) ? 8 : 0));
  }
  return e;
}

static double dequant(uint8_t code, uint8_t scale_byte) {
  return ldexp(oracle_e2m1_value(code), (int)scale_byte - 127);
}

float oracle_decode_half(uint16_t bits, int dtype) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)bits << 16; /* bfloat16 is the top half of binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
  }
  /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */
  int s = bits >> 15, E = (bits >> 10) & 31, F = bits & 1023;
  double v;
  if (E == 0) v = ldexp((double)F, -24);
  else if (E == 31) v = F ? NAN : INFINITY;
  else v = ldexp((double)(F + 1024), E - 25);
  return (float)(s ? -v : v);
}

void oracle_hadamard_rotate_f32(float* x, int d) {
  for (int h = 1; h < d; h <<= 1)
    for (int i = 0; i < d; ++i)
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  const float r = (float)(1.0 / sqrt((double)d));
  for (int i = 0; i < d; ++i) x[i] = x[i] * r;
}

/* ------------------------------------------------------------------ */
/* small thread pool: workers pull item indices from an atomic counter  */

typedef void (*item_fn)(void* ctx, int64_t item, void* scratch);

typedef struct {
  item_fn fn;
  void* ctx;
  int64_t n_items;
  size_t scratch_bytes;
  atomic_llong next;
  atomic_int failed;
} pool_t;

static void* pool_worker(void* arg) {
  pool_t* p = (pool_t*)arg;
  void* scratch = p->scratch_bytes ? malloc(p->scratch_bytes) : NULL;
  if (p->scratch_bytes && !scratch) {
    atomic_store(&p->failed, 1);
    return NULL;
  }
  for (;;) {
    int64_t it = atomic_fetch_add(&p->next, 1);
    if (it >= p->n_items) break;
    p->fn(p->ctx, it, scratch);
  }
  free(scratch);
  return NULL;
}

static int run_pool(item_fn fn, void* ctx, int64_t n_items, size_t scratch_bytes, int nthreads) {
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.n_items = n_items;
  p.scratch_bytes = scratch_bytes;
  atomic_init(&p.next, 0);
  atomic_init(&p.failed, 0);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_items) nthreads = (int)(n_items > 0 ? n_items : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -1;
  int started = 0;
  for (int t = 0; t < nthreads; ++t)
    if (pthread_create(&th[t], NULL, pool_worker, &p) == 0) ++started;
  if (started == 0) pool_worker(&p);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  return atomic_load(&p.failed) ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* tensor quantization                                                  */

typedef struct {
  const uint16_t* x;
  int dtype, B, H, N, d, rotate, rule;
  double q;
  int64_t sB, sH, sN;
  const int64_t* rows;
  uint8_t* codes;
  uint8_t* scales;
} qrows_ctx;

static void strides_or_contig(const int64_t* strides, int H, int N, int d, int64_t* sB, int64_t* sH,
                              int64_t* sN) {
  if (strides) {
    *sB = strides[0];
    *sH = strides[1];
    *sN = strides[2];
  } else {
    *sN = d;
    *sH = (int64_t)N * d;
    *sB = (int64_t)H * N * d;
  }
}

/* One Q/K row: decode, optionally rotate (binary32), then quantize each
 * 32-channel block along the head dimension [P1 Alg. 2]. */
static void quantize_row(const qrows_ctx* c, int64_t g, uint8_t* codes, uint8_t* scales, float* buf) {
  int64_t bh = g / c->N, n = g % c->N;
  int64_t b = bh / c->H, h = bh % c->H;
  const uint16_t* src = c->x + b * c->sB + h * c->sH + n * c->sN;
  for (int i = 0; i < c->d; ++i) buf[i] = oracle_decode_half(src[i], c->dtype);
  if (c->rotate) oracle_hadamard_rotate_f32(buf, c->d);
  double blk[32];
  for (int k = 0; k < c->d / 32; ++k) {
    for (int i = 0; i < 32; ++i) blk[i] = (double)buf[32 * k + i];
    oracle_quantize_block(blk, 32, c->rule, c->q, &scales[k], &codes[32 * k]);
  }
}

static void qrows_item(void* ctx, int64_t it, void* scratch) {
  const qrows_ctx* c = (const qrows_ctx*)ctx;
  int64_t g = c->rows ? c->rows[it] : it;
  quantize_row(c, g, c->codes + it * c->d, c->scales + it * (c->d / 32), (float*)scratch);
}

static int shape_ok(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 32) return 0;
  if ((d & (d - 1)) != 0) return 0; /* the Sylvester construction needs a power of two */
  return 1;
}

int oracle_quantize_rows(const uint16_t* x, int dtype, int B, int H, int N, int d,
                         const int64_t* strides, int rotate, int rule, double q,
                         const int64_t* rows, int64_t n_rows,
                         uint8_t* codes, uint8_t* scales, int nthreads) {
  if (!x || !codes || !scales || !shape_ok(B, H, N, d) || n_rows < 0) return -1;
  qrows_ctx c = {x, dtype, B, H, N, d, rotate, rule, q, 0, 0, 0, rows, codes, scales};
  strides_or_contig(strides, H, N, d, &c.sB, &c.sH, &c.sN);
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= (int64_t)B * H * N) return -1;
  return run_pool(qrows_item, &c, n_rows, sizeof(float) * (size_t)d, nthreads);
}

typedef struct {
  const uint16_t* x;
  int dtype, B, H, N, d, rule;
  double q;
  int64_t sB, sH, sN, NB;
  const int64_t* blocks;
  uint8_t* codes;
  uint8_t* scales;
} qblk_ctx;

/* One V token block: for every channel, the 32 tokens 32*kb..32*kb+31
 * (+0 past the end) form one MXFP4 block [P3, Quantizing attention]. */
static void qblk_item(void* ctx, int64_t it, void* scratch) {
  (void)scratch;
  const qblk_ctx* c = (const qblk_ctx*)ctx;
  int64_t gb = c->blocks ? c->blocks[it] : it;
  int64_t bh = gb / c->NB, kb = gb % c->NB;
  int64_t b = bh / c->H, h = bh % c->H;
  const uint16_t* base = c->x + b * c->sB + h * c->sH;
  double blk[32];
  for (int ch = 0; ch < c->d; ++ch) {
    for (int t = 0; t < 32; ++t) {
      int64_t n = 32 * kb + t;
      blk[t] = n < c->N ? (double)oracle_decode_half(base[n * c->sN + ch], c->dtype) : 0.0;
    }
    oracle_quantize_block(blk, 32, c->rule, c->q, &c->scales[it * c->d + ch],
                          &c->codes[(it * c->d + ch) * 32]);
  }
}

int oracle_quantize_token_blocks(const uint16_t* x, int dtype, int B, int H, int N, int d,
                                 const int64_t* strides, int rule, double q,
                                 const int64_t* blocks, int64_t n_blocks,
                                 uint8_t* codes, uint8_t* scales, int nthreads) {
  if (!x || !codes || !scales || !shape_ok(B, H, N, d) || n_blocks < 0) return -1;
  qblk_ctx c = {x, dtype, B, H, N, d, rule, q, 0, 0, 0, (N + 31) / 32, blocks, codes, scales};
  strides_or_contig(strides, H, N, d, &c.sB, &c.sH, &c.sN);
  if (blocks)
    for (int64_t r = 0; r < n_blocks; ++r)
      if (blocks[r] < 0 || blocks[r] >= (int64_t)B * H * c.NB) return -1;
  return run_pool(qblk_item, &c, n_blocks, 0, nthreads);
}

/* ------------------------------------------------------------------ */
/* Q_max sweep                                                          */

typedef struct {
  const uint16_t* x;
  int dtype, B, H, N, d, axis, rotate, n_q;
  const double* qs;
  int64_t sB, sH, sN;
  const int64_t* heads;
  double* sse;
} sweep_ctx;

/* squared error of one block quantized with e = ceil(log2(M/q)), added to acc */
static double block_sse(const double* blk, double q) {
  uint8_t codes[32], sb;
  oracle_quantize_block(blk, 32, ORACLE_RULE_CEIL_Q, q, &sb, codes);
  double s = 0.0;
  for (int i = 0; i < 32; ++i) {
    const double r = blk[i] - dequant(codes[i], sb);
    s += r * r;
  }
  return s;
}

/* One head: every block of the tensor the quantizer sees, in row (or token
 * block, then channel) order, each quantized once per boundary q_j. */
static void sweep_item(void* ctx, int64_t it, void* scratch) {
  const sweep_ctx* c = (const sweep_ctx*)ctx;
  const int64_t bh = c->heads ? c->heads[it] : it;
  const int64_t b = bh / c->H, h = bh % c->H;
  const uint16_t* base = c->x + b * c->sB + h * c->sH;
  double* out = c->sse + it * c->n_q;
  float* buf = (float*)scratch;
  double blk[32];
  for (int j = 0; j < c->n_q; ++j) out[j] = 0.0;
  if (c->axis == ORACLE_AXIS_HEAD_DIM) {
    for (int n = 0; n < c->N; ++n) {
      for (int i = 0; i < c->d; ++i) buf[i] = oracle_decode_half(base[n * c->sN + i], c->dtype);
      if (c->rotate) oracle_hadamard_rotate_f32(buf, c->d);
      for (int k = 0; k < c->d / 32; ++k) {
        for (int i = 0; i < 32; ++i) blk[i] = (double)buf[32 * k + i];
        for (int j = 0; j < c->n_q; ++j) out[j] += block_sse(blk, c->qs[j]);
      }
    }
  } else {
    for (int kb = 0; kb < (c->N + 31) / 32; ++kb)
      for (int ch = 0; ch < c->d; ++ch) {
        for (int t = 0; t < 32; ++t) {
          const int64_t n = 32 * kb + t;
          blk[t] = n < c->N ? (double)oracle_decode_half(base[n * c->sN + ch], c->dtype) : 0.0;
        }
        for (int j = 0; j < c->n_q; ++j) out[j] += block_sse(blk, c->qs[j]);
      }
  }
}

int oracle_scale_sweep(const uint16_t* x, int dtype, int B, int H, int N, int d,
                       const int64_t* strides, int axis, int rotate, const double* qs, int n_q,
                       const int64_t* heads, int64_t n_heads, double* sse, int nthreads) {
  if (!x || !qs || !sse || !shape_ok(B, H, N, d) || n_q < 1 || n_heads < 0) return -1;
  if (axis != ORACLE_AXIS_HEAD_DIM && axis != ORACLE_AXIS_TOKEN) return -1;
  if (rotate && axis != ORACLE_AXIS_HEAD_DIM) return -1;
  for (int j = 0; j < n_q; ++j)
    if (!(qs[j] > 0.0) || !isfinite(qs[j])) return -1;
  sweep_ctx c = {x, dtype, B, H, N, d, axis, rotate, n_q, qs, 0, 0, 0, heads, sse};
  strides_or_contig(strides, H, N, d, &c.sB, &c.sH, &c.sN);
  if (heads)
    for (int64_t r = 0; r < n_heads; ++r)
      if (heads[r] < 0 || heads[r] >= (int64_t)B * H) return -1;
  return run_pool(sweep_item, &c, n_heads, sizeof(float) * (size_t)d, nthreads);
}

/* ------------------------------------------------------------------ */
/* attention                                                            */

typedef struct {
  const oracle_attn_cfg* cfg;
  const uint16_t *q, *k, *v;
  int64_t sB, sH, sN;     /* element strides of Q                  */
  int64_t kB, kH, kN;     /* element strides of K and V            */
  int32_t Nk;             /* key / value tokens                    */
  const int32_t* rows;
  int32_t n_rows;
  int32_t chunks_per_head, rows_per_chunk;
  double *out, *m_out, *l_out, *rowsum, *amb, *absmass, *amb_rowsum;
} attn_ctx;

/* Dequantized (or plain) K and V of one head, and the query row, in binary64. */
static void load_head_kv(const attn_ctx* c, int64_t b, int64_t h, double* K, double* V, float* buf,
                         uint8_t* codes, double* blk) {
  const oracle_attn_cfg* g = c->cfg;
  const int N = c->Nk, d = g->d;
  const uint16_t* kb = c->k + b * c->kB + h * c->kH;
  const uint16_t* vb = c->v + b * c->kB + h * c->kH;
  for (int j = 0; j < N; ++j) {
    for (int i = 0; i < d; ++i) buf[i] = oracle_decode_half(kb[(int64_t)j * c->kN + i], g->dtype);
    if (g->rotate) oracle_hadamard_rotate_f32(buf, d);
    if (g->quant) {
      for (int kk = 0; kk < d / 32; ++kk) {
        uint8_t sb;
        for (int i = 0; i < 32; ++i) blk[i] = (double)buf[32 * kk + i];
        oracle_quantize_block(blk, 32, g->rule, g->q, &sb, codes);
        for (int i = 0; i < 32; ++i) K[(int64_t)j * d + 32 * kk + i] = dequant(codes[i], sb);
      }
    } else {
      for (int i = 0; i < d; ++i) K[(int64_t)j * d + i] = (double)buf[i];
    }
  }
  if (g->quant) {
    /* V along tokens, 32-token blocks aligned to token 0, +0 padding [P3] */
    for (int kb32 = 0; kb32 < (N + 31) / 32; ++kb32)
      for (int ch = 0; ch < d; ++ch) {
        uint8_t sb;
        for (int t = 0; t < 32; ++t) {
          int n = 32 * kb32 + t;
          blk[t] = n < N ? (double)oracle_decode_half(vb[(int64_t)n * c->kN + ch], g->dtype) : 0.0;
        }
        oracle_quantize_block(blk, 32, g->rule, g->q, &sb, codes);
        for (int t = 0; t < 32; ++t) {
          int n = 32 * kb32 + t;
          if (n < N) V[(int64_t)n * d + ch] = dequant(codes[t], sb);
        }
      }
  } else {
    for (int j = 0; j < N; ++j)
      for (int ch = 0; ch < d; ++ch)
        V[(int64_t)j * d + ch] = (double)oracle_decode_half(vb[(int64_t)j * c->kN + ch], g->dtype);
  }
}

static void load_query(const attn_ctx* c, int64_t b, int64_t h, int i, double* qv, float* buf,
                       uint8_t* codes, double* blk) {
  const oracle_attn_cfg* g = c->cfg;
  const int d = g->d;
  const uint16_t* src = c->q + b * c->sB + h * c->sH + (int64_t)i * c->sN;
  for (int t = 0; t < d; ++t) buf[t] = oracle_decode_half(src[t], g->dtype);
  if (g->rotate) oracle_hadamard_rotate_f32(buf, d);
  if (g->quant) {
    for (int kk = 0; kk < d / 32; ++kk) {
      uint8_t sb;
      for (int t = 0; t < 32; ++t) blk[t] = (double)buf[32 * kk + t];
      oracle_quantize_block(blk, 32, g->rule, g->q, &sb, codes);
      for (int t = 0; t < 32; ++t) qv[32 * kk + t] = dequant(codes[t], sb);
    }
  } else {
    for (int t = 0; t < d; ++t) qv[t] = (double)buf[t];
  }
}

/* Quantize one 32-key block of exponentials p[0..31] (a tile segment, zeros
 * for keys that are masked or past N) [P1 Alg. 1 applied to P~, Eq. 44] and
 * return the dequantized values in ph.  If dp is given, also write into it
 * the largest change of each element that a decision lying within relative
 * margin delta of its threshold could make (the decision allowance):
 *   - an element whose normalized value p/2^e lies within delta of a
 *     rounding midpoint may round to the neighbouring grid point;
 *   - a block whose normalized maximum lies within delta of one end of the
 *     rule's range (lo, hi] may take the neighbouring exponent, and every
 *     element of the block is then re-projected.
 * The margin stands for the rounding of a binary32 evaluation of P~.  One
 * value is not subject to it: the exponential at the row maximum is
 * exp(0) = 1 exactly, and in the post-normalization mode P = 1/l* at the row
 * maximum lies below 1 exactly when l* > 1 (gamma P below gamma, for a
 * power-of-two gamma).  With exact_ref > 0, the block's maximum is that
 * element, known exactly relative to exact_ref (1 or gamma), so a scale
 * boundary equal to exact_ref (lo 2^e or hi 2^e, as OCP has at powers of two)
 * is not a close decision and offers no alternative.  Returns the block
 * exponent. */
int oracle_p_block_allowance(const double* p, int rule, double q, double delta, double exact_ref, double* ph,
                             double* dp) {
  uint8_t codes[32], sb;
  int e = oracle_quantize_block(p, 32, rule, q, &sb, codes);
  for (int t = 0; t < 32; ++t) ph[t] = dequant(codes[t], sb);
  if (!dp) return e;
  for (int t = 0; t < 32; ++t) {
    dp[t] = 0.0;
    double y = ldexp(p[t], -e);
    for (int c = 0; c < 7; ++c) {
      double mid = 0.5 * (GRID[c] + GRID[c + 1]);
      if (fabs(y - mid) <= delta * mid) {
        double step = ldexp(GRID[c + 1] - GRID[c], e);
        if (step > dp[t]) dp[t] = step;
      }
    }
  }
  double M = 0.0;
  for (int t = 0; t < 32; ++t)
    if (p[t] > M) M = p[t];
  if (M <= 0.0) return e;
  /* normalized block max and the two ends of its admissible interval */
  double r = ldexp(M, -e), hi, lo;
  switch (rule) {
    case ORACLE_RULE_UOS: hi = 7.25; lo = 3.625; break;
    case ORACLE_RULE_OCP: hi = 8.0; lo = 4.0; break;
    default: hi = q; lo = 0.5 * q; break; /* ceiling rule: M/2^e in (q/2, q] */
  }
  int alts[2], na = 0;
  if (fabs(r - hi) <= delta * hi && e < 127 && !(ldexp(hi, e) == exact_ref)) alts[na++] = e + 1;
  if (fabs(r - lo) <= delta * lo && e > -127 && !(ldexp(lo, e) == exact_ref)) alts[na++] = e - 1;
  for (int a = 0; a < na; ++a) {
    int ea = alts[a];
    for (int t = 0; t < 32; ++t) {
      double alt = ldexp(GRID[oracle_e2m1_project(ldexp(p[t], -ea))], ea);
      double diff = fabs(alt - ph[t]);
      if (diff > dp[t]) dp[t] = diff;
    }
  }
  return e;
}

static int quantize_p_block(const oracle_attn_cfg* g, const double* p, double exact_ref, double* ph, double* dp) {
  return oracle_p_block_allowance(p, g->rule, g->q, g->amb_delta, exact_ref, ph, dp);
}

/* Whether the row maximum s1 stands alone: the runner-up s2 (-inf if none)
 * gives exp(s2 - s1) < 1 - delta, so a binary32 evaluation of the scores
 * cannot make another key the maximum.  An exact tie of two keys is not
 * alone either. */
static int max_stands_alone(double s1, double s2, double delta) {
  return s2 == -INFINITY || exp(s2 - s1) < 1.0 - delta;
}

/* Smallest mass rho = l* - 1 of the keys other than the row maximum that a
 * binary32 sum of binary32 exponentials still sees as nonzero: with at most
 * 2^17 keys, rho >= 2^-100 has a term >= 2^-117, a normal binary32. */
#define ORACLE_RHO_VISIBLE 0x1p-100

static void attn_item(void* vctx, int64_t item, void* scratch_raw) {
  const attn_ctx* c = (const attn_ctx*)vctx;
  const oracle_attn_cfg* g = c->cfg;
  const int N = c->Nk, d = g->d, Bc = g->kv_tile;  /* N: keys of the row */
  const int T = (N + Bc - 1) / Bc;
  const int64_t bh = item / c->chunks_per_head;
  const int chunk = (int)(item % c->chunks_per_head);
  const int64_t b = bh / g->H, h = bh % g->H;
  int r0 = chunk * c->rows_per_chunk, r1 = r0 + c->rows_per_chunk;
  if (r1 > c->n_rows) r1 = c->n_rows;
  if (r0 >= r1) return;

  /* scratch layout */
  char* s = (char*)scratch_raw;
  double* K = (double*)s;  s += sizeof(double) * (size_t)N * d;
  double* V = (double*)s;  s += sizeof(double) * (size_t)N * d;
  double* qv = (double*)s; s += sizeof(double) * d;
  double* o = (double*)s;  s += sizeof(double) * d;
  double* ao = (double*)s; s += sizeof(double) * d;
  double* am = (double*)s; s += sizeof(double) * d;  /* sum of |P^ V^| terms */
  double* sc = (double*)s; s += sizeof(double) * (size_t)N;   /* scores of the row  */
  double* pt = (double*)s; s += sizeof(double) * (size_t)(T * Bc); /* P~ (tile-padded) */
  double* ph = (double*)s; s += sizeof(double) * (size_t)(T * Bc); /* P^              */
  double* dp = (double*)s; s += sizeof(double) * (size_t)(T * Bc); /* allowance       */
  double* tm = (double*)s; s += sizeof(double) * T;  /* m after tile t           */
  double* th = (double*)s; s += sizeof(double) * T;  /* sum of P^ over tile t    */
  double* tt = (double*)s; s += sizeof(double) * T;  /* sum of P~ over tile t    */
  double* tdl = (double*)s; s += sizeof(double) * T; /* allowance of tile t's sum of P^ */
  double* blk = (double*)s; s += sizeof(double) * 32;
  float* buf = (float*)s;  s += sizeof(float) * d;
  uint8_t* codes = (uint8_t*)s;

  load_head_kv(c, b, h, K, V, buf, codes, blk);

  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  const int quantize_p = g->quant && g->p_mode != ORACLE_P_EXACT;
  const int want_amb = c->amb && quantize_p && g->amb_delta > 0.0;

  for (int r = r0; r < r1; ++r) {
    const int i = c->rows ? c->rows[r] : r;
    load_query(c, b, h, i, qv, buf, codes, blk);
    const int jvis = g->causal ? (i + 1 < N ? i + 1 : N) : N; /* keys [0, jvis) visible */
    /* S_ij = q^ . k^_j / sqrt(d) [P1 Eq. 2, Alg. 2] */
    for (int j = 0; j < jvis; ++j) {
      double acc = 0.0;
      for (int t = 0; t < d; ++t) acc += qv[t] * K[(int64_t)j * d + t];
      sc[j] = acc * inv_sqrt_d;
    }
    double* orow = c->out + (bh * c->n_rows + r) * d;
    double* arow = c->amb ? c->amb + (bh * c->n_rows + r) * d : NULL;
    double* mrow = c->absmass ? c->absmass + (bh * c->n_rows + r) * d : NULL;
    const int64_t ridx = bh * c->n_rows + r;
    for (int t = 0; t < d; ++t) { o[t] = 0.0; ao[t] = 0.0; am[t] = 0.0; }

    if (g->p_mode == ORACLE_P_POSTNORM && g->quant) {
      /* Materialized-P diagnostic [P1 Sec. 5.5.2]: exact softmax first, then
       * quantize the normalized probabilities in aligned 32-key blocks and
       * accumulate O = Q(P) V^ with no renormalization. */
      double ms = -INFINITY, s2 = -INFINITY, ls = 0.0, rho = 0.0;
      int jmax = 0;
      for (int j = 0; j < jvis; ++j) {
        if (sc[j] > ms) { s2 = ms; ms = sc[j]; jmax = j; }
        else if (sc[j] > s2) s2 = sc[j];
      }
      for (int j = 0; j < jvis; ++j) ls += exp(sc[j] - ms);
      /* rho = l* - 1, summed without the maximum's exp(0) = 1 so that a tiny
       * rho keeps its relative precision */
      for (int j = 0; j < jvis; ++j) if (j != jmax) rho += exp(sc[j] - ms);
      /* P at the row maximum, 1/l*, is below 1 exactly when rho > 0: an
       * exact decision while rho stays visible in binary32 and no other key
       * ties the maximum */
      const int exact_max = max_stands_alone(ms, s2, g->amb_delta) && rho >= ORACLE_RHO_VISIBLE && rho < 1.0;
      /* P at the row maximum is 1/l* = 1/(1 + rho), strictly below 1 when
       * rho > 0; for rho < 2^-53 binary64 rounds it up to 1, onto OCP's
       * scale boundary.  The largest binary64 below 1 stands in for it: no
       * threshold of the block quantizer lies between the two. */
      const double pmax = (rho > 0.0 && 1.0 / ls == 1.0) ? nextafter(1.0, 0.0) : 1.0 / ls;
      double sum_hat = 0.0, sum_dp = 0.0;
      for (int j0 = 0; j0 < jvis; j0 += 32) {
        double pb[32], hb[32], db[32];
        for (int t = 0; t < 32; ++t)
          pb[t] = (j0 + t >= jvis) ? 0.0 : (j0 + t == jmax ? pmax : exp(sc[j0 + t] - ms) / ls);
        quantize_p_block(g, pb, (exact_max && jmax >= j0 && jmax < j0 + 32) ? 1.0 : 0.0, hb, want_amb ? db : NULL);
        for (int t = 0; t < 32 && j0 + t < jvis; ++t) {
          sum_hat += hb[t];
          for (int ch = 0; ch < d; ++ch) o[ch] += hb[t] * V[(int64_t)(j0 + t) * d + ch];
          for (int ch = 0; ch < d; ++ch) am[ch] += hb[t] * fabs(V[(int64_t)(j0 + t) * d + ch]);
          if (want_amb) {
            sum_dp += db[t];
            for (int ch = 0; ch < d; ++ch) ao[ch] += db[t] * fabs(V[(int64_t)(j0 + t) * d + ch]);
          }
        }
      }
      for (int ch = 0; ch < d; ++ch) orow[ch] = o[ch];
      if (mrow) for (int ch = 0; ch < d; ++ch) mrow[ch] = am[ch];
      if (arow) for (int ch = 0; ch < d; ++ch) arow[ch] = want_amb ? ao[ch] : 0.0;
      if (c->m_out) c->m_out[ridx] = ms;
      if (c->l_out) c->l_out[ridx] = ls;
      if (c->rowsum) c->rowsum[ridx] = sum_hat;
      /* the induced row sum is sum_j P^_ij itself: a decision moves it by its own change */
      if (c->amb_rowsum) c->amb_rowsum[ridx] = want_amb ? sum_dp : 0.0;
      continue;
    }

    /* Online softmax over key tiles in ascending order [P1 Alg. 2;
     * Eqs. 3-7 with Eqs. 44-48 (PNQ) or Eq. 42 (direct)]. */
    double m = -INFINITY, l = 0.0, al = 0.0;
    double s2 = -INFINITY; /* runner-up of the scores seen so far */
    int ntiles_seen = 0;
    for (int tile = 0; tile < T; ++tile) {
      const int j0 = tile * Bc;
      int j1 = j0 + Bc < jvis ? j0 + Bc : jvis;
      tm[tile] = -INFINITY; th[tile] = 0.0; tt[tile] = 0.0; tdl[tile] = 0.0;
      if (j1 <= j0) continue; /* no visible key for this row: a no-op */
      ++ntiles_seen;
      double smax = -INFINITY;
      for (int j = j0; j < j1; ++j) if (sc[j] > smax) smax = sc[j];
      const double m_new = m > smax ? m : smax;                 /* Eq. 3  */
      {
        /* runner-up over every key seen so far (tiles 0..tile) */
        double s1 = m;
        for (int j = j0; j < j1; ++j) {
          if (sc[j] > s1) { s2 = s1; s1 = sc[j]; }
          else if (sc[j] > s2) s2 = sc[j];
        }
      }
      /* keys at the running maximum have P~ = exp(0) = 1 exactly */
      const int alone = max_stands_alone(m_new, s2, g->amb_delta);
      const double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new); /* Eq. 4 */
      double* P = pt + j0;
      double* Ph = ph + j0;
      double* D = dp + j0;
      for (int t = 0; t < Bc; ++t) P[t] = (j0 + t < j1) ? exp(sc[j0 + t] - m_new) : 0.0; /* Eq. 5 */
      for (int t0 = 0; t0 < Bc; t0 += 32) {
        int one = 0; /* the block holds the running maximum */
        for (int t = t0; t < t0 + 32; ++t) one |= (j0 + t < j1 && sc[j0 + t] == m_new);
        if (quantize_p) quantize_p_block(g, P + t0, (alone && one) ? 1.0 : 0.0, Ph + t0, want_amb ? D + t0 : NULL); /* Eq. 44 */
        else for (int t = 0; t < 32; ++t) Ph[t0 + t] = P[t0 + t];
      }
      double sum_hat = 0.0, sum_til = 0.0;
      for (int t = 0; t < Bc; ++t) { sum_hat += Ph[t]; sum_til += P[t]; }
      /* l update: Eq. 47 (PNQ) or Eq. 16 / Eq. 42 (direct) */
      l = alpha * l + ((g->p_mode == ORACLE_P_DIRECT && quantize_p) ? sum_til : sum_hat);
      /* O update: Eq. 48 / Eq. 17 */
      for (int ch = 0; ch < d; ++ch) { o[ch] *= alpha; am[ch] *= alpha; }
      for (int j = j0; j < j1; ++j) {
        const double w = Ph[j - j0];
        if (w != 0.0)
          for (int ch = 0; ch < d; ++ch) {
            o[ch] += w * V[(int64_t)j * d + ch];
            am[ch] += w * fabs(V[(int64_t)j * d + ch]);
          }
      }
      if (want_amb) {
        double dl = 0.0;
        for (int ch = 0; ch < d; ++ch) ao[ch] *= alpha;
        for (int j = j0; j < j1; ++j) {
          const double w = D[j - j0];
          if (w != 0.0) {
            dl += w;
            for (int ch = 0; ch < d; ++ch) ao[ch] += w * fabs(V[(int64_t)j * d + ch]);
          }
        }
        al = alpha * al + dl;
        tdl[tile] = dl;
      }
      tm[tile] = m_new; th[tile] = sum_hat; tt[tile] = sum_til;
      m = m_new;                                     /* the running maximum moves on */
    }
    (void)ntiles_seen;
    /* O_i = o / l  [Eq. 8; Alg. 2]; POSTNORM without quantization
     * reduces to the same exact softmax attention. */
    for (int ch = 0; ch < d; ++ch) orow[ch] = o[ch] / l;
    if (mrow) for (int ch = 0; ch < d; ++ch) mrow[ch] = am[ch] / l;
    if (arow) {
      for (int ch = 0; ch < d; ++ch) {
        if (!want_amb) arow[ch] = 0.0;
        else if (g->p_mode == ORACLE_P_DIRECT) arow[ch] = ao[ch] / l;
        else arow[ch] = (l > al) ? (ao[ch] + fabs(orow[ch]) * al) / (l - al) : INFINITY;
      }
    }
    if (c->m_out) c->m_out[ridx] = m;
    if (c->l_out) c->l_out[ridx] = l;
    if (c->rowsum || c->amb_rowsum) {
      /* effective full-row form: beta_t = exp(m_t - m_final) [App. H Eq. 99] */
      double num = 0.0, den = 0.0, anum = 0.0;
      for (int tile = 0; tile < T; ++tile) {
        if (tm[tile] == -INFINITY) continue;
        const double beta = exp(tm[tile] - m);
        num += beta * th[tile];
        den += beta * tt[tile];
        anum += beta * tdl[tile];
      }
      const int direct_q = g->p_mode == ORACLE_P_DIRECT && quantize_p;
      if (c->rowsum) c->rowsum[ridx] = direct_q ? num / den : num / l; /* Eq. 110 / Eq. 51 */
      /* DIRECT: the decisions move only the numerator (by beta-weighted tile
       * allowances); PNQ: the row sum is 1 whatever they decide */
      if (c->amb_rowsum) c->amb_rowsum[ridx] = (want_amb && direct_q) ? anum / den : 0.0;
    }
  }
}

int oracle_attention(const oracle_attn_cfg* cfg,
                     const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const int64_t* strides, const int32_t* rows, int32_t n_rows,
                     double* out, double* m_out, double* l_out, double* rowsum,
                     double* amb, double* absmass, double* amb_rowsum) {
  if (!cfg || !q || !k || !v || !out) return -1;
  if (!shape_ok(cfg->B, cfg->H, cfg->N, cfg->d)) return -1;
  if (cfg->kv_tile < 32 || cfg->kv_tile % 32 != 0) return -1;
  if (cfg->p_mode < 0 || cfg->p_mode > 3) return -1;
  if (!rows) n_rows = cfg->N;
  if (n_rows < 1) return -1;
  /* cross-attention: Nk keys and values; causal masking needs Nk = N, and
   * caller strides describe one shape, so they need Nk = N too */
  const int Nk = cfg->Nk > 0 ? cfg->Nk : cfg->N;
  if (cfg->Nk < 0 || (Nk != cfg->N && (cfg->causal || strides))) return -1;
  if (!shape_ok(cfg->B, cfg->H, Nk, cfg->d)) return -1;
  if (rows)
    for (int r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= cfg->N) return -1;
  attn_ctx c;
  memset(&c, 0, sizeof c);
  c.cfg = cfg;
  c.q = q; c.k = k; c.v = v;
  strides_or_contig(strides, cfg->H, cfg->N, cfg->d, &c.sB, &c.sH, &c.sN);
  strides_or_contig(strides, cfg->H, Nk, cfg->d, &c.kB, &c.kH, &c.kN);
  c.Nk = Nk;
  c.rows = rows;
  c.n_rows = n_rows;
  c.out = out; c.m_out = m_out; c.l_out = l_out; c.rowsum = rowsum; c.amb = amb;
  c.absmass = absmass;
  c.amb_rowsum = amb_rowsum;
  const int64_t heads = (int64_t)cfg->B * cfg->H;
  int nth = cfg->nthreads > 0 ? cfg->nthreads : 1;
  int cph = (int)((2 * (int64_t)nth + heads - 1) / heads);
  if (cph < 1) cph = 1;
  if (cph > n_rows) cph = n_rows;
  c.chunks_per_head = cph;
  c.rows_per_chunk = (n_rows + cph - 1) / cph;
  const int N = Nk, d = cfg->d, T = (N + cfg->kv_tile - 1) / cfg->kv_tile;
  size_t scratch = sizeof(double) * ((size_t)2 * N * d + 4 * (size_t)d + N + 3 * (size_t)T * cfg->kv_tile +
                                     4 * (size_t)T + 32) +
                   sizeof(float) * d + 64;
  return run_pool(attn_item, &c, heads * cph, scratch, nth);
}

/* ------------------------------------------------------------------ */
/* materialized-P row-sum diagnostics                                   */

typedef struct {
  const oracle_attn_cfg* cfg;
  const uint16_t *q, *k;
  int64_t sB, sH, sN;
  const int32_t* rows;
  int32_t n_rows;
  int32_t chunks_per_head, rows_per_chunk;
  double gamma;
  double *diag, *amb;
} diag_ctx;

/* One chunk of rows of one head [P1 Sec. 5.5.2, Fig. 7]: the exact softmax
 * row P_i. = exp(S_i. - m) / l over the visible keys, then P^ = Q(gamma P) /
 * gamma with the block quantizer on aligned 32-key blocks (a pre-quantization
 * global scale gamma, 1 for the plain diagnostic, Fig. 7 (C)).  The row-sum
 * error sum_j (P^ - P) is split by the outcome of each element: zeroing
 * (P > 0, P^ = 0), saturation (gamma P / 2^e beyond the largest grid value
 * 6), and otherwise downward (P^ < P) or upward (P^ > P) rounding; plus the
 * row's entropy -sum P ln P (nats, Fig. 7 (D)). */
static void diag_item(void* vctx, int64_t item, void* scratch_raw) {
  const diag_ctx* c = (const diag_ctx*)vctx;
  const oracle_attn_cfg* g = c->cfg;
  const int N = g->N, d = g->d;
  const int64_t bh = item / c->chunks_per_head;
  const int chunk = (int)(item % c->chunks_per_head);
  const int64_t b = bh / g->H, h = bh % g->H;
  int r0 = chunk * c->rows_per_chunk, r1 = r0 + c->rows_per_chunk;
  if (r1 > c->n_rows) r1 = c->n_rows;
  if (r0 >= r1) return;
  char* s = (char*)scratch_raw;
  double* K = (double*)s;  s += sizeof(double) * (size_t)N * d;
  double* V = (double*)s;  s += sizeof(double) * (size_t)N * d;
  double* qv = (double*)s; s += sizeof(double) * d;
  double* sc = (double*)s; s += sizeof(double) * (size_t)N;
  double* blk = (double*)s; s += sizeof(double) * 32;
  float* buf = (float*)s;  s += sizeof(float) * d;
  uint8_t* codes = (uint8_t*)s;
  attn_ctx ac;
  memset(&ac, 0, sizeof ac);
  ac.cfg = g; ac.q = c->q; ac.k = c->k; ac.v = c->k;
  ac.sB = c->sB; ac.sH = c->sH; ac.sN = c->sN;
  ac.kB = c->sB; ac.kH = c->sH; ac.kN = c->sN; ac.Nk = N;
  load_head_kv(&ac, b, h, K, V, buf, codes, blk);
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  for (int r = r0; r < r1; ++r) {
    const int i = c->rows ? c->rows[r] : r;
    load_query(&ac, b, h, i, qv, buf, codes, blk);
    const int jvis = g->causal ? (i + 1 < N ? i + 1 : N) : N;
    double ms = -INFINITY, s2 = -INFINITY, ls = 0.0, rho = 0.0;
    int jmax = 0;
    for (int j = 0; j < jvis; ++j) {
      double acc = 0.0;
      for (int t = 0; t < d; ++t) acc += qv[t] * K[(int64_t)j * d + t];
      sc[j] = acc * inv_sqrt_d;
      if (sc[j] > ms) { s2 = ms; ms = sc[j]; jmax = j; }
      else if (sc[j] > s2) s2 = sc[j];
    }
    for (int j = 0; j < jvis; ++j) ls += exp(sc[j] - ms);
    for (int j = 0; j < jvis; ++j) if (j != jmax) rho += exp(sc[j] - ms);
    /* gamma P at the row maximum is gamma / l*, below gamma exactly when
     * rho = l* - 1 > 0; for a power-of-two gamma that is an exact decision
     * while rho stays visible in binary32 and no other key ties the maximum
     * (see oracle_p_block_allowance) */
    int gexp;
    const int gamma_pow2 = frexp(c->gamma, &gexp) == 0.5;
    const int exact_max = gamma_pow2 && max_stands_alone(ms, s2, g->amb_delta) && rho >= ORACLE_RHO_VISIBLE &&
                          rho < 1.0;
    /* P at the row maximum: 1/(1 + rho), kept below 1 when rho > 0 (see the
     * post-normalization mode of the attention forward) */
    const double pmax = (rho > 0.0 && 1.0 / ls == 1.0) ? nextafter(1.0, 0.0) : 1.0 / ls;
    double out[6] = {0, 0, 0, 0, 0, 0}, amb = 0.0;
    for (int j0 = 0; j0 < jvis; j0 += 32) {
      double P[32], gp[32], hb[32], db[32];
      for (int t = 0; t < 32; ++t) {
        P[t] = (j0 + t >= jvis) ? 0.0 : (j0 + t == jmax ? pmax : exp(sc[j0 + t] - ms) / ls);
        gp[t] = c->gamma * P[t];
      }
      const int e = quantize_p_block(g, gp, (exact_max && jmax >= j0 && jmax < j0 + 32) ? c->gamma : 0.0, hb,
                                     c->amb ? db : NULL);
      for (int t = 0; t < 32 && j0 + t < jvis; ++t) {
        const double ph = hb[t] / c->gamma, diff = ph - P[t];
        out[0] += ph;
        if (P[t] > 0.0 && ph == 0.0) out[1] += diff;
        else if (ldexp(gp[t], -e) > 6.0) out[2] += diff;
        else if (diff < 0.0) out[3] += diff;
        else if (diff > 0.0) out[4] += diff;
        if (P[t] > 0.0) out[5] -= P[t] * log(P[t]);
        if (c->amb) amb += db[t] / c->gamma;
      }
    }
    const int64_t ridx = bh * c->n_rows + r;
    for (int k = 0; k < 6; ++k) c->diag[ridx * 6 + k] = out[k];
    if (c->amb) c->amb[ridx] = amb;
  }
}

int oracle_p_diagnostics(const oracle_attn_cfg* cfg, const uint16_t* q, const uint16_t* k,
                         const int64_t* strides, const int32_t* rows, int32_t n_rows, double gamma,
                         double* diag, double* amb) {
  if (!cfg || !q || !k || !diag) return -1;
  if (!shape_ok(cfg->B, cfg->H, cfg->N, cfg->d)) return -1;
  if (!(gamma > 0.0) || !isfinite(gamma) || !cfg->quant) return -1;
  if (cfg->rule != ORACLE_RULE_UOS && cfg->rule != ORACLE_RULE_OCP) return -1;
  if (!rows) n_rows = cfg->N;
  if (n_rows < 1) return -1;
  if (rows)
    for (int r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= cfg->N) return -1;
  diag_ctx c;
  memset(&c, 0, sizeof c);
  c.cfg = cfg; c.q = q; c.k = k;
  strides_or_contig(strides, cfg->H, cfg->N, cfg->d, &c.sB, &c.sH, &c.sN);
  c.rows = rows; c.n_rows = n_rows; c.gamma = gamma; c.diag = diag; c.amb = amb;
  const int64_t heads = (int64_t)cfg->B * cfg->H;
  int nth = cfg->nthreads > 0 ? cfg->nthreads : 1;
  int cph = (int)((2 * (int64_t)nth + heads - 1) / heads);
  if (cph < 1) cph = 1;
  if (cph > n_rows) cph = n_rows;
  c.chunks_per_head = cph;
  c.rows_per_chunk = (n_rows + cph - 1) / cph;
  const int N = cfg->N, d = cfg->d;
  size_t scratch = sizeof(double) * ((size_t)2 * N * d + d + N + 32) + sizeof(float) * d + 64;
  return run_pool(diag_item, &c, heads * cph, scratch, nth);
}
