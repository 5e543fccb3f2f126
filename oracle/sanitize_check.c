/*
 * sanitize_check.c -- test infrastructure for the CPU oracle (oracle.c).
 *
 * A small driver that calls every oracle entry point on small synthetic
 * inputs (ragged token counts, strided inputs, self- and cross-attention,
 * causal masks, every P placement and scale rule, the sweep and the
 * diagnostics, and arguments the oracle must reject).  tests/ builds it
 * together with oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer
 * (gcc, host code only) and runs it: any out-of-bounds access, use of freed
 * memory, leak or undefined operation in the oracle aborts the run.  It
 * checks return codes only; the values are pinned elsewhere.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;

static double next_unit(void) {  /* uniform in [0, 1) */
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg_state >> 11) * (1.0 / 9007199254740992.0);
}

/* bf16 bit pattern of v, rounded to nearest even (v finite) */
static uint16_t to_bf16(float v) {
  uint32_t b;
  memcpy(&b, &v, sizeof b);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* n values: mostly N(0, s)-like, some zeros, subnormals and large values */
static uint16_t* make_input(size_t n, double s) {
  uint16_t* x = (uint16_t*)malloc(n * sizeof(uint16_t));
  if (!x) exit(3);
  for (size_t i = 0; i < n; ++i) {
    const double u = next_unit();
    double v = (next_unit() + next_unit() + next_unit() - 1.5) * 2.0 * s;
    if (u < 0.03) v = 0.0;
    else if (u < 0.05) v = ldexp(v, -130);
    else if (u < 0.06) v *= 1e4;
    x[i] = to_bf16((float)v);
  }
  return x;
}

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: returned %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static void check_quantizers(void) {
  const int B = 1, H = 2, N = 37, d = 64;
  /* strided input: rows of 96 elements, heads of 40 rows */
  const int64_t strides[3] = {(int64_t)H * 40 * 96, 40 * 96, 96};
  uint16_t* x = make_input((size_t)B * H * 40 * 96, 2.0);
  const int64_t nr = (int64_t)B * H * N;
  uint8_t* codes = (uint8_t*)malloc((size_t)nr * d);
  uint8_t* scales = (uint8_t*)malloc((size_t)nr * (d / 32));
  for (int rule = 0; rule <= 3; ++rule)
    for (int rotate = 0; rotate <= 1; ++rotate)
      expect(oracle_quantize_rows(x, ORACLE_BF16, B, H, N, d, strides, rotate, rule, 6.5, NULL, nr, codes, scales, 3),
             0, "quantize_rows");
  const int64_t rows[4] = {0, 5, N - 1, 2 * N - 1};
  expect(oracle_quantize_rows(x, ORACLE_FP16, B, H, N, d, strides, 1, ORACLE_RULE_UOS, 0.0, rows, 4, codes, scales, 2),
         0, "quantize_rows subset");
  expect(oracle_quantize_rows(x, ORACLE_BF16, B, H, N, 96, NULL, 1, ORACLE_RULE_UOS, 0.0, NULL, nr, codes, scales, 1),
         -1, "quantize_rows d=96");

  const int NB = (N + 31) / 32;
  const int64_t nb = (int64_t)B * H * NB;
  uint8_t* tcodes = (uint8_t*)malloc((size_t)nb * d * 32);
  uint8_t* tscales = (uint8_t*)malloc((size_t)nb * d);
  for (int rule = 0; rule <= 3; ++rule)
    expect(oracle_quantize_token_blocks(x, ORACLE_BF16, B, H, N, d, strides, rule, 7.0, NULL, nb, tcodes, tscales, 3),
           0, "quantize_token_blocks");
  const int64_t blocks[2] = {1, nb - 1};
  expect(oracle_quantize_token_blocks(x, ORACLE_BF16, B, H, N, d, strides, ORACLE_RULE_OCP, 0.0, blocks, 2, tcodes,
                                      tscales, 1),
         0, "quantize_token_blocks subset");

  const double qs[3] = {6.0, 7.25, 8.0};
  double sse[2 * 3];
  for (int axis = 0; axis <= 1; ++axis)
    expect(oracle_scale_sweep(x, ORACLE_BF16, B, H, N, d, strides, axis, axis == 0, qs, 3, NULL, B * H, sse, 2), 0,
           "scale_sweep");
  free(x);
  free(codes);
  free(scales);
  free(tcodes);
  free(tscales);
}

static void run_attention(int N, int Nk, int d, int causal, int quant, int rule, int p_mode, int kv_tile,
                          const int32_t* rows, int n_rows) {
  const int B = 2, H = 1;
  const int nq = n_rows > 0 ? n_rows : N;
  uint16_t* q = make_input((size_t)B * H * N * d, 1.0);
  uint16_t* k = make_input((size_t)B * H * Nk * d, 1.0);
  uint16_t* v = make_input((size_t)B * H * Nk * d, 3.0);
  const size_t no = (size_t)B * H * nq;
  double* out = (double*)malloc(no * d * sizeof(double));
  double* m = (double*)malloc(no * sizeof(double));
  double* l = (double*)malloc(no * sizeof(double));
  double* rs = (double*)malloc(no * sizeof(double));
  double* amb = (double*)malloc(no * d * sizeof(double));
  double* am = (double*)malloc(no * d * sizeof(double));
  oracle_attn_cfg cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.B = B; cfg.H = H; cfg.N = N; cfg.d = d;
  cfg.dtype = ORACLE_BF16;
  cfg.causal = causal;
  cfg.rotate = 1;
  cfg.quant = quant;
  cfg.rule = rule;
  cfg.p_mode = p_mode;
  cfg.kv_tile = kv_tile;
  cfg.nthreads = 3;
  cfg.q = 7.25;
  cfg.amb_delta = 0x1p-13;
  cfg.Nk = Nk == N ? 0 : Nk;
  double* ars = (double*)malloc(no * sizeof(double));
  expect(oracle_attention(&cfg, q, k, v, NULL, n_rows > 0 ? rows : NULL, n_rows > 0 ? n_rows : N, out, m, l, rs, amb,
                          am, ars),
         0, "attention");
  free(ars);
  /* nullable outputs left out */
  expect(oracle_attention(&cfg, q, k, v, NULL, n_rows > 0 ? rows : NULL, n_rows > 0 ? n_rows : N, out, NULL, NULL,
                          NULL, NULL, NULL, NULL),
         0, "attention, outputs only");
  if (Nk == N && quant && (rule == ORACLE_RULE_UOS || rule == ORACLE_RULE_OCP)) {
    double* diag = (double*)malloc(no * 6 * sizeof(double));
    double* damb = (double*)malloc(no * sizeof(double));
    expect(oracle_p_diagnostics(&cfg, q, k, NULL, n_rows > 0 ? rows : NULL, n_rows > 0 ? n_rows : N, 1.25, diag,
                                damb),
           0, "p_diagnostics");
    free(diag);
    free(damb);
  }
  free(q); free(k); free(v);
  free(out); free(m); free(l); free(rs); free(amb); free(am);
}

static void check_attention(void) {
  const int32_t rows[5] = {0, 1, 17, 33, 44};
  for (int p_mode = 0; p_mode <= 3; ++p_mode)
    for (int rule = 0; rule <= 1; ++rule) {
      run_attention(45, 45, 64, 1, 1, rule, p_mode, 32, NULL, 0);
      run_attention(45, 45, 128, 0, 1, rule, p_mode, 64, rows, 5);
    }
  run_attention(45, 45, 64, 1, 0, ORACLE_RULE_UOS, ORACLE_P_EXACT, 32, NULL, 0);
  run_attention(20, 70, 128, 0, 1, ORACLE_RULE_UOS, ORACLE_P_PNQ, 64, NULL, 0); /* cross-attention */
  run_attention(70, 3, 64, 0, 1, ORACLE_RULE_OCP, ORACLE_P_DIRECT, 32, rows, 5);
  run_attention(1, 1, 64, 1, 1, ORACLE_RULE_UOS, ORACLE_P_PNQ, 128, NULL, 0);

  /* arguments the oracle must reject */
  oracle_attn_cfg cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.B = 1; cfg.H = 1; cfg.N = 8; cfg.d = 64; cfg.quant = 1; cfg.kv_tile = 40; cfg.nthreads = 1;
  uint16_t dummy[8 * 64] = {0};
  double out[8 * 64];
  expect(oracle_attention(&cfg, dummy, dummy, dummy, NULL, NULL, 8, out, NULL, NULL, NULL, NULL, NULL, NULL), -1,
         "attention kv_tile=40");
  cfg.kv_tile = 32;
  cfg.d = 80;
  expect(oracle_attention(&cfg, dummy, dummy, dummy, NULL, NULL, 8, out, NULL, NULL, NULL, NULL, NULL, NULL), -1,
         "attention d=80");
}

static void check_scalars(void) {
  volatile double sink = 0.0;
  for (int c = 0; c < 16; ++c) sink += oracle_e2m1_value(c) + oracle_e2m1_magnitude(c & 7);
  for (int i = -2000; i <= 2000; ++i) sink += oracle_e2m1_project(i / 250.0);
  const double Ms[] = {0.0, 0x1p-149, 0x1p-126, 1.0, 7.25, 14.5, 3.0e38, 1e300};
  for (unsigned i = 0; i < sizeof Ms / sizeof Ms[0]; ++i)
    for (int rule = 0; rule <= 3; ++rule) sink += oracle_scale_exponent(Ms[i], rule, 6.75);
  int32_t e[8];
  oracle_scale_exponents(Ms, 8, ORACLE_RULE_UOS, 0.0, e);
  for (uint32_t b = 0; b < 65536; ++b) {
    const float a = oracle_decode_half((uint16_t)b, ORACLE_BF16), h = oracle_decode_half((uint16_t)b, ORACLE_FP16);
    if (isfinite(a)) sink += a * 0.0;
    if (isfinite(h)) sink += h * 0.0;
  }
  float r[128];
  for (int i = 0; i < 128; ++i) r[i] = (float)(next_unit() - 0.5);
  oracle_hadamard_rotate_f32(r, 64);
  oracle_hadamard_rotate_f32(r, 128);
  /* the block allowance over both rules, zero / tiny / boundary blocks and
   * both exact references */
  double p[32], ph[32], dp[32];
  for (int rule = 0; rule < 4; ++rule)
    for (int kind = 0; kind < 4; ++kind) {
      for (int i = 0; i < 32; ++i) p[i] = kind == 0 ? 0.0 : (kind == 1 ? 0x1p-140 * next_unit() : next_unit());
      if (kind == 3) p[7] = 1.0;
      sink += oracle_p_block_allowance(p, rule, 6.5, 1e-3, kind == 3 ? 1.0 : 0.0, ph, dp) * 0.0;
      sink += oracle_p_block_allowance(p, rule, 6.5, 0.0, 0.0, ph, NULL) * 0.0;
      for (int i = 0; i < 32; ++i) sink += ph[i] * 0.0 + dp[i] * 0.0;
    }
  (void)sink;
}

int main(void) {
  check_scalars();
  check_quantizers();
  check_attention();
  if (failures) {
    fprintf(stderr, "%d unexpected return codes\n", failures);
    return 1;
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}
