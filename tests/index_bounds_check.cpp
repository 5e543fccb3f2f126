// index_bounds_check.cpp -- test infrastructure for the quantizer kernels'
// input addressing.
//
// Host-only: compiled with g++ against csrc/quant_index.h, the header whose
// functions the kernels call for every input load (under g++ __host__ and
// __device__ expand to nothing).  For a list of shapes and strides it walks
// every lane of the launch grids the launchers use (256 threads per
// workgroup; the head-dimension quantizer has one 32-channel block per
// thread, the token quantizer d/2 threads per 32-token block) and checks that
// each load lies inside the input tensor and reads a real token (n < N).
// The token quantizer's fast path is taken per wave, when every active lane's
// block lies inside [0, N); the walk follows that choice per wave.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "internal.h"
#include "quant_index.h"

using namespace mxattn_internal;

struct Case {
  int B, H, N, d;
  int layout;  // 0 contiguous [B,H,N,d]; 1 physical [B,N,H,d]; 2 every other token of [B,H,2N,d]
};

static int failures = 0;

static void fail(const Case& c, const char* what, int64_t off, int64_t extent) {
  if (failures < 20)
    fprintf(stderr, "B%d H%d N%d d%d layout %d: %s at element %lld (extent %lld)\n", c.B, c.H, c.N, c.d, c.layout,
            what, (long long)off, (long long)extent);
  ++failures;
}

static void check(const Case& c) {
  int64_t sB, sH, sN;
  if (c.layout == 1) {
    sN = (int64_t)c.H * c.d;
    sH = c.d;
    sB = (int64_t)c.N * c.H * c.d;
  } else if (c.layout == 2) {
    sN = 2 * (int64_t)c.d;
    sH = 2 * (int64_t)c.N * c.d;
    sB = (int64_t)c.H * sH;
  } else {
    sN = c.d;
    sH = (int64_t)c.N * c.d;
    sB = (int64_t)c.H * sH;
  }
  // one past the last element the tensor owns
  const int64_t extent = (int64_t)(c.B - 1) * sB + (int64_t)(c.H - 1) * sH + (int64_t)(c.N - 1) * sN + c.d;
  const int Np = (int)padded_tokens(c.N);

  // head-dimension quantizer: unit u = group * 256 + thread
  {
    const int bpr = c.d / 32;
    const int64_t total = (int64_t)c.B * c.H * Np * bpr;
    const int64_t groups = (total + 255) / 256;
    for (int64_t u = 0; u < groups * 256; ++u) {
      const HeaddimUnit w = headdim_unit(u, Np, bpr);
      const int64_t off = headdim_load_offset(w, total, u, c.H, c.N, sB, sH, sN);
      if (off < 0) continue;
      if (w.n >= c.N) fail(c, "head-dim load of a padding row", off, extent);
      if (off < 0 || off + 32 > extent) fail(c, "head-dim load outside the tensor", off, extent);
    }
  }
  // token quantizer: lane gl = group * 256 + thread; d/2 lanes per block
  {
    const int lpb = c.d / 2;
    const int nbp = Np / 32;
    const int64_t total = (int64_t)c.B * c.H * nbp;
    const int64_t groups = (total * lpb + 255) / 256;
    for (int64_t w0 = 0; w0 < groups * 256; w0 += 64) {  // one wave at a time
      bool all_inside = true;
      for (int64_t gl = w0; gl < w0 + 64; ++gl) {
        const int64_t gblk = gl / lpb;
        if (gblk >= total) continue;  // the lane has returned
        if (!tokens_block_inside((int)(gblk % nbp), c.N)) all_inside = false;
      }
      for (int64_t gl = w0; gl < w0 + 64; ++gl) {
        const int64_t gblk = gl / lpb;
        if (gblk >= total) continue;
        const int cp = (int)(gl % lpb);
        const int64_t bh = gblk / nbp;
        const int kb = (int)(gblk % nbp);
        const int64_t base = tokens_lane_base(bh, cp, c.H, sB, sH);
        for (int k = 0; k < 32; ++k) {
          const int tok = all_inside ? 32 * kb + k : tokens_guarded_token(kb, k, c.N);
          const int64_t off = base + (int64_t)tok * sN;
          if (tok < 0 || tok >= c.N) fail(c, "token load past N", off, extent);
          if (off < 0 || off + 2 > extent) fail(c, "token load outside the tensor", off, extent);
        }
      }
    }
  }
}

int main() {
  const Case cases[] = {
      {2, 3, 150, 128, 1},    // strided [B,N,H,d] view; Np - N = 106: three blocks wholly in the padding
      {2, 3, 150, 128, 0},    {2, 3, 150, 128, 2}, {1, 1, 1, 64, 0},   {1, 1, 1, 128, 1},
      {2, 2, 31, 64, 0},      {2, 2, 31, 64, 1},   {1, 3, 129, 128, 0}, {2, 2, 300, 64, 2},
      {3, 2, 97, 64, 1},      {1, 2, 4100, 128, 0},
      {1, 2, 118800, 128, 0},  // the Hunyuan-like token count on two heads: Np - N = 112
      {1, 40, 32760, 128, 0},  // the Wan-like shape
      {1, 40, 32760, 128, 1},
  };
  for (const Case& c : cases) check(c);
  if (failures) {
    fprintf(stderr, "%d out-of-range loads\n", failures);
    return 1;
  }
  printf("all quantizer loads inside their tensors (%zu shapes)\n", sizeof cases / sizeof cases[0]);
  return 0;
}
