// Input addressing of the two quantizer kernels, in one place so that a
// host-only bounds check (compiled with g++, where __host__ and __device__
// expand to nothing) exercises the very functions the kernels call.
//
// A 16-bit input tensor [B, H, N, d] is addressed with element strides
// (sB, sH, sN) and a unit stride along d.  Its last element sits at
// (B-1) sB + (H-1) sH + (N-1) sN + d - 1; no load may go past it, and no load
// may read a token n >= N (those belong to the caller, not to this tensor).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxattn_internal {

// Head-dimension quantizer (Q, K): work unit u = one 32-channel block of one
// row of the padded token range [0, Np).  Rows n >= N are padding and load
// nothing.  Returns the element offset of the block's first element, or -1
// for a unit that loads nothing.
struct HeaddimUnit {
  int64_t bh;
  int n, blk;
};

__host__ __device__ __forceinline__ HeaddimUnit headdim_unit(int64_t u, int Np, int blocks_per_row) {
  HeaddimUnit r;
  const int64_t row = u / blocks_per_row;
  r.blk = (int)(u % blocks_per_row);
  r.bh = row / Np;
  r.n = (int)(row % Np);
  return r;
}

__host__ __device__ __forceinline__ int64_t headdim_load_offset(const HeaddimUnit& w, int64_t total_units,
                                                                int64_t u, int H, int N, int64_t sB, int64_t sH,
                                                                int64_t sN) {
  if (u >= total_units || w.n >= N) return -1;
  const int64_t b = w.bh / H, h = w.bh % H;
  return b * sB + h * sH + (int64_t)w.n * sN + 32 * w.blk;
}

// Token-axis quantizer (V): work unit = one 32-token block kb of one head,
// split over d/2 lanes, lane cp owning channels 2cp and 2cp + 1.  Blocks run
// over the padded token range [0, Np), so a block may lie partly or wholly
// past N.  A lane whose block lies wholly inside [0, N) reads tokens
// 32 kb .. 32 kb + 31 in order; any other lane reads, for its k-th token, the
// token clamped into [0, N) and discards the value when 32 kb + k >= N.
__host__ __device__ __forceinline__ int64_t tokens_lane_base(int64_t bh, int cp, int H, int64_t sB, int64_t sH) {
  const int64_t b = bh / H, h = bh % H;
  return b * sB + h * sH + 2 * cp;
}

__host__ __device__ __forceinline__ bool tokens_block_inside(int kb, int N) { return 32 * kb + 31 < N; }

// token read for the k-th element of block kb on the guarded path: always a
// real token (N >= 1), whatever kb is
__host__ __device__ __forceinline__ int tokens_guarded_token(int kb, int k, int N) {
  const int t = 32 * kb + k;
  return t < N ? t : N - 1;
}

}  // namespace mxattn_internal
