// Internal interface between the C-ABI layer (api.cpp) and the kernel
// launchers (quantize.hip, attention.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxattn_internal {

constexpr int kTokenAlign = 128;  // Np = N rounded up to this
constexpr int kKvTile = 128;      // B_c of the forward

inline int64_t padded_tokens(int N) { return ((int64_t)N + kTokenAlign - 1) / kTokenAlign * kTokenAlign; }

struct QuantArgs {
  const void* x;
  int dtype;  // 0 bf16, 1 fp16
  int B, H, N, d;
  int64_t sB, sH, sN;  // element strides
  int rotate;
  int rule;  // 0 UOS, 1 OCP
  uint8_t* codes;
  uint8_t* scales;
};

hipError_t launch_quantize_headdim(const QuantArgs& a, hipStream_t stream);
hipError_t launch_quantize_tokens(const QuantArgs& a, hipStream_t stream);

enum AttnMode : int {
  kModePnq = 0,
  kModeDirect = 1,
  kModePostnorm = 2,
};

struct AttnArgs {
  const uint8_t* qc;
  const uint8_t* qs;
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int B, H, N, d;  // N: query rows
  int Nk;           // key / value tokens (cross-attention); N for self-attention
  int causal;
  int mode;  // AttnMode
  int rule;  // scale rule of the softmax-path quantizer
  float* out;        // [B, H, N, d]
  float* row_stats;  // nullable [B, H, N, 2] (m, l)
  float* row_sums;   // nullable [B, H, N]
  float* stats_ws;   // POSTNORM: [B, H, Np, 2] exact (m, l) of pass 1
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

}  // namespace mxattn_internal
