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
  int rule;        // 0 UOS, 1 OCP, 2 ceiling rule with boundary qbits
  uint32_t qbits;  // rule 2: binary32 bits of the boundary q rounded down
  uint8_t* codes;
  uint8_t* scales;
};

hipError_t launch_quantize_headdim(const QuantArgs& a, hipStream_t stream);
hipError_t launch_quantize_tokens(const QuantArgs& a, hipStream_t stream);
// Q and K along d (rotated if q.rotate), V along tokens, in one launch; the
// three share dtype, d and rule (UOS or OCP)
hipError_t launch_quantize_qkv(const QuantArgs& q, const QuantArgs& k, const QuantArgs& v, hipStream_t stream);

constexpr int kSweepMax = 48;  // boundaries per sweep call

struct SweepArgs {
  const void* x;
  int dtype;
  int B, H, N, d;
  int64_t sB, sH, sN;
  int axis;    // 0 head dimension, 1 tokens
  int rotate;  // head dimension only
  int nq;
  uint32_t qbits[kSweepMax];  // binary32 bits of each boundary rounded down
  uint32_t qmin_bits;         // the smallest boundary (largest exponent)
  int chunks;                 // workgroups per head, sweep_chunks()
  double* partial;            // workspace [B*H][chunks][nq]
  double* sse;                // [B*H][nq]
};

int sweep_chunks(int axis, int N, int d);
hipError_t launch_scale_sweep(const SweepArgs& a, hipStream_t stream);
// The same with a.partial ignored: the partial sums go to the library's
// static per-GPU scratch array (the caller has checked the size against
// MXATTN_SWEEP_SCRATCH_BYTES).
hipError_t launch_scale_sweep_static(const SweepArgs& a, hipStream_t stream);

enum AttnMode : int {
  kModePnq = 0,
  kModeDirect = 1,
  kModePostnorm = 2,
  kModeDiag = 4,  // row-sum diagnostics of materialized P (no PV product)
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
  float* stats_ws;   // POSTNORM, DIAG: [B, H, Np, 4] exact (m, l, l - 1, unused) of pass 1
  float* diag;       // DIAG: [B, H, N, 6]
  float gamma;       // DIAG: pre-quantization global scale of P
  // fused Q prologue (PNQ with the UOS softmax rule only): when qx is set,
  // qc / qs are unused and Q is rotated (qrotate) and quantized with qrule
  // inside the forward
  const void* qx = nullptr;
  int qdtype = 0;
  // the caller allows the resident-key kernel (non-causal PNQ forward whose
  // key/value tiles all fit in LDS); the results are the same bit for bit
  int resident_ok = 0;
  int64_t qsB = 0, qsH = 0, qsN = 0;
  int qrotate = 0, qrule = 0;
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

}  // namespace mxattn_internal
