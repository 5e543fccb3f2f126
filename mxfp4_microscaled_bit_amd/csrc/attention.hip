// Fused MXFP4 attention forward of MXAttention for gfx950 (MI355X).
//
// One workgroup = 4 waves = 128 queries of one (batch, head); each wave owns
// 32 queries as two 16-query sub-blocks.  Key/value tiles of B_c = 128 keys
// are staged through LDS (double buffered) and visited in ascending order
// (MXAttention paper, Alg. 2 steps 10-19):
//
//   S^T  = K^ Q^T         scaled-FP4 MFMA 16x16x128, one per 16 keys x 16
//                         queries (block scales along d ride in the MFMA)
//   m    = max(m, rowmax) running max per query                  (Eq. 3)
//   P~   = exp(S - m)     exponentials                           (Eq. 5)
//   P^   = Q*(P~)         UOS quantization per 32-key block      (Eq. 44)
//   l    = a l + P^ 1     the same P^ ...                        (Eq. 47)
//   O~   = a O~ + P^ V^   ... feeds both updates (PNQ)           (Eq. 48)
//   O    = O~ / l                                                (Eq. 8)
//
// Register layouts follow the gfx950 scaled MFMA: in a 16x16x128 product,
// lane L supplies row/column L%16 and the 32-element K-chunk L/16, and holds
// D[4*(L/16)+i][L%16].  The A operand of S^T takes the keys in the permuted
// order row r <- key 32*(r/4) + 4t + r%4 (t = 16-key sub-tile), so after the
// eight S products lane L holds, for query L%16, the 32 consecutive keys
// 32*(L/16) .. +31 -- exactly one 32-key quantization block, and exactly the
// B-operand chunk of the PV product.  P^ therefore never moves between lanes;
// its block maximum is lane-local.  l comes from one more MFMA against a tile
// of ones, so l and O~ are updated from the same quantized tile by the same
// instruction stream (the PNQ identity).
//
// Scores stay in raw units (q^.k^); exp(s - m) is evaluated as
// exp2(fma(s, c, -m c)) with c = log2(e)/sqrt(d), and the block scale 2^e is
// folded into the exponent argument so P~/2^e goes straight to the FP4
// convert (round to nearest even, saturating at 6).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace mxattn_internal {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBr = 128;       // queries per workgroup
constexpr int kBc = kKvTile;   // keys per tile
constexpr int kRuleUos = 0;
constexpr int kRuleOcp = 1;
constexpr int kModeStats = 3;  // first pass of POSTNORM: exact (m, l) only

struct Params {
  const uint8_t* qc;
  const uint8_t* qs;
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  float* out;
  float* row_stats;
  float* row_sums;
  float* stats;
  int H, N, Np, nqt;
};

// byte offsets inside one LDS stage
template <int D>
struct Lds {
  static constexpr int KC = 0;                  // K^ codes, swizzled 16-byte granules
  static constexpr int KS = KC + kBc * D / 2;   // K^ scales as [chunk][r][t]
  static constexpr int VC = KS + kBc * D / 32;  // V^ codes [block][channel][16]
  static constexpr int VS = VC + 64 * D;        // V^ scales as [block][r][ct]
  static constexpr int STAGE = VS + 4 * D;
};

// 16-byte granule of (key k, d-chunk c) in the K^ stage.  The MFMA operand
// read has 16 lanes of one chunk fetch keys 32g + 4t + i (g, i = 0..3); the
// XOR spreads them over distinct bank groups for both 8- and 16-lane phases.
template <int D>
__device__ __forceinline__ int kc_granule(int k, int c) {
  if constexpr (D == 128) return 4 * k + (c ^ ((k >> 5) & 3) ^ (k & 2));
  else return (2 * k + c) ^ ((k >> 5) & 1) ^ (((k >> 6) & 1) << 3);
}

// (key, d-chunk) held by LDS granule G of the K^ stage (the inverse of kc_granule)
template <int D>
__device__ __forceinline__ int kc_source_chunk(int G) {
  if constexpr (D == 128) {
    const int k = G >> 2;
    return 4 * k + ((G & 3) ^ ((k >> 5) & 3) ^ (k & 2));
  } else {
    const int g0 = (G >> 6) & 1, g1 = (G >> 7) & 1;
    return G ^ g0 ^ (g1 << 3);  // = 2k + c
  }
}

// Stage one key/value tile into LDS.  The code bytes (16 KB at d = 128) go
// straight from global memory into LDS with global_load_lds_dwordx4: lane i
// of a wave writes LDS granule base + i, so each lane fetches the global
// 16-byte chunk that belongs in that (swizzled) granule.  The scale bytes are
// few; they pass through registers and are scattered into their operand
// order with byte stores (scale_store).
// LDS-destination copy of one 16-byte chunk per lane (device code only: the
// builtin takes an LDS address-space pointer, which the host pass cannot form)
__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                            reinterpret_cast<uintptr_t>(lds_base)),
                                   16, 0, 0);
#endif
}

template <int D>
__device__ __forceinline__ void codes_dma(const Params& p, int64_t bh, int kt, uint8_t* stage, int tid) {
  using L = Lds<D>;
  constexpr int KG = kBc * D / 2 / 16;  // K^ granules per tile
  constexpr int VG = 64 * D / 16;       // V^ granules per tile
  const int NBp = p.Np / 32;
  const int wave = tid >> 6, lane = tid & 63;
  const uint8_t* kb = p.kc + (bh * p.Np + (int64_t)kt * kBc) * (D / 2);
  const uint8_t* vb = p.vc + (bh * NBp + (int64_t)kt * 4) * D * 16;
#pragma unroll
  for (int u = 0; u < KG / 256; ++u) {
    const int G0 = u * 256 + wave * 64;
    dma16(kb + 16 * kc_source_chunk<D>(G0 + lane), stage + L::KC + 16 * G0);
  }
#pragma unroll
  for (int u = 0; u < VG / 256; ++u) {
    const int G0 = u * 256 + wave * 64;
    dma16(vb + 16 * (G0 + lane), stage + L::VC + 16 * G0);
  }
}

struct ScaleRegs {
  uint32_t ks;
  uint32_t vs;
};

template <int D>
__device__ __forceinline__ ScaleRegs scale_load(const Params& p, int64_t bh, int kt, int tid) {
  const int NBp = p.Np / 32;
  ScaleRegs r = {0u, 0u};
  if (tid < kBc) {
    const uint8_t* ksrc = p.ks + (bh * p.Np + (int64_t)kt * kBc + tid) * (D / 32);
    if constexpr (D == 128) r.ks = *reinterpret_cast<const uint32_t*>(ksrc);
    else r.ks = *reinterpret_cast<const uint16_t*>(ksrc);
  }
  if (tid < D) r.vs = *reinterpret_cast<const uint32_t*>(p.vs + (bh * NBp + (int64_t)kt * 4) * D + 4 * tid);
  return r;
}

template <int D>
__device__ __forceinline__ void scale_store(const ScaleRegs& r, uint8_t* stage, int tid) {
  using L = Lds<D>;
  if (tid < kBc) {
    const int k = tid, g = k >> 5, t = (k >> 2) & 7, i = k & 3, rr = 4 * g + i;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) stage[L::KS + (c * 16 + rr) * 8 + t] = (uint8_t)(r.ks >> (8 * c));
  }
  if (tid < D) {
    const int g = (4 * tid) / D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = (4 * tid) % D + j, ct = ch / 16, rr = ch % 16;
      stage[L::VS + (g * 16 + rr) * (D / 16) + ct] = (uint8_t)(r.vs >> (8 * j));
    }
  }
}

__device__ __forceinline__ v8i as_op(uint4 a) {
  v8i r = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  return r;
}

template <int OPSEL_A>
__device__ __forceinline__ v4f mfma4(uint4 a, uint4 b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_op(a), as_op(b), c, 4, 4, OPSEL_A, sa, 0, sb);
}

// Shared-scale exponent of a block with max M >= 0 from the binary32 fields
// of M (see the quantizer kernels for the derivation).
template <int RULE>
__device__ __forceinline__ int scale_exponent(float M) {
  const uint32_t b = __float_as_uint(M);
  if (b == 0u) return 0;
  const int E = (int)(b >> 23);
  if (E == 0) return -127;
  int e = E - 129;
  if constexpr (RULE == kRuleUos) e += ((b & 0x7FFFFFu) > 0x680000u) ? 1 : 0;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ float xor_lanes(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ uint32_t pack_fp4x8(const float* y) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// Per-query state of one 16-query sub-block, replicated in the four lanes that
// share a query.
struct RowState {
  float m;    // running max of raw scores (or m* for POSTNORM)
  float mc;   // m * c + off
  float off;  // POSTNORM: log2 l* (P = exp(s - m*) / l*); otherwise 0
  float l;    // DIRECT / STATS: running sum of unquantized exponentials
};

template <int D, int MODE, int RULE>
struct FwdConsts {
  static constexpr int NCT = D / 16;  // 16-channel output tiles
  // Exponent arguments.  The fused path evaluates (s - m) c as one
  // fma(s, c, -m c); the row maximum then gives P~ = 1 within an ulp, which
  // the UOS rule maps to the interior value 4.  The OCP rule puts P~ = 1 on
  // its scale boundary (floor(log2 1) - 2), and the reference modes must
  // reproduce exact ties, so they evaluate fma(s - m, c, -off), which is
  // exact when s = m.
  static constexpr bool kExactArg = !(MODE == kModePnq && RULE == kRuleUos);
  static constexpr float kC = (D == 128) ? 0x1.0527dcp-3f : 0x1.715476p-3f;  // log2(e)/sqrt(d)
  static constexpr float kInvSqrtD = (D == 128) ? 0x1.6a09e6p-4f : 0x1p-3f;  // 1/sqrt(d)
};

// Online-softmax update and P^ of one 16-query sub-block for one key tile:
// s holds the lane's 32 scores (one 32-key block of query L%16).  Returns the
// packed FP4 B operand of the PV product; writes its E8M0 scale and alpha.
template <int D, int MODE, int RULE>
__device__ __forceinline__ uint4 softmax_block(v4f (&s)[8], RowState& rs, int& psc, float& alpha) {
  using F = FwdConsts<D, MODE, RULE>;
  float bmax = s[0][0];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[t][i]);
  float a = 1.0f;
  if constexpr (MODE != kModePostnorm) {
    float rmax = fmaxf(bmax, xor_lanes(bmax, 16));
    rmax = fmaxf(rmax, xor_lanes(rmax, 32));
    const float m_new = fmaxf(rs.m, rmax);
    if (m_new != -INFINITY) {
      a = __builtin_amdgcn_exp2f((rs.m - m_new) * F::kC);  // 0 on the first visited tile
      rs.m = m_new;
      rs.mc = m_new * F::kC;
    }
  }
  alpha = a;
  const float mc = rs.mc, mref = rs.m, off = rs.off;
  if constexpr (MODE == kModeStats) {
    float sum = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f((s[t][i] - mref) * F::kC);
    sum += xor_lanes(sum, 16);
    sum += xor_lanes(sum, 32);
    rs.l = a * rs.l + sum;
    psc = 127;
    return make_uint4(0, 0, 0, 0);
  } else {
    // block scale from the block max of the exponentials (exp is monotone)
    const float Mb = F::kExactArg ? __builtin_amdgcn_exp2f(fmaf(bmax - mref, F::kC, -off))
                                  : __builtin_amdgcn_exp2f(fmaf(bmax, F::kC, -mc));
    const int e = scale_exponent<RULE>(Mb);
    float y[32];
    if constexpr (F::kExactArg) {
      const float nb = -(off + (float)e);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[4 * t + i] = __builtin_amdgcn_exp2f(fmaf(s[t][i] - mref, F::kC, nb));
    } else {
      const float nb = -(mc + (float)e);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[4 * t + i] = __builtin_amdgcn_exp2f(fmaf(s[t][i], F::kC, nb));
    }
    if constexpr (MODE == kModeDirect) {
      float sum = 0.0f;
#pragma unroll
      for (int k = 0; k < 32; ++k) sum += y[k];
      sum = __builtin_amdgcn_ldexpf(sum, e);
      sum += xor_lanes(sum, 16);
      sum += xor_lanes(sum, 32);
      rs.l = a * rs.l + sum;
    }
    psc = e + 127;
    return make_uint4(pack_fp4x8(y), pack_fp4x8(y + 8), pack_fp4x8(y + 16), pack_fp4x8(y + 24));
  }
}

template <int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void mask_scores(v4f (&s)[8], int kt, int N, int q, int grp) {
  if constexpr (MASKED) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt * kBc + 32 * grp + 4 * t + i;
        if (!(key < N && (!CAUSAL || key <= q))) s[t][i] = -INFINITY;
      }
  }
}

// O~ (and the l column) of one sub-block: rescale by alpha when a running
// max moved, then accumulate P^ V^ and P^ 1 with the matrix cores.
template <int D, int MODE>
__device__ __forceinline__ void pv_block(const uint4 (&vop)[D / 16], uint2 vsw, uint4 pq, int psc, float alpha,
                                         v4f (&acc)[D / 16 + 1]) {
  constexpr int NCT = D / 16;
  if constexpr (MODE != kModePostnorm) {
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int ct = 0; ct <= NCT; ++ct) acc[ct] *= alpha;
    }
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int sc = (ct < 4) ? (int)vsw.x : (int)vsw.y;
    switch (ct & 3) {
      case 0: acc[ct] = mfma4<0>(vop[ct], pq, acc[ct], sc, psc); break;
      case 1: acc[ct] = mfma4<1>(vop[ct], pq, acc[ct], sc, psc); break;
      case 2: acc[ct] = mfma4<2>(vop[ct], pq, acc[ct], sc, psc); break;
      default: acc[ct] = mfma4<3>(vop[ct], pq, acc[ct], sc, psc); break;
    }
  }
  const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);  // E2M1 1.0
  acc[NCT] = mfma4<0>(ones, pq, acc[NCT], 127, psc);
}

// One key tile for the wave's 32 queries, ordered so the matrix cores and the
// vector ALU overlap inside the wave: both sub-blocks' S products are issued
// first; the softmax of sub-block 0 runs while those of sub-block 1 are in
// flight; its PV products are issued before the softmax of sub-block 1, which
// then runs while they execute.  MASKED tiles (the ragged last tile and the
// causal diagonal) set scores of invisible keys to -inf; every other tile runs
// without any per-element test.
template <int D, bool CAUSAL, int MODE, int RULE, bool MASKED>
__device__ __forceinline__ void tile_step(const uint8_t* __restrict__ buf, int kt, int N, const uint4 (&qop)[2],
                                          const int (&qsc)[2], const int (&qi)[2], RowState (&rs)[2],
                                          v4f (&acc)[2][D / 16 + 1], int r16, int grp) {
  using L = Lds<D>;
  constexpr int NCT = D / 16;
  // ---- S^T = K^ Q^T for 128 keys x 32 queries
  uint2 ksw = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  if (grp < D / 32) ksw = *reinterpret_cast<const uint2*>(buf + L::KS + (grp * 16 + r16) * 8);
  uint4 kop[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int k = 32 * (r16 >> 2) + 4 * t + (r16 & 3);
    kop[t] = *reinterpret_cast<const uint4*>(buf + L::KC + 16 * kc_granule<D>(k, grp & (D / 32 - 1)));
    if (D == 64 && grp >= 2) kop[t] = make_uint4(0, 0, 0, 0);
  }
  v4f s0[8], s1[8];
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    v4f (&s)[8] = sb ? s1 : s0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int sc = (t < 4) ? (int)ksw.x : (int)ksw.y;
      switch (t & 3) {
        case 0: s[t] = mfma4<0>(kop[t], qop[sb], z, sc, qsc[sb]); break;
        case 1: s[t] = mfma4<1>(kop[t], qop[sb], z, sc, qsc[sb]); break;
        case 2: s[t] = mfma4<2>(kop[t], qop[sb], z, sc, qsc[sb]); break;
        default: s[t] = mfma4<3>(kop[t], qop[sb], z, sc, qsc[sb]); break;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- sub-block 0: softmax and P^, while the S products of sub-block 1 run
  mask_scores<D, CAUSAL, MASKED>(s0, kt, N, qi[0], grp);
  int psc0;
  float a0;
  const uint4 pq0 = softmax_block<D, MODE, RULE>(s0, rs[0], psc0, a0);
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (MODE != kModeStats) {
    uint2 vsw = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    if constexpr (D == 128) vsw = *reinterpret_cast<const uint2*>(buf + L::VS + (grp * 16 + r16) * 8);
    else vsw.x = *reinterpret_cast<const uint32_t*>(buf + L::VS + (grp * 16 + r16) * 4);
    uint4 vop[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      vop[ct] = *reinterpret_cast<const uint4*>(buf + L::VC + 16 * (grp * D + 16 * ct + r16));
    pv_block<D, MODE>(vop, vsw, pq0, psc0, a0, acc[0]);
    __builtin_amdgcn_sched_barrier(0);

    // ---- sub-block 1, while the PV products of sub-block 0 run
    mask_scores<D, CAUSAL, MASKED>(s1, kt, N, qi[1], grp);
    int psc1;
    float a1;
    const uint4 pq1 = softmax_block<D, MODE, RULE>(s1, rs[1], psc1, a1);
    __builtin_amdgcn_sched_barrier(0);
    pv_block<D, MODE>(vop, vsw, pq1, psc1, a1, acc[1]);
  } else {
    mask_scores<D, CAUSAL, MASKED>(s1, kt, N, qi[1], grp);
    int psc1;
    float a1;
    (void)softmax_block<D, MODE, RULE>(s1, rs[1], psc1, a1);
  }
}

template <int D, bool CAUSAL, int MODE, int RULE>
__global__ __launch_bounds__(256, 2) void k_attention(Params p) {
  using L = Lds<D>;
  using F = FwdConsts<D, MODE, RULE>;
  constexpr int NCT = F::NCT;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;

  // workgroup -> (head, query tile); consecutive logical tiles land on the
  // same XCD (the hardware deals workgroups round-robin over 8 XCDs) so the
  // query tiles of one head share that XCD's L2 copy of its K^ and V^
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3, qx = G >> 3, rx = G & 7;
  const int logical = (xcd < rx) ? xcd * (qx + 1) + idx : rx * (qx + 1) + (xcd - rx) * qx + idx;
  const int64_t bh = logical / p.nqt;
  int qt = logical % p.nqt;
  if (CAUSAL) qt = p.nqt - 1 - qt;  // longest causal rows first
  const int nkt_all = (p.N + kBc - 1) / kBc;
  const int nkt = CAUSAL ? min(qt + 1, nkt_all) : nkt_all;
  // leading tiles in which every key is visible to every query of the tile
  const int nfull = CAUSAL ? min(qt, nkt) : p.N / kBc;

  // Q^ operands of the two sub-blocks (B operand: lane = query L%16, d-chunk L/16)
  uint4 qop[2];
  int qsc[2], qi[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    qi[sb] = qt * kBr + 32 * wave + 16 * sb + r16;
    const int64_t row = bh * p.Np + qi[sb];
    if (grp < D / 32) {
      qop[sb] = *reinterpret_cast<const uint4*>(p.qc + row * (D / 2) + 16 * grp);
      qsc[sb] = p.qs[row * (D / 32) + grp];
    } else {
      qop[sb] = make_uint4(0, 0, 0, 0);
      qsc[sb] = 127;
    }
  }

  RowState rs[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    rs[sb].m = -INFINITY;
    rs[sb].mc = 0.0f;
    rs[sb].off = 0.0f;
    rs[sb].l = 0.0f;
    if constexpr (MODE == kModePostnorm) {
      const float* st = p.stats + (bh * p.Np + qi[sb]) * 2;
      rs[sb].m = st[0];
      rs[sb].off = __builtin_amdgcn_logf(st[1]);  // log2 of l*
      rs[sb].mc = st[0] * F::kC + rs[sb].off;
    }
  }
  v4f acc[2][NCT + 1];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int ct = 0; ct <= NCT; ++ct) acc[sb][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  codes_dma<D>(p, bh, 0, lds, tid);
  scale_store<D>(scale_load<D>(p, bh, 0, tid), lds, tid);
  __builtin_amdgcn_s_waitcnt(0);  // the DMA has landed in LDS
  __syncthreads();

  // full tiles: no per-element masking; the next tile is copied into the
  // other buffer while this one is processed (on the last iteration the
  // clamped index copies this tile again into a buffer nothing reads later)
  for (int kt = 0; kt < nfull; ++kt) {
    const uint8_t* buf = lds + (kt & 1) * L::STAGE;
    uint8_t* nxt = lds + ((kt + 1) & 1) * L::STAGE;
    const int kn = min(kt + 1, nkt - 1);
    codes_dma<D>(p, bh, kn, nxt, tid);
    const ScaleRegs sr = scale_load<D>(p, bh, kn, tid);
    tile_step<D, CAUSAL, MODE, RULE, false>(buf, kt, p.N, qop, qsc, qi, rs, acc, r16, grp);
    scale_store<D>(sr, nxt, tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // at most one masked tile: the ragged end of the keys or the causal diagonal
  if (nfull < nkt)
    tile_step<D, CAUSAL, MODE, RULE, true>(lds + (nfull & 1) * L::STAGE, nfull, p.N, qop, qsc, qi, rs, acc,
                                           r16, grp);

  // ---- epilogue
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int q = qi[sb];
    if constexpr (MODE == kModeStats) {
      if (grp == 0) {
        float* st2 = p.stats + (bh * p.Np + q) * 2;
        st2[0] = rs[sb].m;
        st2[1] = rs[sb].l;
      }
      continue;
    }
    if (q >= p.N) continue;
    const float lsum = acc[sb][NCT][0];  // sum of beta-weighted P^ (the ones column)
    // O = O~ / l with a correctly rounded division (Eq. 8): with V^ constant
    // per channel, O~ = v^ l exactly, and the division returns v^ exactly
    float l;
    if constexpr (MODE == kModePnq) l = lsum;
    else if constexpr (MODE == kModeDirect) l = rs[sb].l;
    else l = 1.0f;
    float* orow = p.out + (bh * p.N + q) * D + 4 * grp;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const v4f o = acc[sb][ct];
      *reinterpret_cast<float4*>(orow + 16 * ct) = make_float4(o[0] / l, o[1] / l, o[2] / l, o[3] / l);
    }
    if (grp == 0) {
      if (p.row_stats) {
        p.row_stats[(bh * p.N + q) * 2 + 0] = rs[sb].m * F::kInvSqrtD;
        p.row_stats[(bh * p.N + q) * 2 + 1] = l;
      }
      if (p.row_sums) p.row_sums[bh * p.N + q] = (MODE == kModePostnorm) ? lsum : lsum / l;
    }
  }
}

template <int D, bool CAUSAL, int MODE, int RULE>
hipError_t launch_one(const Params& prm, int BH, hipStream_t stream) {
  const int64_t groups = (int64_t)BH * prm.nqt;
  hipLaunchKernelGGL((k_attention<D, CAUSAL, MODE, RULE>), dim3((unsigned)groups), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dispatch_mode(const AttnArgs& a, const Params& prm, hipStream_t s) {
  const int BH = a.B * a.H;
  if (a.mode == kModePnq && a.rule == kRuleUos) return launch_one<D, CAUSAL, kModePnq, kRuleUos>(prm, BH, s);
  if (a.mode == kModePnq) return launch_one<D, CAUSAL, kModePnq, kRuleOcp>(prm, BH, s);
  if (a.mode == kModeDirect)
    return a.rule == kRuleUos ? launch_one<D, CAUSAL, kModeDirect, kRuleUos>(prm, BH, s)
                              : launch_one<D, CAUSAL, kModeDirect, kRuleOcp>(prm, BH, s);
  // POSTNORM: exact row statistics first, then the quantized pass
  hipError_t err = launch_one<D, CAUSAL, kModeStats, kRuleUos>(prm, BH, s);
  if (err != hipSuccess) return err;
  return a.rule == kRuleUos ? launch_one<D, CAUSAL, kModePostnorm, kRuleUos>(prm, BH, s)
                            : launch_one<D, CAUSAL, kModePostnorm, kRuleOcp>(prm, BH, s);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  Params prm;
  prm.qc = a.qc; prm.qs = a.qs; prm.kc = a.kc; prm.ks = a.ks; prm.vc = a.vc; prm.vs = a.vs;
  prm.out = a.out;
  prm.row_stats = a.row_stats;
  prm.row_sums = a.row_sums;
  prm.stats = a.stats_ws;
  prm.H = a.H;
  prm.N = a.N;
  prm.Np = (int)padded_tokens(a.N);
  prm.nqt = prm.Np / kBr;
  if (a.d == 128) return a.causal ? dispatch_mode<128, true>(a, prm, stream) : dispatch_mode<128, false>(a, prm, stream);
  return a.causal ? dispatch_mode<64, true>(a, prm, stream) : dispatch_mode<64, false>(a, prm, stream);
}

}  // namespace mxattn_internal
