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

template <int D>
struct StageRegs {
  static constexpr int KCU = (kBc * D / 2 / 16) / 256;  // uint4 per thread
  static constexpr int VCU = (64 * D / 16) / 256;
  uint4 kc[KCU];
  uint4 vc[VCU];
  uint32_t ks;
  uint32_t vs;
};

template <int D>
__device__ __forceinline__ void stage_load(StageRegs<D>& st, const Params& p, int64_t bh, int kt, int tid) {
  const int NBp = p.Np / 32;
  const uint4* kb = reinterpret_cast<const uint4*>(p.kc + (bh * p.Np + (int64_t)kt * kBc) * (D / 2));
#pragma unroll
  for (int u = 0; u < StageRegs<D>::KCU; ++u) st.kc[u] = kb[tid + 256 * u];
  const uint4* vb = reinterpret_cast<const uint4*>(p.vc + (bh * NBp + (int64_t)kt * 4) * D * 16);
#pragma unroll
  for (int u = 0; u < StageRegs<D>::VCU; ++u) st.vc[u] = vb[tid + 256 * u];
  st.ks = 0;
  st.vs = 0;
  if (tid < kBc) {
    const uint8_t* ksrc = p.ks + (bh * p.Np + (int64_t)kt * kBc + tid) * (D / 32);
    if constexpr (D == 128) st.ks = *reinterpret_cast<const uint32_t*>(ksrc);
    else st.ks = *reinterpret_cast<const uint16_t*>(ksrc);
  }
  if (tid < D) st.vs = *reinterpret_cast<const uint32_t*>(p.vs + (bh * NBp + (int64_t)kt * 4) * D + 4 * tid);
}

template <int D>
__device__ __forceinline__ void stage_store(const StageRegs<D>& st, uint8_t* lds, int tid) {
  using L = Lds<D>;
#pragma unroll
  for (int u = 0; u < StageRegs<D>::KCU; ++u) {
    const int idx = tid + 256 * u;
    const int k = idx / (D / 32), c = idx % (D / 32);
    *reinterpret_cast<uint4*>(lds + L::KC + 16 * kc_granule<D>(k, c)) = st.kc[u];
  }
#pragma unroll
  for (int u = 0; u < StageRegs<D>::VCU; ++u)
    *reinterpret_cast<uint4*>(lds + L::VC + 16 * (tid + 256 * u)) = st.vc[u];
  if (tid < kBc) {
    const int k = tid, g = k >> 5, t = (k >> 2) & 7, i = k & 3, r = 4 * g + i;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) lds[L::KS + (c * 16 + r) * 8 + t] = (uint8_t)(st.ks >> (8 * c));
  }
  if (tid < D) {
    const int g = (4 * tid) / D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = (4 * tid) % D + j, ct = ch / 16, r = ch % 16;
      lds[L::VS + (g * 16 + r) * (D / 16) + ct] = (uint8_t)(st.vs >> (8 * j));
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

template <int D, bool CAUSAL, int MODE, int RULE>
__global__ __launch_bounds__(256) void k_attention(Params p) {
  using L = Lds<D>;
  constexpr int NCT = D / 16;  // 16-channel output tiles
  // Exponent arguments.  The fused path evaluates (s - m) c as one
  // fma(s, c, -m c); the row maximum then gives P~ = 1 within an ulp, which
  // the UOS rule maps to the interior value 4.  The OCP rule puts P~ = 1 on
  // its scale boundary (floor(log2 1) - 2), and the reference modes must
  // reproduce exact ties, so they evaluate fma(s - m, c, -off), which is
  // exact when s = m.
  constexpr bool kExactArg = !(MODE == kModePnq && RULE == kRuleUos);
  constexpr float kC = (D == 128) ? 0x1.0527dcp-3f : 0x1.715476p-3f;      // log2(e)/sqrt(d)
  constexpr float kInvSqrtD = (D == 128) ? 0x1.6a09e6p-4f : 0x1p-3f;      // 1/sqrt(d)
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
      rs[sb].mc = st[0] * kC + rs[sb].off;
    }
  }
  v4f acc[2][NCT + 1];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int ct = 0; ct <= NCT; ++ct) acc[sb][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  StageRegs<D> st;
  stage_load<D>(st, p, bh, 0, tid);
  stage_store<D>(st, lds, tid);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    uint8_t* buf = lds + (kt & 1) * L::STAGE;
    if (kt + 1 < nkt) stage_load<D>(st, p, bh, kt + 1, tid);

    // ---- S^T = K^ Q^T for 128 keys x 32 queries
    uint2 ksw = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    if (grp < D / 32) ksw = *reinterpret_cast<const uint2*>(buf + L::KS + (grp * 16 + r16) * 8);
    v4f s[2][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int k = 32 * (r16 >> 2) + 4 * t + (r16 & 3);
      uint4 a = *reinterpret_cast<const uint4*>(buf + L::KC + 16 * kc_granule<D>(k, grp & (D / 32 - 1)));
      if (grp >= D / 32) a = make_uint4(0, 0, 0, 0);
      const int sc = (t < 4) ? (int)ksw.x : (int)ksw.y;
      const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        switch (t & 3) {
          case 0: s[sb][t] = mfma4<0>(a, qop[sb], z, sc, qsc[sb]); break;
          case 1: s[sb][t] = mfma4<1>(a, qop[sb], z, sc, qsc[sb]); break;
          case 2: s[sb][t] = mfma4<2>(a, qop[sb], z, sc, qsc[sb]); break;
          default: s[sb][t] = mfma4<3>(a, qop[sb], z, sc, qsc[sb]); break;
        }
      }
    }

    // masks: keys past N (last tile) and keys after the query (causal diagonal)
    const bool need_mask = (kt * kBc + kBc > p.N) || (CAUSAL && kt == qt);
    if (need_mask) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt * kBc + 32 * grp + 4 * t + i;
            const bool ok = key < p.N && (!CAUSAL || key <= qi[sb]);
            if (!ok) s[sb][t][i] = -INFINITY;
          }
    }

    // ---- online softmax and P^ per sub-block
    uint4 pq[2];
    int psc[2];
    float alpha[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      float bmax = s[sb][0][0];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[sb][t][i]);
      float a = 1.0f;
      if constexpr (MODE != kModePostnorm) {
        float rmax = fmaxf(bmax, xor_lanes(bmax, 16));
        rmax = fmaxf(rmax, xor_lanes(rmax, 32));
        const float m_new = fmaxf(rs[sb].m, rmax);
        if (m_new != -INFINITY) {
          a = __builtin_amdgcn_exp2f((rs[sb].m - m_new) * kC);  // 0 on the first visited tile
          rs[sb].m = m_new;
          rs[sb].mc = m_new * kC;
        }
      }
      alpha[sb] = a;
      const float mc = rs[sb].mc;
      const float mref = rs[sb].m, off = rs[sb].off;
      if constexpr (MODE == kModeStats) {
        float sum = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f((s[sb][t][i] - mref) * kC);
        sum += xor_lanes(sum, 16);
        sum += xor_lanes(sum, 32);
        rs[sb].l = a * rs[sb].l + sum;
        pq[sb] = make_uint4(0, 0, 0, 0);
        psc[sb] = 127;
      } else {
        // block scale from the block max of the exponentials (exp is monotone)
        const float Mb = kExactArg ? __builtin_amdgcn_exp2f(fmaf(bmax - mref, kC, -off))
                                   : __builtin_amdgcn_exp2f(fmaf(bmax, kC, -mc));
        const int e = scale_exponent<RULE>(Mb);
        float y[32];
        if constexpr (kExactArg) {
          const float nb = -(off + (float)e);
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[4 * t + i] = __builtin_amdgcn_exp2f(fmaf(s[sb][t][i] - mref, kC, nb));
        } else {
          const float nb = -(mc + (float)e);
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[4 * t + i] = __builtin_amdgcn_exp2f(fmaf(s[sb][t][i], kC, nb));
        }
        if constexpr (MODE == kModeDirect) {
          float sum = 0.0f;
#pragma unroll
          for (int k = 0; k < 32; ++k) sum += y[k];
          sum = __builtin_amdgcn_ldexpf(sum, e);
          sum += xor_lanes(sum, 16);
          sum += xor_lanes(sum, 32);
          rs[sb].l = a * rs[sb].l + sum;
        }
        pq[sb] = make_uint4(pack_fp4x8(y), pack_fp4x8(y + 8), pack_fp4x8(y + 16), pack_fp4x8(y + 24));
        psc[sb] = e + 127;
      }
    }

    if constexpr (MODE != kModeStats) {
      // ---- rescale O~ (and the l column) when any running max moved
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (MODE != kModePostnorm && __any(alpha[sb] != 1.0f)) {
#pragma unroll
          for (int ct = 0; ct <= NCT; ++ct) acc[sb][ct] *= alpha[sb];
        }
      }
      // ---- O~ += P^ V^ and l += P^ 1
      uint2 vsw = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
      if constexpr (D == 128) vsw = *reinterpret_cast<const uint2*>(buf + L::VS + (grp * 16 + r16) * 8);
      else vsw.x = *reinterpret_cast<const uint32_t*>(buf + L::VS + (grp * 16 + r16) * 4);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint4 a = *reinterpret_cast<const uint4*>(buf + L::VC + 16 * (grp * D + 16 * ct + r16));
        const int sc = (ct < 4) ? (int)vsw.x : (int)vsw.y;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          switch (ct & 3) {
            case 0: acc[sb][ct] = mfma4<0>(a, pq[sb], acc[sb][ct], sc, psc[sb]); break;
            case 1: acc[sb][ct] = mfma4<1>(a, pq[sb], acc[sb][ct], sc, psc[sb]); break;
            case 2: acc[sb][ct] = mfma4<2>(a, pq[sb], acc[sb][ct], sc, psc[sb]); break;
            default: acc[sb][ct] = mfma4<3>(a, pq[sb], acc[sb][ct], sc, psc[sb]); break;
          }
        }
      }
      const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);  // E2M1 1.0
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) acc[sb][NCT] = mfma4<0>(ones, pq[sb], acc[sb][NCT], 127, psc[sb]);
    }

    if (kt + 1 < nkt) stage_store<D>(st, lds + ((kt + 1) & 1) * L::STAGE, tid);
    __syncthreads();
  }

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
        p.row_stats[(bh * p.N + q) * 2 + 0] = rs[sb].m * kInvSqrtD;
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
