// Fused MXFP4 attention forward of MXAttention for gfx950 (MI355X).
//
// One workgroup = 4 waves = 128 queries of one (batch, head); each wave owns
// 32 queries.  Key/value tiles of B_c = 128 keys are staged through LDS
// (double buffered) and visited in ascending order (MXAttention paper,
// Alg. 2, the loop over key/value tiles):
//
//   S^T  = K^ Q^T         scaled-FP4 MFMA 32x32x64: four 32-key x 32-query
//                         sub-tiles, d/64 products each (block scales along d
//                         ride in the MFMA)
//   m    = max(m, rowmax) running max per query                  (Eq. 3)
//   P~   = exp(S - m)     exponentials                           (Eq. 5)
//   P^   = Q*(P~)         UOS quantization per 32-key block      (Eq. 44)
//   l    = a l + P^ 1     the same P^ ...                        (Eq. 47)
//   O~   = a O~ + P^ V^   ... feeds both updates (PNQ)           (Eq. 48)
//   O    = O~ / l                                                (Eq. 8)
//
// Register layouts follow the gfx950 scaled MFMA 32x32x64: lane L supplies
// row/column L%32 and the 32-element K chunk L/32, and holds
// D[8j + 4(L/32) + i][L%32] in accumulator element 4j+i.  The A operand of
// sub-tile t of S^T takes its rows in the permuted key order
//   row r <- key 64(t/2) + 32((r/4)%2) + 16(t%2) + 4(r/8) + r%4,
// so that lane L (g = L/32) ends up with, for query L%32, the 32 consecutive
// keys 32g..32g+31 in sub-tiles 0 and 1 and the keys 64+32g..64+32g+31 in
// sub-tiles 2 and 3, each in ascending order.  Each is one 32-key
// quantization block, and each is exactly the lane's B-operand chunk of one
// 64-key step of the PV product: P^ never moves between lanes and its block
// maximum is lane-local.  The two lanes L and L^32 that share a query
// exchange their maxima with one v_permlane32_swap.
//
// l comes from a 16x16x128 MFMA of P^ against a 0/1 pattern: A row r takes
// the K chunks whose parity equals (r/4)%2, which sums, for every column, the
// two lanes that hold the same query, and lands l of query L%32 in all four
// accumulator elements of lane L.  l and O~ are thus updated from the same
// quantized tile by the same instruction stream (the PNQ identity).
//
// Scores stay in raw units (q^.k^); exp(s - m) is evaluated as
// exp2(fma(s, c, -m c)) with c = log2(e)/sqrt(d), and the block scale 2^e is
// folded into the exponent argument so P~/2^e goes straight to the FP4
// convert (round to nearest even, saturating at 6).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "internal.h"
#include "mx_block.h"
#include "row_divide.h"

namespace mxattn_internal {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBr = 128;       // queries per workgroup
constexpr int kThreads = 256;  // threads per workgroup
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
  float* diag;
  float gamma_f;      // DIAG: gamma = 2^k gamma_f, gamma_f in [1, 2)
  float inv_gamma_f;  // DIAG: 1 / gamma_f
  const uint16_t* qx;        // fused Q prologue: 16-bit Q [B, H, Nq, d]
  int64_t qsB, qsH, qsN;     // its element strides
  int qdtype;                // 0 bf16, 1 fp16
  int qrotate;               // Hadamard-rotate Q first
  int qrule;                 // 0 UOS, 1 OCP
  int H;
  int N, Np;    // keys / values: count and padded count
  int Nq, Nqp;  // queries: count and padded count
  int nqt;      // query tiles per head
};

// byte offsets inside one LDS stage
template <int D>
struct Lds {
  static constexpr int KC = 0;                  // K^ codes, swizzled 16-byte granules
  static constexpr int KS = KC + kBc * D / 2;   // K^ scales, [lane][sub-tile pair] dwords
  static constexpr int VC = KS + 64 * 8;        // V^ codes [block][channel][16]
  static constexpr int VS = VC + 64 * D;        // V^ scales, [lane][PV step] dwords
  static constexpr int STAGE = VS + 64 * 8;
  // the fused Q prologue parks Q^ of the workgroup's kBr rows in a stage
  static_assert(kBr * D / 2 <= KS - KC && kBr * D / 32 <= VC - KS, "Q^ scratch exceeds a stage");
};

// key (0..127 within the tile) on A-operand row r of S^T sub-tile t
__device__ __forceinline__ int tile_key(int t, int r) {
  return 64 * (t >> 1) + 32 * ((r >> 2) & 1) + 16 * (t & 1) + 4 * (r >> 3) + (r & 3);
}

// K^ tile in LDS: key k's 16-byte d-chunk c sits in granule (d/32) k + (c ^ x(k)).
// An operand read of one sub-tile has lanes 0..7 fetch keys b+{0..3} and
// b+32+{0..3}, lanes 8..15 keys b+4+{0..3} and b+36+{0..3} (same chunk); the
// XOR term makes both every 8-lane and every 16-lane group of such a read
// touch distinct granules modulo 8 and modulo 16.
template <int D>
__device__ __forceinline__ int kc_swizzle(int k) {
  if constexpr (D == 128) return (((k >> 1) ^ (k >> 2)) & 1) | (((k >> 5) & 1) << 1);
  else return (k >> 5) & 1;
}

template <int D>
__device__ __forceinline__ int kc_granule(int k, int c) {
  return (D / 32) * k + (c ^ kc_swizzle<D>(k));
}

// (key, d-chunk) index (d/32) k + c held by LDS granule G (inverse of kc_granule)
template <int D>
__device__ __forceinline__ int kc_source_chunk(int G) {
  constexpr int NC = D / 32;
  const int k = G / NC;
  return NC * k + ((G % NC) ^ kc_swizzle<D>(k));
}

// Stage one key/value tile into LDS.  The code bytes (16 KB at d = 128) go
// straight from global memory into LDS with global_load_lds_dwordx4: lane i
// of a wave writes LDS granule base + i, so each lane fetches the global
// 16-byte chunk that belongs in that (swizzled) granule.  The scale bytes are
// few; they pass through registers and are scattered into their operand
// order with small stores (scale_store).
// Tile copies go through buffer descriptors: the tile's base address and
// size live in scalar registers and each lane adds a 32-bit offset, so moving
// to the next tile is scalar arithmetic only (with flat 64-bit addresses the
// vector unit spent a 64-bit add per copy and tile).  An offset past `bytes`
// reads zeros instead of faulting.  Device code only: the descriptor type and
// the LDS address space do not exist in the host pass.
#if defined(__HIP_DEVICE_COMPILE__)
constexpr int kRawBufferWord3 = 0x00020000;  // descriptor word 3: raw dwords

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, kRawBufferWord3);
}

// LDS-destination copy of one 16-byte chunk per lane, from byte voff + soff
// of the descriptor's range
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int soff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_base)), 16,
      (int)voff, soff, 0, 0);
}
#endif

// Per-lane source offsets of the DMA: loop-invariant, computed once.  The
// wave index is uniform; keeping it scalar makes each LDS base (M0) a scalar
// value.
template <int D>
struct DmaPlan {
  static constexpr int KU = kBc * D / 2 / 16 / 256;  // K^ granules per lane
  static constexpr int VU = 64 * D / 16 / 256;       // V^ granules per lane
  uint32_t koff[KU];
  int lds0;  // 16 * (64 * wave): granule base of this wave in each 256-granule round
  __device__ __forceinline__ DmaPlan(int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    lds0 = 16 * 64 * wave;
#pragma unroll
    for (int u = 0; u < KU; ++u) koff[u] = (uint32_t)(16 * kc_source_chunk<D>(u * 256 + wave * 64 + lane));
  }
};

template <int D>
__device__ __forceinline__ void codes_dma(const Params& p, const DmaPlan<D>& plan, int64_t bh, int kt, uint8_t* stage,
                                          int tid) {
  using L = Lds<D>;
  const int NBp = p.Np / 32;
  const uint32_t voff = (uint32_t)(plan.lds0 + 16 * (tid & 63));
  const uint8_t* kb = p.kc + (bh * p.Np + (int64_t)kt * kBc) * (D / 2);
  const uint8_t* vb = p.vc + (bh * NBp + (int64_t)kt * 4) * D * 16;
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kb, kBc * D / 2), vr = tile_rsrc(vb, 64 * D);
#pragma unroll
  for (int u = 0; u < DmaPlan<D>::KU; ++u) dma16(kr, plan.koff[u], 0, stage + L::KC + u * 4096 + plan.lds0);
#pragma unroll
  for (int u = 0; u < DmaPlan<D>::VU; ++u) dma16(vr, voff, u * 4096, stage + L::VC + u * 4096 + plan.lds0);
#endif
}

struct ScaleRegs {
  uint32_t ks;
  uint32_t vs;
};

// Thread k < 128 (waves 0-1) loads the d/32 scale bytes of key k; the last
// d threads (waves 2-3 at d = 128), j = tid - (256 - d), load scale bytes
// 4j..4j+3 of the tile's [block][channel] V^ scales: the staging work is
// split between the waves, which meet at every tile's barrier.
template <int D>
__device__ __forceinline__ ScaleRegs scale_load(const Params& p, int64_t bh, int kt, int tid) {
  const int NBp = p.Np / 32;
  ScaleRegs r = {0u, 0u};
#if defined(__HIP_DEVICE_COMPILE__)
  if (tid < kBc) {
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(p.ks + (bh * p.Np + (int64_t)kt * kBc) * (D / 32), kBc * D / 32);
    if constexpr (D == 128) r.ks = __builtin_amdgcn_raw_buffer_load_b32(kr, 4 * tid, 0, 0);
    else r.ks = __builtin_amdgcn_raw_buffer_load_b16(kr, 2 * tid, 0, 0);
  }
  if (tid >= kThreads - D) {
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(p.vs + (bh * NBp + (int64_t)kt * 4) * D, 4 * D);
    r.vs = __builtin_amdgcn_raw_buffer_load_b32(vr, 4 * (tid - (kThreads - D)), 0, 0);
  }
#endif
  return r;
}

// Scatter the scale bytes into per-lane operand order.
//   K^: lane r + 32g, dword t/2, byte (t%2)(d/64) + h holds the scale of key
//       tile_key(t, r), d-block 2h + g (the A operand of S^T sub-tile t, step h);
//   V^: lane L, dword h, byte ct holds the scale of block 2h + L/32, channel
//       32ct + L%32 (the A operand of PV step h, channel tile ct).
template <int D>
__device__ __forceinline__ void scale_store(const ScaleRegs& sr, uint8_t* stage, int tid) {
  using L = Lds<D>;
  if (tid < kBc) {
    const int k = tid;
    const int t = 2 * (k >> 6) + ((k >> 4) & 1);
    const int r = 8 * ((k >> 2) & 3) + 4 * ((k >> 5) & 1) + (k & 3);
    uint8_t* base = stage + L::KS + 4 * (t >> 1);
    const uint32_t s = sr.ks;
    if constexpr (D == 128) {
      *reinterpret_cast<uint16_t*>(base + 8 * r + 2 * (t & 1)) = (uint16_t)((s & 0xFFu) | ((s >> 8) & 0xFF00u));
      *reinterpret_cast<uint16_t*>(base + 8 * (r + 32) + 2 * (t & 1)) =
          (uint16_t)(((s >> 8) & 0xFFu) | ((s >> 16) & 0xFF00u));
    } else {
      base[8 * r + (t & 1)] = (uint8_t)(s & 0xFFu);
      base[8 * (r + 32) + (t & 1)] = (uint8_t)((s >> 8) & 0xFFu);
    }
  }
  if (tid >= kThreads - D) {
    const int j = tid - (kThreads - D);
    const int bl = (4 * j) / D, ch0 = (4 * j) % D;
    const int lane0 = 32 * (bl & 1) + (ch0 & 31);
    uint8_t* base = stage + L::VS + 4 * (bl >> 1) + (ch0 >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) base[8 * (lane0 + i)] = (uint8_t)(sr.vs >> (8 * i));
  }
}

__device__ __forceinline__ v8i as_op(uint4 a) {
  v8i r = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  return r;
}

template <int OA, int OB>
__device__ __forceinline__ v16f mfma32(uint4 a, uint4 b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_op(a), as_op(b), c, 4, 4, OA, sa, OB, sb);
}

// scale-byte selectors are immediates; after unrolling oa and ob are constants
__device__ __forceinline__ v16f mfma32_sel(int oa, int ob, uint4 a, uint4 b, v16f c, int sa, int sb) {
  if (ob == 0) {
    switch (oa) {
      case 0: return mfma32<0, 0>(a, b, c, sa, sb);
      case 1: return mfma32<1, 0>(a, b, c, sa, sb);
      case 2: return mfma32<2, 0>(a, b, c, sa, sb);
      default: return mfma32<3, 0>(a, b, c, sa, sb);
    }
  }
  switch (oa) {
    case 0: return mfma32<0, 1>(a, b, c, sa, sb);
    case 1: return mfma32<1, 1>(a, b, c, sa, sb);
    case 2: return mfma32<2, 1>(a, b, c, sa, sb);
    default: return mfma32<3, 1>(a, b, c, sa, sb);
  }
}

__device__ __forceinline__ v4f mfma16(uint4 a, uint4 b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_op(a), as_op(b), c, 4, 4, 0, sa, 0, sb);
}

// The E8M0 scale operands of the scaled MFMAs are read by the matrix core
// after the instruction issues (rows of a 32x32 product that execute in later
// passes see later register contents), but the compiler treats them as read
// at issue and may reuse their registers at once.  Every scale register is
// therefore kept live until a value exists that the matrix core can only
// have produced after that product: keep_live() ties the registers to such a
// value with an empty asm statement.  The PV products of a tile are followed,
// on the same matrix core, by the S products of the next tile, so the next
// tile's score maximum serves; after the last tile, the accumulators do.
__device__ __forceinline__ void keep_live(float after, int a, int b = 0, int c = 0, int d = 0) {
  asm volatile("" ::"v"(after), "v"(a), "v"(b), "v"(c), "v"(d));
}

// Shared-scale exponent of a block with max M >= 0 from the binary32 fields
// of M (see the quantizer kernels for the derivation); M = 0 gives 0, a
// subnormal M the clamp value -127.  Written without branches: M comes from
// exp2 and is never negative, infinite or NaN.
template <int RULE>
__device__ __forceinline__ int scale_exponent(float M) {
  const uint32_t b = __float_as_uint(M);
  const int E = (int)(b >> 23);
  int e = E - 129;
  if constexpr (RULE == kRuleUos) e += ((b & 0x7FFFFFu) > 0x680000u) ? 1 : 0;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return b == 0u ? 0 : e;
}

// max / sum over the two lanes L and L^32 that hold the same query; both
// lanes get the same value (the sum is formed in the same order in both)
__device__ __forceinline__ float pair_max(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(x[0]) + __uint_as_float(x[1]);
}

// eight E2M1 codes, element 2k in the low nibble of byte k; the four converts
// write all four bytes, so the merge input of the first one is irrelevant
// (passing y[0]'s bits spares a register clear)
__device__ __forceinline__ uint32_t pack_fp4x8(const float* y) {
  uint32_t w = __float_as_uint(y[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// Per-query state, replicated in the two lanes that share a query.
struct RowState {
  float m;    // running max of raw scores (or m* for POSTNORM)
  float mc;   // m * c + off
  float mcL;  // mc + log2(7.25): the fused UOS block-scale offset
  float off;  // POSTNORM: log2 l* (P = exp(s - m*) / l*); otherwise 0
  float l;    // DIRECT: running sum of unquantized exponentials
  // STATS: the row's exponentials split at the running maximum, l = cnt + sig:
  // cnt keys at it (each exp(0) = 1 exactly) and the mass sig of the keys
  // below it, so that rho = l - 1 = (cnt - 1) + sig keeps its relative
  // precision however small it is.  POSTNORM / DIAG read rho back.
  float cnt;
  float sig;
  float rho;
};

// OCP exponent floor(log2(x)) - 2 of a block whose maximum is the row
// maximum's element, x = gamma_f / l* with l* = 1 + rho and gamma_f in [1, 2)
// (1 for the post-normalized P).  While rho < 1, x lies in (1/2, 2) and
// x >= 1 exactly when gamma_f - 1 >= rho, a comparison of two binary32 values
// with no rounding (gamma_f - 1 is exact): the decision at the boundary x = 1
// is exact, as P = 1/l* < 1 whenever any other key has mass.  Beyond, the
// binary32 quotient decides.
__device__ __forceinline__ int ocp_exponent_at_row_max(float gamma_f, float rho) {
  if (rho < 1.0f) return (gamma_f - 1.0f >= rho) ? -2 : -3;
  const float x = gamma_f / (1.0f + rho);
  return (int)(__float_as_uint(x) >> 23) - 129;  // x is a normal binary32 in (0, 1)
}

template <int D, int MODE, int RULE>
struct FwdConsts {
  // Exponent arguments.  The fused path evaluates (s - m) c as one
  // fma(s, c, -m c); the row maximum then gives P~ = 1 within an ulp, which
  // the UOS rule maps to the interior value 4.  The OCP rule puts P~ = 1 on
  // its scale boundary (floor(log2 1) - 2), and the reference modes must
  // reproduce exact ties, so they evaluate fma(s - m, c, -off), which is
  // exact when s = m.
  static constexpr bool kExactArg = !(MODE == kModePnq && RULE == kRuleUos);
  // the running maximum is fixed (exact statistics of a first pass)
  static constexpr bool kFixedM = (MODE == kModePostnorm || MODE == kModeDiag);
  static constexpr float kC = (D == 128) ? 0x1.0527dcp-3f : 0x1.715476p-3f;  // log2(e)/sqrt(d)
  static constexpr float kInvSqrtD = (D == 128) ? 0x1.6a09e6p-4f : 0x1p-3f;  // 1/sqrt(d)
};

// P^ of one 32-key block of the lane's query: the 16 scores of sub-tile pair
// (s0, s1) in key order, block max bmax.  Returns the packed FP4 B operand of
// the PV step; writes its E8M0 scale and (DIRECT) the block's contribution to
// the unquantized row sum.
template <int D, int MODE, int RULE>
__device__ __forceinline__ uint4 quantize_block(const v16f& s0, const v16f& s1, float bmax, const RowState& rs,
                                                int& psc, float& lpart) {
  using F = FwdConsts<D, MODE, RULE>;
  // block scale from the block max of the exponentials (exp is monotone)
  int e = 0;
  float ef = 0.0f;
  if constexpr (F::kExactArg) {
    e = scale_exponent<RULE>(__builtin_amdgcn_exp2f(fmaf(bmax - rs.m, F::kC, -rs.off)));
    // post-normalized P at the row maximum is 1/l*, below 1 exactly when
    // rho = l* - 1 > 0; OCP has a scale boundary at 1, so that block's
    // exponent is decided from rho, not from the rounded exp2(-log2 l*)
    if constexpr (MODE == kModePostnorm && RULE == kRuleOcp)
      if (bmax == rs.m) e = ocp_exponent_at_row_max(1.0f, rs.rho);
  } else {
    // UOS in the log domain: e = ceil(log2(Mb) - log2(7.25)) with
    // log2(Mb) = bmax c - m c, the same argument the exponentials use; its
    // binary32 rounding moves a scale decision only within the decision
    // margin of the exp2 evaluation.  A fully masked block (-inf) takes the
    // clamp; its elements are all zero whatever the scale.
    // (bmax <= m, so e <= ceil(-log2 7.25) = -2: no upper clamp)
    ef = __builtin_ceilf(fmaxf(fmaf(bmax, F::kC, -rs.mcL), -127.0f));
  }
  float y[32];
  if constexpr (F::kExactArg) {
    const float nb = -(rs.off + (float)e);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      y[k] = __builtin_amdgcn_exp2f(fmaf(s0[k] - rs.m, F::kC, nb));
      y[16 + k] = __builtin_amdgcn_exp2f(fmaf(s1[k] - rs.m, F::kC, nb));
    }
  } else {
    const float nb = -(rs.mc + ef);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      y[k] = __builtin_amdgcn_exp2f(fmaf(s0[k], F::kC, nb));
      y[16 + k] = __builtin_amdgcn_exp2f(fmaf(s1[k], F::kC, nb));
    }
  }
  if constexpr (MODE == kModeDirect) {
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) sum += y[k];
    lpart = __builtin_amdgcn_ldexpf(sum, e);
  }
  // the E8M0 byte: e + 127 as the low byte of ef + (1.5 2^23 + 127) (an
  // exact sum; the products read only byte 0 of their scale registers)
  if constexpr (F::kExactArg) psc = e + 127;
  else psc = __float_as_int(ef + 12583039.0f);
  return make_uint4(pack_fp4x8(y), pack_fp4x8(y + 8), pack_fp4x8(y + 16), pack_fp4x8(y + 24));
}

// the two E2M1 values in byte BYTE of w (elements 2 BYTE and 2 BYTE + 1)
template <int BYTE>
__device__ __forceinline__ void decode_fp4x2(uint32_t w, float& lo, float& hi) {
  const auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, BYTE);
  lo = p[0];
  hi = p[1];
}

// Row-sum diagnostics of one 32-key block of the lane's query (Sec. 5.5.2,
// Fig. 7) for the exact softmax P = exp2(a), a = (s - m) c - off with
// off = log2 l.  The quantizer input is gamma P.  A power-of-two factor of
// gamma = 2^k gamma_f only moves the block exponent by k and cancels in
// Q(gamma P) / gamma, so only gamma_f enters: the block scale 2^e comes from
// gamma_f max(P), and y = gamma_f P / 2^e goes to the FP4 convert.  Per
// block, in units of 2^e / gamma_f: the grid values g give the row sum
// (sum g) and the errors g - y split by outcome -- zeroing (g = 0 < y),
// saturation (y > 6), downward or upward rounding; the entropy term
// P log2 P = y (a) in the same units.
// dg: [row sum, zeroing, saturation, down, up, sum P log2 P].
//
// Per element only the sums that need a threshold are formed, without lane
// masks (y >= 0, and g = 0 or g >= 1/2):
//   up    max(g - y, 0);
//   sat   min(6 - y, 0), which is g - y where y > 6 (the convert saturates
//         to g = 6 there) and 0 elsewhere;
//   zero  -y times z = max(1 - 4g, 0), which is 1 at g = 0 and 0 at any
//         other grid value (a fused multiply-add, exact for z in {0, 1}).
// The four classes of one element add up to g - y, so the block's down sum
// is (sum g - sum y) - up - zero - sat, and its entropy term is
// e sum y + sum y a' with a' = log2(P / 2^e) the convert's exponent argument.
// Each product and difference is rounded on its own (no contraction), so the
// errors are those of the convert's actual input y.  Invisible keys (masked
// tiles only) have a' = -inf and y = 0; there a' is clamped to keep 0 a'
// finite.
template <int D, int RULE, bool MASKED>
__device__ __forceinline__ void diag_block(const v16f& s0, const v16f& s1, float bmax, const RowState& rs,
                                           float gamma_f, float inv_gamma_f, float (&dg)[6]) {
  using F = FwdConsts<D, kModeDiag, RULE>;
  int e = scale_exponent<RULE>(__builtin_amdgcn_exp2f(fmaf(bmax - rs.m, F::kC, -rs.off)) * gamma_f);
  // gamma_f P at the row maximum is gamma_f / l*: at OCP's scale boundary
  // gamma_f / l* = 1 the exponent is decided exactly from rho = l* - 1
  if constexpr (RULE == kRuleOcp)
    if (bmax == rs.m) e = ocp_exponent_at_row_max(gamma_f, rs.rho);
  const float nb = -(rs.off + (float)e);
  float gsum = 0.0f, ysum = 0.0f, cz = 0.0f, cs = 0.0f, cu = 0.0f, yarg = 0.0f;
  // eight elements at a time: exponentials, codes, their values, the sums
#pragma unroll
  for (int c8 = 0; c8 < 4; ++c8) {
    const v16f& src = (c8 < 2) ? s0 : s1;
    float arg[8], y[8], gq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      arg[k] = fmaf(src[8 * (c8 & 1) + k] - rs.m, F::kC, nb);  // log2(P / 2^e)
      y[k] = __builtin_amdgcn_exp2f(arg[k]) * gamma_f;
    }
    const uint32_t w = pack_fp4x8(y);
    decode_fp4x2<0>(w, gq[0], gq[1]);
    decode_fp4x2<1>(w, gq[2], gq[3]);
    decode_fp4x2<2>(w, gq[4], gq[5]);
    decode_fp4x2<3>(w, gq[6], gq[7]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
#pragma clang fp contract(off)
      const float g = gq[k], yy = y[k];
      gsum += g;
      ysum += yy;
      cu += fmaxf(g - yy, 0.0f);
      cz = fmaf(-yy, fmaxf(fmaf(-4.0f, g, 1.0f), 0.0f), cz);
      cs += fminf(6.0f - yy, 0.0f);
      yarg = fmaf(yy, MASKED ? fmaxf(arg[k], -0x1.fffffep+127f) : arg[k], yarg);
    }
    __builtin_amdgcn_sched_barrier(0);  // one group of eight live at a time
  }
  const float cd = (((gsum - ysum) - cu) - cz) - cs;
  const float ent = fmaf((float)e, ysum, yarg);
  // back from block units: P^ = g 2^e / gamma_f, P = y 2^e / gamma_f
  const float unit = __builtin_amdgcn_ldexpf(inv_gamma_f, e);
  dg[0] = fmaf(gsum, unit, dg[0]);
  dg[1] = fmaf(cz, unit, dg[1]);
  dg[2] = fmaf(cs, unit, dg[2]);
  dg[3] = fmaf(cd, unit, dg[3]);
  dg[4] = fmaf(cu, unit, dg[4]);
  dg[5] = fmaf(ent, unit, dg[5]);
}

// scores of keys the query may not see -> -inf (element 4j+i of sub-tile t
// of lane group g is key 64(t/2) + 32g + 16(t%2) + 4j + i of the tile)
template <bool CAUSAL, bool MASKED>
__device__ __forceinline__ void mask_scores(v16f (&s)[4], int kt, int N, int q, int g) {
  if constexpr (MASKED) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kt * kBc + 64 * (t >> 1) + 32 * g + 16 * (t & 1) + e;
        if (!(key < N && (!CAUSAL || key <= q))) s[t][e] = -INFINITY;
      }
  }
}

// one running chain, which the compiler turns into v_max3_f32 (two new
// elements per instruction)
__device__ __forceinline__ float max32(const v16f& a, const v16f& b) {
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < 16; ++k) m = fmaxf(m, a[k]);
#pragma unroll
  for (int k = 0; k < 16; ++k) m = fmaxf(m, b[k]);
  return m;
}

// Fused Q prologue (Sec. 4.3: the rotation belongs to the Q preprocessing):
// the wave rotates and quantizes its own 32 query rows exactly as the
// standalone head-dimension quantizer does, with the same block device code,
// and leaves codes and scales in the Q^ layout: rows of d/2 code bytes at
// `codes`, rows of d/32 scale bytes at `scales`.  Lane L takes the
// 32-channel blocks u = 64 it + L, it < d/64: row u / (d/32), block
// u % (d/32), so each row's blocks sit in one quad, as the butterflies need.
// Rows past the last query are zero (codes 0, scale 2^0), as in Q^'s padding.
template <int D>
__device__ __forceinline__ void q_prologue_load(const Params& p, int64_t bh, int row0, int lane,
                                                uint4 (&raw)[D / 64][4]) {
  constexpr int BPR = D / 32;
  const int64_t b = bh / p.H, h = bh % p.H;
#pragma unroll
  for (int it = 0; it < D / 64; ++it) {
    const int u = 64 * it + lane;
    const int n = row0 + u / BPR, blk = u % BPR;
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[it][k] = make_uint4(0u, 0u, 0u, 0u);
    if (n < p.Nq) {
      const uint4* src = reinterpret_cast<const uint4*>(p.qx + b * p.qsB + h * p.qsH + (int64_t)n * p.qsN + 32 * blk);
#pragma unroll
      for (int k = 0; k < 4; ++k) raw[it][k] = src[k];
    }
  }
}

template <int D>
__device__ __forceinline__ void q_prologue_quantize(const Params& p, int lane, const uint4 (&raw)[D / 64][4],
                                                    uint8_t* codes, uint8_t* scales) {
  constexpr int BPR = D / 32;
#pragma unroll
  for (int it = 0; it < D / 64; ++it) {
    const int u = 64 * it + lane;
    const int row = u / BPR, blk = u % BPR;
    float v[32];
    if (p.qdtype == 0) mxblock::unpack_block<0>(raw[it], v);
    else mxblock::unpack_block<1>(raw[it], v);
    float M;
    if (p.qrotate) {
      mxblock::rotate_block<D>(v, blk);
      M = mxblock::finish_block<D, true>(v);
    } else {
      M = mxblock::finish_block<D, false>(v);
    }
    const int e = (p.qrule == kRuleUos) ? mxblock::scale_exponent<mxblock::kRuleUos>(M)
                                        : mxblock::scale_exponent<mxblock::kRuleOcp>(M);
    *reinterpret_cast<uint4*>(codes + row * (D / 2) + 16 * blk) = mxblock::block_codes(v, e);
    scales[row * BPR + blk] = (uint8_t)(e + 127);
  }
}

// Deferred PV products.  At d = 64, and under the causal mask, the PV
// products of a tile's second 64-key half are issued in the next tile, right
// after its score products, instead of at the end of their own tile (after
// the last key tile they are issued before the epilogue).  At d = 64 this
// leaves fewer registers live across the tile boundary (165 instead of 184
// VGPRs, so three waves fit per SIMD instead of two) and measured 17-19 %
// faster; under the causal mask it measured 2-4 % faster at d = 128, and
// 1-2 % slower on the non-causal d = 128 shape, which keeps the original
// order.  The order of the products on each accumulator is unchanged, so the
// results are bit-identical.
template <int D, bool CAUSAL>
constexpr bool kDeferPV = (D == 64) || CAUSAL;

template <int D>
struct PendingPV {
  uint4 vop[D / 32];  // V^ operands of the deferred half
  uint4 pq;           // its P^ codes (all zero: nothing deferred yet)
  int vsc, psc;       // its V^ and P^ scale registers
};

template <int D>
__device__ __forceinline__ void issue_pending(const PendingPV<D>& pd, v16f (&acc)[D / 32], v4f& accl, uint4 ones,
                                              int one_sc) {
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) acc[ct] = mfma32_sel(ct, 0, pd.vop[ct], pd.pq, acc[ct], pd.vsc, pd.psc);
  accl = mfma16(ones, pd.pq, accl, one_sc, pd.psc);
}

// One key tile for the wave's 32 queries.  Order: all S products; block and
// row maxima (with kDeferPV, the previous tile's deferred PV products go out
// here); P^ of the first 64-key half and its PV products, which run on the
// matrix cores while P^ of the second half is formed; then the second half's
// PV products (with kDeferPV, kept for the next tile).  MASKED tiles (the
// ragged last tile and the causal diagonal) set scores of invisible keys to
// -inf; every other tile runs without any per-element test.
template <int D, bool CAUSAL, int MODE, int RULE, bool MASKED>
__device__ __forceinline__ void tile_step(const uint8_t* __restrict__ buf, int kt, int N, const uint4 (&qop)[D / 64],
                                          int qsc, int q, uint4 ones, int one_sc, RowState& rs, v16f (&acc)[D / 32],
                                          v4f& accl, int (&held)[4], int lane, const int (&koff)[D / 64],
                                          float (&dg)[6], float gamma_f, float inv_gamma_f, PendingPV<D>& pend) {
  using L = Lds<D>;
  using F = FwdConsts<D, MODE, RULE>;
  constexpr int NH = D / 64;   // K steps of one S^T sub-tile
  constexpr int NCT = D / 32;  // 32-channel output tiles
  const int r = lane & 31, g = lane >> 5;

  // ---- S^T = K^ Q^T for 128 keys x 32 queries
  const uint2 ksw = *reinterpret_cast<const uint2*>(buf + L::KS + 8 * lane);
  uint4 kop[4][NH];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int h = 0; h < NH; ++h)
      kop[t][h] = *reinterpret_cast<const uint4*>(buf + koff[h] + (D / 2) * (64 * (t >> 1) + 16 * (t & 1)));
  // the burst of score products runs at raised wave priority, so that it
  // reaches the matrix core ahead of the co-resident wave's vector work.  On
  // unmasked tiles without deferred products, the first block maximum (which
  // needs only the first two sub-tiles) is formed between the last products,
  // so the wave's own vector work runs under its burst.
  constexpr bool kDefer = kDeferPV<D, CAUSAL> && MODE != kModeStats && MODE != kModeDiag;
  constexpr bool kSplit = !MASKED && !kDefer;
  v16f s[4];
  float bmax[2];
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s[t] = v16f{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int h = 0; h < NH; ++h)
      s[t] = mfma32_sel((t & 1) * NH + h, h, kop[t][h], qop[h], s[t], (t < 2) ? (int)ksw.x : (int)ksw.y, qsc);
  }
  if constexpr (kSplit) {
    bmax[0] = max32(s[0], s[1]);
    // order: 2 NH + 1 products, then (4 vector instructions, 1 product) x (2 NH - 1)
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NH + 1, 0);
#pragma unroll
    for (int i = 0; i < 2 * NH - 1; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- running max, block maxima, alpha (and the deferred PV products of
  // the previous tile, which must precede this tile's rescale)
  mask_scores<CAUSAL, MASKED>(s, kt, N, q, g);
  if constexpr (!kSplit) bmax[0] = max32(s[0], s[1]);
  if constexpr (kDefer) issue_pending<D>(pend, acc, accl, ones, one_sc);
  bmax[1] = max32(s[2], s[3]);
  const float tmax = fmaxf(bmax[0], bmax[1]);
  // this tile's S products and the previous tile's PV products have read
  // their scales once tmax exists
  keep_live(tmax, (int)ksw.x, (int)ksw.y, one_sc, qsc);
  keep_live(tmax, held[0], held[1], held[2], held[3]);
  float a = 1.0f;
  bool moved = false;  // the running maximum rose in this tile
  if constexpr (!F::kFixedM) {
    const float m_new = fmaxf(rs.m, pair_max(tmax));
    moved = m_new > rs.m;
    if (m_new != -INFINITY) {
      a = __builtin_amdgcn_exp2f((rs.m - m_new) * F::kC);  // 0 on the first visited tile
      rs.m = m_new;
      rs.mc = m_new * F::kC;
      rs.mcL = rs.mc + 0x1.6dd252p+1f;  // log2(7.25)
    }
  }
  if constexpr (MODE == kModeStats) {
    // keys below the (new) running maximum add their exponentials to sig,
    // keys at it count one each; invisible keys (-inf) add nothing
    float sum = 0.0f, cnt = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = s[t][e];
        if (v < rs.m) sum += __builtin_amdgcn_exp2f((v - rs.m) * F::kC);
        else if (v == rs.m) cnt += 1.0f;
      }
    sum = pair_sum(sum);
    cnt = pair_sum(cnt);
    if (moved) {  // every earlier key now lies below the maximum
      rs.sig = a * (rs.cnt + rs.sig) + sum;
      rs.cnt = cnt;
    } else {
      rs.sig += sum;
      rs.cnt += cnt;
    }
  } else if constexpr (MODE == kModeDiag) {
    __builtin_amdgcn_sched_barrier(0);
    diag_block<D, RULE, MASKED>(s[0], s[1], bmax[0], rs, gamma_f, inv_gamma_f, dg);
    diag_block<D, RULE, MASKED>(s[2], s[3], bmax[1], rs, gamma_f, inv_gamma_f, dg);
  } else {
    const uint2 vsw = *reinterpret_cast<const uint2*>(buf + L::VS + 8 * lane);
    if constexpr (MODE != kModePostnorm) {
      if (__any(a != 1.0f)) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] *= a;
        accl *= a;
      }
    }
    float lsum = 0.0f;
    if constexpr (kDefer) {  // scales of the deferred products issued above
      held[0] = pend.vsc;
      held[1] = pend.psc;
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      uint4 vop[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        vop[ct] = *reinterpret_cast<const uint4*>(buf + L::VC + 16 * ((2 * hb + g) * D + 32 * ct + r));
      int psc;
      float lpart = 0.0f;
      const uint4 pq = quantize_block<D, MODE, RULE>(s[2 * hb], s[2 * hb + 1], bmax[hb], rs, psc, lpart);
      lsum += lpart;
      const int vsc = hb ? (int)vsw.y : (int)vsw.x;
      if (kDefer && hb == 1) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) pend.vop[ct] = vop[ct];
        pend.pq = pq;
        pend.vsc = vsc;
        pend.psc = psc;
      } else {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] = mfma32_sel(ct, 0, vop[ct], pq, acc[ct], vsc, psc);
        accl = mfma16(ones, pq, accl, one_sc, psc);
        __builtin_amdgcn_sched_barrier(0);
        // scale registers of the products issued in this tile
        if (kDefer) {
          held[2] = vsc;
          held[3] = psc;
        } else {
          held[hb] = vsc;
          held[2 + hb] = psc;
        }
      }
    }
    if constexpr (MODE == kModeDirect) rs.l = a * rs.l + pair_sum(lsum);
  }
}

template <int D>
constexpr int kLdsBytes = 2 * Lds<D>::STAGE;  // two key/value stages

// Key/value tiles the resident-key kernel keeps in LDS for a whole head: at
// two workgroups per CU, 4 x 17 KB at d = 128 and 8 x 9 KB at d = 64.
template <int D>
constexpr int kResidentTiles = D == 128 ? 4 : 8;

// Q^ operand of one wave's 32 queries of query tile qt (B operand of S^T:
// lane = query L%32, d-chunk 2h + L/32 in step h) and its scale bytes
// (sb[h] = d-block 2h + L/32), kept apart until the operand is used so that
// loading them waits for nothing
template <int D>
struct QOperand {
  uint4 op[D / 64];
  int sb[D / 64];
  // scale register of the products: byte h = sb[h]
  __device__ __forceinline__ int sc() const {
    if constexpr (D == 128) return sb[0] | (sb[1] << 8);
    else return sb[0];
  }
};

template <int D>
__device__ __forceinline__ void load_qoperand(const Params& p, int64_t bh, int qt, int wave, int r, int g,
                                              QOperand<D>& q) {
  const int64_t qrow = bh * p.Nqp + qt * kBr + 32 * wave + r;
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    q.op[h] = *reinterpret_cast<const uint4*>(p.qc + qrow * (D / 2) + 16 * (2 * h + g));
    q.sb[h] = (int)p.qs[qrow * (D / 32) + 2 * h + g];
  }
}

// Lane (r, g) holds channels 32 ct + 8 j + 4 g + (0..3) of its query in
// accumulator elements 4 j .. 4 j + 3: one 16-byte store each of O~ / l,
// rounded once (a correctly rounded division).  RECIP: through the row's
// reciprocal when the row allows it, else element by element; the fallback
// only rewrites registers, so the stores stay unconditional.  Both routes
// give the same bits; the reciprocal pays where the epilogue is a large
// share of a query tile (a short key loop: the resident-key kernel) and
// measured no gain, or a small loss, in the streaming kernel.
template <int D, bool RECIP>
__device__ __forceinline__ void store_row(float* orow, const v16f (&acc)[D / 32], float l, int g) {
  if constexpr (!RECIP) {
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) {
      const v16f& o = acc[ct];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(orow + 32 * ct + 8 * j + 4 * g) =
            make_float4(o[4 * j] / l, o[4 * j + 1] / l, o[4 * j + 2] / l, o[4 * j + 3] / l);
    }
    return;
  }
  uint32_t lo = 0xFFFFFFFFu;
  float hi = 0.0f;
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
      lo = min(lo, min(row_divide_key(acc[ct][k]), row_divide_key(acc[ct][k + 1])));
      hi = fmaxf(hi, fmaxf(fabsf(acc[ct][k]), fabsf(acc[ct][k + 1])));
    }
  const bool by_reciprocal = row_divide_by_reciprocal(l, lo, hi);
  const float y = 1.0f / l;
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) {
    float q[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) q[k] = quotient_from_reciprocal(acc[ct][k], l, y);
    if (!by_reciprocal) {
#pragma unroll
      for (int k = 0; k < 16; ++k) q[k] = acc[ct][k] / l;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(orow + 32 * ct + 8 * j + 4 * g) =
          make_float4(q[4 * j], q[4 * j + 1], q[4 * j + 2], q[4 * j + 3]);
  }
}

// One query tile (128 queries of head bh): the whole online-softmax pass over
// its key tiles and the epilogue.
// RESIDENT: every key/value tile of the head is already in LDS, tile kt in
// stage kt (the resident-key kernel), and the Q^ operand comes in `pre`.
// NEXT (resident only): query tile qt + 1 of the head follows; its Q^ is
// loaded into `pre` as this tile starts, landing under this tile's key loop,
// and this tile's rows are all real queries, so its output stores go
// unguarded -- the next tile's wait for its Q^ then leaves them in flight.
template <int D, bool CAUSAL, int MODE, int RULE, bool FUSEDQ, bool RESIDENT = false, bool NEXT = false>
__device__ __forceinline__ void attention_qtile(const Params& p, uint8_t* lds, int64_t bh, int qt, int tid,
                                                QOperand<D>* pre = nullptr) {
  using L = Lds<D>;
  using F = FwdConsts<D, MODE, RULE>;
  constexpr int NH = D / 64;
  constexpr int NCT = D / 32;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, g = lane >> 5;

  const int nkt_all = (p.N + kBc - 1) / kBc;
  const int nkt = CAUSAL ? min(qt + 1, nkt_all) : nkt_all;
  // leading tiles in which every key is visible to every query of the tile
  const int nfull = CAUSAL ? min(qt, nkt) : p.N / kBc;

  // Q^ operand (B operand of S^T: lane = query L%32, d-chunk 2h + L/32 in
  // step h) and its scales (byte h = d-block 2h + L/32)
  const int qi = qt * kBr + 32 * wave + r;
  const int64_t qrow = bh * p.Nqp + qi;
  uint4 qop[NH];
  int qsc;
  if constexpr (RESIDENT) {
#pragma unroll
    for (int h = 0; h < NH; ++h) qop[h] = pre->op[h];
    qsc = pre->sc();
    if constexpr (NEXT) load_qoperand<D>(p, bh, qt + 1, wave, r, g, *pre);
  } else if constexpr (!FUSEDQ) {
    QOperand<D> q;
    load_qoperand<D>(p, bh, qt, wave, r, g, q);
#pragma unroll
    for (int h = 0; h < NH; ++h) qop[h] = q.op[h];
    qsc = q.sc();
  }

  // 0/1 A operand of the l product (row L%16, K chunk L/16)
  const uint32_t onew = ((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1)) ? 0x22222222u : 0u;  // E2M1 1.0
  const uint4 ones = make_uint4(onew, onew, onew, onew);
  int one_sc = 127;                 // E8M0 x1, in a register of its own
  asm volatile("" : "+v"(one_sc));  // (never rematerialized; see keep_live)
  int held[4] = {0, 0, 0, 0};       // scale registers of the latest PV products
  // K^ operand offset of sub-tile 0, step h; sub-tile t adds a constant,
  // (d/2)(64(t/2) + 16(t%2)) bytes: its key bits 4 and 6 leave the swizzle
  // term unchanged
  int koff[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) koff[h] = L::KC + 16 * kc_granule<D>(tile_key(0, r), 2 * h + g);

  RowState rs;
  rs.m = -INFINITY;
  rs.mc = 0.0f;
  rs.mcL = 0.0f;
  rs.off = 0.0f;
  rs.l = 0.0f;
  rs.cnt = 0.0f;
  rs.sig = 0.0f;
  rs.rho = 0.0f;
  if constexpr (F::kFixedM) {
    const float4 st = *reinterpret_cast<const float4*>(p.stats + qrow * 4);
    rs.m = st.x;
    rs.off = __builtin_amdgcn_logf(st.y);  // log2 of l*
    rs.mc = st.x * F::kC + rs.off;
    rs.rho = st.z;
  }
  float dg[6] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  v16f acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
    acc[ct] = v16f{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  v4f accl = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  PendingPV<D> pend;  // nothing deferred yet: zero codes add nothing
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) pend.vop[ct] = make_uint4(0u, 0u, 0u, 0u);
  pend.pq = make_uint4(0u, 0u, 0u, 0u);
  pend.vsc = 0x7F7F7F7F;
  pend.psc = 127;

  const DmaPlan<D> plan(tid);
  if constexpr (RESIDENT) {
    // the key/value tiles are resident: no copies, no barriers
  } else if constexpr (FUSEDQ) {
    // Q rows are loaded under the first tile's DMA, quantized into the second
    // LDS stage (free until the loop's first copy), and read back in operand
    // order; a second barrier frees that stage again
    uint4 raw[D / 64][4];
    q_prologue_load<D>(p, bh, qt * kBr + 32 * wave, lane, raw);
    codes_dma<D>(p, plan, bh, 0, lds, tid);
    scale_store<D>(scale_load<D>(p, bh, 0, tid), lds, tid);
    uint8_t* qlds = lds + L::STAGE + L::KC + 32 * wave * (D / 2);  // this wave's 32 rows
    uint8_t* qslds = lds + L::STAGE + L::KS + 32 * wave * (D / 32);
    q_prologue_quantize<D>(p, lane, raw, qlds, qslds);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint8_t* qr = qlds + r * (D / 2);
    const uint8_t* qsr = qslds + r * (D / 32);
#pragma unroll
    for (int h = 0; h < NH; ++h) qop[h] = *reinterpret_cast<const uint4*>(qr + 16 * (2 * h + g));
    if constexpr (D == 128) qsc = (int)qsr[g] | ((int)qsr[2 + g] << 8);
    else qsc = (int)qsr[g];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  } else {
    codes_dma<D>(p, plan, bh, 0, lds, tid);
    scale_store<D>(scale_load<D>(p, bh, 0, tid), lds, tid);
    __builtin_amdgcn_s_waitcnt(0);  // the DMA has landed in LDS
    __syncthreads();
  }

  // full tiles: no per-element masking; the next tile is copied into the
  // other buffer while this one is processed (on the last iteration the
  // clamped index copies this tile again into a buffer nothing reads later)
  for (int kt = 0; kt < nfull; ++kt) {
    if constexpr (RESIDENT) {
      tile_step<D, CAUSAL, MODE, RULE, false>(lds + kt * L::STAGE, kt, p.N, qop, qsc, qi, ones, one_sc, rs, acc,
                                              accl, held, lane, koff, dg, p.gamma_f, p.inv_gamma_f, pend);
    } else {
      const uint8_t* buf = lds + (kt & 1) * L::STAGE;
      uint8_t* nxt = lds + ((kt + 1) & 1) * L::STAGE;
      const int kn = min(kt + 1, nkt - 1);
      codes_dma<D>(p, plan, bh, kn, nxt, tid);
      const ScaleRegs sr = scale_load<D>(p, bh, kn, tid);
      tile_step<D, CAUSAL, MODE, RULE, false>(buf, kt, p.N, qop, qsc, qi, ones, one_sc, rs, acc, accl, held, lane,
                                              koff, dg, p.gamma_f, p.inv_gamma_f, pend);
      scale_store<D>(sr, nxt, tid);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
  // at most one masked tile: the ragged end of the keys or the causal diagonal
  if (nfull < nkt) {
    int nkeys = p.N;
    // (resident keys: the same masks for every query tile of a run, which
    // would otherwise be hoisted out of the run's loop into scalar registers)
    if constexpr (RESIDENT) asm volatile("" : "+s"(nkeys));
    tile_step<D, CAUSAL, MODE, RULE, true>(lds + (RESIDENT ? nfull : (nfull & 1)) * L::STAGE, nfull, nkeys, qop, qsc,
                                           qi, ones, one_sc, rs, acc, accl, held, lane, koff, dg, p.gamma_f,
                                           p.inv_gamma_f, pend);
    // No later tile's maximum covers the scales of this tile's products: a
    // read of every accumulator (which waits for all products so far) does,
    // inside this block, before the register moves that lead into the
    // deferred second half below can reuse them.
    if constexpr (kDeferPV<D, CAUSAL> && MODE != kModeStats && MODE != kModeDiag) {
      float all = accl[0];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) all += acc[ct][0];
      keep_live(all, held[0], held[1], held[2], held[3]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (kDeferPV<D, CAUSAL> && MODE != kModeStats && MODE != kModeDiag) {
    issue_pending<D>(pend, acc, accl, ones, one_sc);  // the last tile's second half
    held[0] = pend.vsc;
    held[1] = pend.psc;
  }

  // ---- epilogue
  if constexpr (MODE == kModeStats) {
    // (m*, l* = cnt + sig, rho = l* - 1, unused): per row 16 bytes
    if (g == 0)
      *reinterpret_cast<float4*>(p.stats + qrow * 4) = make_float4(rs.m, rs.cnt + rs.sig, (rs.cnt - 1.0f) + rs.sig, 0.0f);
    return;
  }
  if constexpr (MODE == kModeDiag) {
#pragma unroll
    for (int k = 0; k < 6; ++k) dg[k] = pair_sum(dg[k]);
    if (g == 0 && qi < p.Nq) {
      float* dr = p.diag + (bh * p.Nq + qi) * 6;
      dr[0] = dg[0];
      dr[1] = dg[1];
      dr[2] = dg[2];
      dr[3] = dg[3];
      dr[4] = dg[4];
      dr[5] = -0x1.62e430p-1f * dg[5];  // -ln 2 * sum P log2 P
    }
    return;
  }
  const float lsum = accl[0];  // sum of beta-weighted P^ (the 0/1 product)
  {
    float done = lsum;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) done += acc[ct][0];
    keep_live(done, held[0], held[1], held[2], held[3]);
    keep_live(done, one_sc);
  }
  // O = O~ / l with a correctly rounded division (Eq. 8): with V^ constant
  // per channel, O~ = v^ l exactly, and the division returns v^ exactly
  float l;
  if constexpr (MODE == kModePnq) l = lsum;
  else if constexpr (MODE == kModeDirect) l = rs.l;
  else l = 1.0f;
  // (Staging the tile through LDS into whole 128-byte row segments measured
  // no faster on the Wan-like shape and 4-5 % slower on the causal and
  // cross-attention shapes, whose short key loops make the epilogue a larger
  // share.)
  float* orow = p.out + (bh * p.Nq + qi) * D;
  if constexpr (RESIDENT && NEXT) store_row<D, true>(orow, acc, l, g);  // qt + 1 < nqt: every row is a query
  else if (qi < p.Nq) store_row<D, RESIDENT>(orow, acc, l, g);
  if (g == 0 && qi < p.Nq) {
    if (p.row_stats) {
      p.row_stats[(bh * p.Nq + qi) * 2 + 0] = rs.m * F::kInvSqrtD;
      p.row_stats[(bh * p.Nq + qi) * 2 + 1] = l;
    }
    if (p.row_sums) p.row_sums[bh * p.Nq + qi] = (MODE == kModePostnorm) ? lsum : lsum / l;
  }
}

// Workgroup -> (head, query tiles).  Consecutive logical indexes land on the
// same XCD (the hardware deals workgroups round-robin over the 8 XCDs), so
// the query tiles of one head share that XCD's L2 copy of its K^ and V^.
// Under the causal mask query tile t visits t + 1 key tiles; a workgroup
// takes the pair (nqt - 1 - i, i), nqt + 1 key tiles in all, so every
// workgroup has the same work (the middle tile of an odd count runs alone).
// Two workgroups (two waves per SIMD) per CU.
template <int D, bool CAUSAL, int MODE, int RULE, bool FUSEDQ>
__global__ __launch_bounds__(256, 2) void k_attention(Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes<D>];
  const int tid = threadIdx.x;
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3, qx = G >> 3, rx = G & 7;
  const int logical = (xcd < rx) ? xcd * (qx + 1) + idx : rx * (qx + 1) + (xcd - rx) * qx + idx;
  if constexpr (CAUSAL) {
    const int npair = (p.nqt + 1) / 2;
    const int64_t bh = logical / npair;
    const int i = logical % npair;
    attention_qtile<D, CAUSAL, MODE, RULE, FUSEDQ>(p, lds, bh, p.nqt - 1 - i, tid);
    if (i != p.nqt - 1 - i) {
      __syncthreads();  // every wave is done with the LDS stages
      attention_qtile<D, CAUSAL, MODE, RULE, FUSEDQ>(p, lds, bh, i, tid);
    }
  } else {
    attention_qtile<D, CAUSAL, MODE, RULE, FUSEDQ>(p, lds, logical / p.nqt, logical % p.nqt, tid);
  }
}

// Resident-key forward for short key/value sequences (every tile of a head
// fits in LDS: cross-attention against a few hundred text tokens).  The
// B H nqt query tiles, in (head, tile) order, are dealt out in runs of
// `per_group`, one run per workgroup, so that every workgroup has the same
// work.  For each head its run touches, a workgroup copies the head's K^, V^
// tiles into LDS once and then runs that head's query tiles against them
// with no further copies or barriers.  Each query tile runs exactly the code
// of the streaming kernel (same tiles, same order), so every output row is
// the same bit for bit; the next query tile's Q^ is loaded as the current
// one starts, and the current one's output stores overlap the next tile's
// work.
template <int D, int MODE, int RULE>
__global__ __launch_bounds__(256, 2) void k_attention_resident(Params p, int64_t total, int per_group) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kResidentTiles<D> * Lds<D>::STAGE];
  const int tid = threadIdx.x;
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3, qx = G >> 3, rx = G & 7;
  const int logical = (xcd < rx) ? xcd * (qx + 1) + idx : rx * (qx + 1) + (xcd - rx) * qx + idx;
  const int64_t g0 = (int64_t)logical * per_group, g1 = min(g0 + per_group, total);
  const int nkt = (p.N + kBc - 1) / kBc;  // <= kResidentTiles<D> (checked by the launcher)
  const int wave = tid >> 6, lane = tid & 63;
  const DmaPlan<D> plan(tid);
  QOperand<D> q;
  for (int64_t gi = g0; gi < g1;) {  // uniform over the workgroup
    const int64_t bh = gi / p.nqt;
    const int qt0 = (int)(gi - bh * p.nqt);
    const int qt1 = (int)min<int64_t>(p.nqt, qt0 + (g1 - gi));
    if (gi != g0) __syncthreads();  // every wave is done with the previous head's tiles
    // every copy and scale load in flight before the first scale store waits
    ScaleRegs sr[kResidentTiles<D>];
#pragma unroll
    for (int kt = 0; kt < kResidentTiles<D>; ++kt)
      if (kt < nkt) {
        codes_dma<D>(p, plan, bh, kt, lds + kt * Lds<D>::STAGE, tid);
        sr[kt] = scale_load<D>(p, bh, kt, tid);
      }
#pragma unroll
    for (int kt = 0; kt < kResidentTiles<D>; ++kt)
      if (kt < nkt) scale_store<D>(sr[kt], lds + kt * Lds<D>::STAGE, tid);
    load_qoperand<D>(p, bh, qt0, wave, lane & 31, lane >> 5, q);
    __builtin_amdgcn_s_waitcnt(0);  // the head's tiles have landed in LDS
    __syncthreads();
    // each query tile derives its per-lane addresses afresh (t), as in the
    // streaming kernel, rather than holding them in registers across tiles;
    // the run's last tile has no successor and is peeled off
    for (int qt = qt0; qt + 1 < qt1; ++qt) {
      int t = tid;
      asm volatile("" : "+v"(t));
      attention_qtile<D, false, MODE, RULE, false, true, true>(p, lds, bh, qt, t, &q);
    }
    {
      int t = tid;
      asm volatile("" : "+v"(t));
      attention_qtile<D, false, MODE, RULE, false, true, false>(p, lds, bh, qt1 - 1, t, &q);
    }
    gi += qt1 - qt0;
  }
}

// Compute units of the current device, looked up once per device.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) v = 256;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Resident-key launch: the query tiles dealt evenly over at most one
// workgroup per slot (two per CU).
template <int D, int MODE, int RULE>
hipError_t launch_resident(const Params& prm, int BH, hipStream_t stream) {
  const int64_t slots = 2 * (int64_t)device_cus();
  const int64_t total = (int64_t)BH * prm.nqt;
  const int64_t per_group = (total + slots - 1) / slots;
  const int64_t groups = (total + per_group - 1) / per_group;
  if (per_group > 0x7FFFFFFF || groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_attention_resident<D, MODE, RULE>), dim3((unsigned)groups), dim3(256), 0, stream, prm, total,
                     (int)per_group);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int MODE, int RULE, bool FUSEDQ = false>
hipError_t launch_one(const Params& prm, int BH, hipStream_t stream) {
  const int64_t groups = (int64_t)BH * (CAUSAL ? (prm.nqt + 1) / 2 : prm.nqt);
  hipLaunchKernelGGL((k_attention<D, CAUSAL, MODE, RULE, FUSEDQ>), dim3((unsigned)groups), dim3(256), 0, stream,
                     prm);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dispatch_mode(const AttnArgs& a, const Params& prm, hipStream_t s) {
  const int BH = a.B * a.H;
  if (a.qx) return launch_one<D, CAUSAL, kModePnq, kRuleUos, true>(prm, BH, s);  // fused Q prologue
  if constexpr (!CAUSAL) {
    // every key/value tile of a head fits in LDS: the resident-key kernel
    if (a.resident_ok && a.mode == kModePnq && a.rule == kRuleUos && (prm.N + kBc - 1) / kBc <= kResidentTiles<D>)
      return launch_resident<D, kModePnq, kRuleUos>(prm, BH, s);
  }
  if (a.mode == kModePnq && a.rule == kRuleUos) return launch_one<D, CAUSAL, kModePnq, kRuleUos>(prm, BH, s);
  if (a.mode == kModePnq) return launch_one<D, CAUSAL, kModePnq, kRuleOcp>(prm, BH, s);
  if (a.mode == kModeDirect)
    return a.rule == kRuleUos ? launch_one<D, CAUSAL, kModeDirect, kRuleUos>(prm, BH, s)
                              : launch_one<D, CAUSAL, kModeDirect, kRuleOcp>(prm, BH, s);
  // POSTNORM, DIAG: exact row statistics first, then the quantized pass
  hipError_t err = launch_one<D, CAUSAL, kModeStats, kRuleUos>(prm, BH, s);
  if (err != hipSuccess) return err;
  if (a.mode == kModeDiag)
    return a.rule == kRuleUos ? launch_one<D, CAUSAL, kModeDiag, kRuleUos>(prm, BH, s)
                              : launch_one<D, CAUSAL, kModeDiag, kRuleOcp>(prm, BH, s);
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
  prm.diag = a.diag;
  {
    // gamma = 2^k gamma_f with gamma_f in [1, 2); 1/gamma_f rounds once
    int k = 0;
    const float gf = a.mode == kModeDiag ? 2.0f * frexpf(a.gamma, &k) : 1.0f;
    prm.gamma_f = gf;
    prm.inv_gamma_f = 1.0f / gf;
  }
  prm.qx = static_cast<const uint16_t*>(a.qx);
  prm.qsB = a.qsB; prm.qsH = a.qsH; prm.qsN = a.qsN;
  prm.qdtype = a.qdtype;
  prm.qrotate = a.qrotate;
  prm.qrule = a.qrule;
  prm.H = a.H;
  prm.N = a.Nk;
  prm.Np = (int)padded_tokens(a.Nk);
  prm.Nq = a.N;
  prm.Nqp = (int)padded_tokens(a.N);
  prm.nqt = prm.Nqp / kBr;
  if (a.d == 128) return a.causal ? dispatch_mode<128, true>(a, prm, stream) : dispatch_mode<128, false>(a, prm, stream);
  return a.causal ? dispatch_mode<64, true>(a, prm, stream) : dispatch_mode<64, false>(a, prm, stream);
}

}  // namespace mxattn_internal
