// MXFP4 quantizers of MXAttention for gfx950 (MI355X).
//
//   k_quantize_headdim: Q and K.  Optional Hadamard rotation along the head
//     dimension (MXAttention paper, Sec. 4.3, Alg. 2), then UOS or
//     OCP block quantization of every 32 consecutive channels (Alg. 1;
//     Alg. 2).
//   k_quantize_tokens: V.  Block quantization along tokens, 32 consecutive
//     tokens of one channel per block (Alg. 2, with the block axis that
//     the PV product contracts over, as the MatX leaky-quantization page
//     explains).
//   k_quantize_qkv: the two above for Q, K and V of one attention call in a
//     single launch.
//   k_sweep_headdim / k_sweep_tokens + k_sweep_reduce: the per-head squared
//     quantization error of the same blocks for a list of ceiling-rule
//     boundaries q (the Q_max sweep of Sec. 5.5.1, Table 4; Eq. 13).
//
// The two quantizers are HBM-bandwidth bound: 2 bytes read and 0.5 + 1/32
// bytes written per element.  The sweep reads 2 bytes per element and does
// two block quantizations plus one selection per boundary per block.
//
// Numerics follow the bit-exact contract of include/mxattn.h:
//   rotation: binary32 butterflies with strides 1, 2, ..., d/2, then one
//             multiply by fl32(1/sqrt(d));
//   scale:    UOS e = ceil(log2(M / 7.25)), OCP e = floor(log2 M) - 2, or the
//             ceiling rule e = ceil(log2(M / q)) for a boundary q in [2, 64],
//             read off the binary32 bit patterns of M (and of q rounded down
//             to binary32); clamped to [-127, 127];
//   elements: round to nearest E2M1 value, ties to the even code, saturating
//             at 6, sign bit kept for values that round to zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"
#include "mx_block.h"
#include "mxattn.h"
#include "quant_index.h"

// Partial sums of mxattn_scale_sweep_noalloc: one array per GPU, created with
// the library's code object on that device and kept until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: host
// code reaches the array only through the address hipGetSymbolAddress returns
// for the current device (sweep_scratch_ptr below).
static __device__ __align__(256) double scratch[MXATTN_SWEEP_SCRATCH_BYTES / sizeof(double)];

namespace mxattn_internal {
namespace {

using namespace mxblock;

// 16-byte store with the non-temporal hint.  The head-dim quantizer writes its
// code bytes this way (nothing in the kernel reads them back).  Measured on
// the MI355X: that launch alone runs about 4 % faster, and the Q, K, V
// quantizer launches of one step about 1.5 % faster in total.  The token-axis
// quantizer measured slightly slower with the hint and keeps plain stores.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(uint4* dst, uint4 a) {
  const u32x4 v = {a.x, a.y, a.z, a.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
}

constexpr int kHdUnitsPerThread = 1;  // row-blocks per thread of the head-dim quantizer

// One tensor of a quantizer launch: 16-bit input [B, H, N, d] with element
// strides, and its MXFP4 codes and scales.  `total` counts the work units:
// row-blocks (B H Np d/32) along d, 32-token blocks (B H Np/32) along tokens.
struct QTensor {
  const uint16_t* x;
  int H, N, Np;
  int64_t sB, sH, sN;
  int64_t total;
  uint8_t* codes;
  uint8_t* scales;
};

// Head-dimension quantizer, workgroup `group` of tensor t.  One lane owns one
// 32-channel block of one row (d/32 lanes per row, in the same quad), so the
// first five butterfly stages stay in registers and the remaining one (d=64)
// or two (d=128) cross lanes through DPP.  Each thread handles one row-block
// (64 bytes in four 16-byte loads); measured on the Wan-like tensors this
// beats two or four blocks per thread (more workgroups in flight rather than
// more loads per lane).
template <int D, int DTYPE, bool ROTATE, int RULE>
__device__ __forceinline__ void headdim_group(const QTensor& t, uint32_t qb, int64_t group) {
  constexpr int BPR = D / 32;  // blocks (lanes) per row
  static_assert(D == 64 || D == 128, "head dim");

  constexpr int QU = kHdUnitsPerThread;
  uint4 raw[QU][4];
  int64_t unit[QU];
#pragma unroll
  for (int it = 0; it < QU; ++it) {
    unit[it] = group * 256 * QU + it * 256 + threadIdx.x;
    const HeaddimUnit w = headdim_unit(unit[it], t.Np, BPR);
    const int64_t off = headdim_load_offset(w, t.total, unit[it], t.H, t.N, t.sB, t.sH, t.sN);
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[it][k] = make_uint4(0, 0, 0, 0);
    if (off >= 0) {  // a padding row (n >= N) loads nothing
      const uint4* p = reinterpret_cast<const uint4*>(t.x + off);
#pragma unroll
      for (int k = 0; k < 4; ++k) raw[it][k] = p[k];
    }
  }

#pragma unroll
  for (int it = 0; it < QU; ++it) {
    const int blk = (int)(unit[it] % BPR);
    float v[32];
    unpack_block<DTYPE>(raw[it], v);
    if constexpr (ROTATE) rotate_block<D>(v, blk);
    const float M = finish_block<D, ROTATE>(v);
    const int e = scale_exponent<RULE>(M, qb);
    // the exact division by 2^e happens inside the convert
    const uint4 packed = block_codes(v, e);
    if (unit[it] < t.total) {
      store_nt16(reinterpret_cast<uint4*>(t.codes) + unit[it], packed);
      t.scales[unit[it]] = (uint8_t)(e + 127);
    }
  }
}

// Token-axis quantizer, workgroup `group` of tensor t.  One lane owns two
// adjacent channels of one 32-token block: it reads the 32 tokens of its
// channel pair (each wave-wide load is one contiguous row of the block), so
// both block maxima are lane-local, and writes 2 x 16 code bytes and 2 scale
// bytes contiguously.
template <int D, int DTYPE, int RULE>
__device__ __forceinline__ void tokens_group(const QTensor& t, uint32_t qb, int64_t group) {
  constexpr int LPB = D / 2;  // lanes per token block
  const int64_t gl = group * 256 + threadIdx.x;
  const int64_t gblk = gl / LPB;
  const int cp = (int)(gl % LPB);
  if (gblk >= t.total) return;
  const int NBp = t.Np / 32;
  const int64_t bh = gblk / NBp;
  const int kb = (int)(gblk % NBp);
  const int N = t.N;
  const int64_t sN = t.sN;
  const uint16_t* lane_base = t.x + tokens_lane_base(bh, cp, t.H, t.sB, t.sH);

  // all 32 loads are issued before any is used; only a block that crosses or
  // lies past N (the last one or few of a head) takes the guarded path,
  // decided once per wave.  The guarded path reads each token clamped into
  // [0, N) (a block wholly in the padding reads token N - 1) and discards the
  // values past N, so no load leaves the tensor.
  uint32_t w[32];
  if (__all(tokens_block_inside(kb, N))) {
    const uint16_t* pt = lane_base + (int64_t)(32 * kb) * sN;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      w[k] = *reinterpret_cast<const uint32_t*>(pt);
      pt += sN;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t wt =
          *reinterpret_cast<const uint32_t*>(lane_base + (int64_t)tokens_guarded_token(kb, k, N) * sN);
      w[k] = (32 * kb + k < N) ? wt : 0u;
    }
  }
  // block maxima of |x| on the 16-bit patterns: for finite bf16 and fp16
  // values the magnitude order is the unsigned order of the low 15 bits, so
  // the maxima need no unpacking (the values are unpacked only for the
  // codes, which keeps fewer registers live)
  uint32_t a0 = 0u, a1 = 0u;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    a0 = max(a0, w[k] & 0x7FFFu);
    a1 = max(a1, (w[k] >> 16) & 0x7FFFu);
  }
  float m0, m1;
  unpack2<DTYPE>(a0 | (a1 << 16), m0, m1);
  const int e0 = scale_exponent<RULE>(m0, qb), e1 = scale_exponent<RULE>(m1, qb);
  // codes eight tokens at a time, as block_codes() forms them: the convert
  // divides by 2^e; at the clamp e = -127 the values are first moved up
  // exactly by 2^127 and converted with unit scale
  const bool tiny = (e0 < -126) | (e1 < -126);
  const int k0 = e0 < -126 ? 127 : 0, k1 = e1 < -126 ? 127 : 0;
  const float s0 = pow2f(e0 < -126 ? 0 : e0), s1 = pow2f(e1 < -126 ? 0 : e1);
  uint32_t c0[4], c1[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) unpack2<DTYPE>(w[8 * c + i], lo[i], hi[i]);
    if (tiny) {
      // ldexp by 0 leaves the other channel's values unchanged (binary32
      // subnormals are kept: these kernels run with denormals enabled)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = __builtin_amdgcn_ldexpf(lo[i], k0);
        hi[i] = __builtin_amdgcn_ldexpf(hi[i], k1);
      }
    }
    c0[c] = cvt8(lo, s0);
    c1[c] = cvt8(hi, s1);
  }
  uint4* dst = reinterpret_cast<uint4*>(t.codes + (gblk * D + 2 * cp) * 16);
  dst[0] = make_uint4(c0[0], c0[1], c0[2], c0[3]);
  dst[1] = make_uint4(c1[0], c1[1], c1[2], c1[3]);
  *reinterpret_cast<uint16_t*>(t.scales + gblk * D + 2 * cp) =
      (uint16_t)((uint32_t)(e0 + 127) | ((uint32_t)(e1 + 127) << 8));
}

template <int D, int DTYPE, bool ROTATE, int RULE>
__global__ __launch_bounds__(256) void k_quantize_headdim(QTensor t, uint32_t qb) {
  headdim_group<D, DTYPE, ROTATE, RULE>(t, qb, blockIdx.x);
}

template <int D, int DTYPE, int RULE>
__global__ __launch_bounds__(256) void k_quantize_tokens(QTensor t, uint32_t qb) {
  tokens_group<D, DTYPE, RULE>(t, qb, blockIdx.x);
}

// Q, K and V of one attention call in one launch: workgroups [0, gq) quantize
// Q and [gq, gq + gk) K along d (rotated if ROTATE), the rest V along tokens.
// One launch instead of three saves two kernel boundaries, where the GPU
// drains one grid before the next one fills it.  With both code paths in one
// function the compiler allocated 105 VGPRs (four waves per SIMD) although
// neither path needs more than the token path's 71 on its own; the bound of
// seven waves per SIMD (at most 72 VGPRs, no spills; eight would spill)
// restores the standalone kernels' memory parallelism.  Measured on the
// MI355X, interleaved, identical codes: Wan-like 230 vs 241 us, Hunyuan-like
// 491 vs 504 us.
template <int D, int DTYPE, bool ROTATE, int RULE>
__global__ __launch_bounds__(256, 7) void k_quantize_qkv(QTensor q, QTensor k, QTensor v, int64_t gq, int64_t gk,
                                                      uint32_t qb) {
  const int64_t g = blockIdx.x;
  if (g < gq) headdim_group<D, DTYPE, ROTATE, RULE>(q, qb, g);
  else if (g < gq + gk) headdim_group<D, DTYPE, ROTATE, RULE>(k, qb, g - gq);
  else tokens_group<D, DTYPE, RULE>(v, qb, g - gq - gk);
}

// ---------------------------------------------------------------------------
// Q_max sweep (Sec. 5.5.1, Table 4): per head and per boundary q_j, the sum of
// squared errors of the ceiling rule e = ceil(log2(M / q_j)) (Eq. 13) over the
// blocks the quantizers above see.  With max q <= 2 min q every block has at
// most two candidate exponents, e(q_min) and one less, so each block is
// quantized twice and every boundary only selects one of the two errors.

// Work units (blocks, or channel pairs of a token block) per lane: enough
// that the per-boundary workgroup reduction is a small share of the work.
constexpr int kSweepUnits = 16;

struct SweepQ {
  uint32_t qb[kSweepMax];  // binary32 bits of each boundary, rounded down
  uint32_t qmin;           // the smallest of them
  int nq;
};

// the two E2M1 values in byte BYTE of w (elements 2 BYTE and 2 BYTE + 1)
template <int BYTE>
__device__ __forceinline__ void decode2(uint32_t w, float& lo, float& hi) {
  const auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, BYTE);
  lo = p[0];
  hi = p[1];
}

__device__ __forceinline__ double pow2d(int k) { return __longlong_as_double((long long)(1023 + k) << 52); }

// Eight E2M1 codes of v[8k .. 8k+7] at exponent e, exactly as block_codes
// forms them (at the clamp e = -127 the values move up by 2^127 before a
// unit-scale convert).
__device__ __forceinline__ uint32_t codes8_at(const float (&v)[32], int k, int e) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = e < -126 ? __builtin_amdgcn_ldexpf(v[8 * k + i], 127) : v[8 * k + i];
  return cvt8(y, pow2f(e < -126 ? 0 : e));
}

// Squared quantization errors of one block at its two candidate exponents,
// s = 4^e sum_i (v_i 2^-e - c_i)^2, where c_i are the E2M1 values of the
// block's codes at exponent e.  The residual r_i = v_i 2^-e - c_i is formed
// by one binary32 fused multiply-add, exactly: v_i 2^-e is a power-of-two
// scaling of v_i, and r_i has at most 24 significant bits (its lowest bit is
// that of v_i 2^-e, its highest at most that of max(v_i 2^-e, 6)).  The one
// exception is v_i 2^-e below 2^-126 (then c_i = 0), where the subnormal
// result is off by at most 2^-150, 2^-250 of the block's own terms.  r_i^2
// (at most 48 bits) is exact in binary64, so only the sums round: one
// binary64 fused multiply-add per element and exponent.  The elements go
// eight at a time (one convert word each), and each sum is kept as four
// interleaved partial sums, added pairwise at the end, so that its dependent
// binary64 adds form four chains of eight instead of one of 32.  CLAMP: some
// block of the wave sits at e = -127, whose codes need the lifted convert.
template <bool CLAMP>
__device__ __forceinline__ void block_sse_pair(const float (&v)[32], int e_hi, int e_lo, double& s_hi,
                                               double& s_lo) {
  double ph[4] = {0.0, 0.0, 0.0, 0.0}, pl[4] = {0.0, 0.0, 0.0, 0.0};
  const float inv_hi = pow2f(-e_hi), inv_lo = pow2f(-e_lo);  // e in [-127, 126]: normal
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t wh = CLAMP ? codes8_at(v, k, e_hi) : cvt8(&v[8 * k], pow2f(e_hi));
    const uint32_t wl = CLAMP ? codes8_at(v, k, e_lo) : cvt8(&v[8 * k], pow2f(e_lo));
    float gh[8], gl[8];  // E2M1 values of the codes (unit scale: exact)
    decode2<0>(wh, gh[0], gh[1]);
    decode2<1>(wh, gh[2], gh[3]);
    decode2<2>(wh, gh[4], gh[5]);
    decode2<3>(wh, gh[6], gh[7]);
    decode2<0>(wl, gl[0], gl[1]);
    decode2<1>(wl, gl[2], gl[3]);
    decode2<2>(wl, gl[4], gl[5]);
    decode2<3>(wl, gl[6], gl[7]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double rh = (double)__fmaf_rn(v[8 * k + i], inv_hi, -gh[i]);
      const double rl = (double)__fmaf_rn(v[8 * k + i], inv_lo, -gl[i]);
      ph[i & 3] = __fma_rn(rh, rh, ph[i & 3]);
      pl[i & 3] = __fma_rn(rl, rl, pl[i & 3]);
    }
  }
  s_hi = __dmul_rn(__dadd_rn(__dadd_rn(ph[0], ph[1]), __dadd_rn(ph[2], ph[3])), pow2d(2 * e_hi));
  s_lo = __dmul_rn(__dadd_rn(__dadd_rn(pl[0], pl[1]), __dadd_rn(pl[2], pl[3])), pow2d(2 * e_lo));
}

__device__ __forceinline__ void accumulate_block(const float (&v)[32], float M, const SweepQ& sq,
                                                 double (&acc)[kSweepMax]) {
  const int e_hi = scale_exponent<kRuleCeilQ>(M, sq.qmin);
  const int e_lo = e_hi > -127 ? e_hi - 1 : e_hi;
  double s_hi, s_lo;
  if (__any(e_lo < -126)) block_sse_pair<true>(v, e_hi, e_lo, s_hi, s_lo);  // rare: tiny or zero blocks
  else block_sse_pair<false>(v, e_hi, e_lo, s_hi, s_lo);
  // Boundary q_j takes e_hi unless ceil(log2(M / q_j)) <= e_hi - 1, i.e.
  // unless M <= q_j 2^(e_hi - 1) (q_j <= 2 q_min leaves only those two).  With
  // m = M 2^(1 - e_hi), exact in binary32 (m lies in (q_min, 2 q_min] when e_hi
  // is not clamped; at the clamp e_lo = e_hi and a zero block has s_hi = s_lo
  // = 0), that is m > q_j: the decision scale_exponent takes, with one
  // compare.  Accumulators past nq collect unused sums and are never stored.
  const float m = __builtin_amdgcn_ldexpf(M, 1 - e_hi);
#pragma unroll
  for (int j = 0; j < kSweepMax; ++j) acc[j] = __dadd_rn(acc[j], m > __uint_as_float(sq.qb[j]) ? s_hi : s_lo);
}

// Workgroup sums of acc[j] in a fixed order, through LDS in rounds of eight
// boundaries: the 256 threads park acc[8r .. 8r+7]; thread t then adds the
// eight values of boundary 8r + t/32 from threads 8(t%32) .. 8(t%32)+7 in
// order, and 64 threads and then 8 add those partials in order (thread index
// order throughout): bit-identical on every run.
__device__ __forceinline__ void store_partial(double (&acc)[kSweepMax], int nq, double* __restrict__ out) {
  __shared__ double park[256][9];  // [thread][boundary of the round], padded against bank conflicts
  __shared__ double lvl1[8][32];
  __shared__ double lvl2[8][4];
  const int t = threadIdx.x;
#pragma unroll
  for (int r = 0; r < kSweepMax / 8; ++r) {
    if (8 * r < nq) {  // uniform
#pragma unroll
      for (int k = 0; k < 8; ++k) park[t][k] = acc[8 * r + k];
      __syncthreads();
      {
        const int jb = t >> 5, seg = t & 31;
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = __dadd_rn(s, park[8 * seg + i][jb]);
        lvl1[jb][seg] = s;
      }
      __syncthreads();
      if (t < 32) {
        const int jb = t >> 2, q4 = t & 3;
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = __dadd_rn(s, lvl1[jb][8 * q4 + i]);
        lvl2[jb][q4] = s;
      }
      __syncthreads();
      if (t < 8 && 8 * r + t < nq)
        out[8 * r + t] = __dadd_rn(__dadd_rn(lvl2[t][0], lvl2[t][1]), __dadd_rn(lvl2[t][2], lvl2[t][3]));
    }
  }
}

// Head-dimension blocks, lanes mapped as in k_quantize_headdim (a row's d/32
// blocks in one quad, so the rotation's DPP steps pair the right lanes).
// Workgroup g covers blocks [1024 c, 1024 c + 1024) of head g / chunks,
// c = g % chunks; blocks past the head's N rows are zeros and add nothing.
template <int D, int DTYPE, bool ROTATE>
__global__ __launch_bounds__(256) void k_sweep_headdim(const uint16_t* __restrict__ x, int H, int N, int64_t sB,
                                                       int64_t sH, int64_t sN, int chunks, SweepQ sq,
                                                       double* __restrict__ partial) {
  constexpr int BPR = D / 32;
  const int64_t bh = blockIdx.x / chunks;
  const int chunk = (int)(blockIdx.x % chunks);
  const int64_t b = bh / H, h = bh % H;
  const int64_t units = (int64_t)N * BPR;
  const uint16_t* xh = x + b * sB + h * sH;
  double acc[kSweepMax];
#pragma unroll
  for (int j = 0; j < kSweepMax; ++j) acc[j] = 0.0;
  for (int i = 0; i < kSweepUnits; ++i) {
    const int64_t u = (int64_t)chunk * (256 * kSweepUnits) + i * 256 + threadIdx.x;
    const int blk = (int)(u % BPR);
    uint4 raw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[k] = make_uint4(0, 0, 0, 0);
    if (u < units) {
      const uint4* p = reinterpret_cast<const uint4*>(xh + (u / BPR) * sN + 32 * blk);
#pragma unroll
      for (int k = 0; k < 4; ++k) raw[k] = p[k];
    }
    float v[32];
    unpack_block<DTYPE>(raw, v);
    if constexpr (ROTATE) rotate_block<D>(v, blk);
    const float M = finish_block<D, ROTATE>(v);
    accumulate_block(v, M, sq, acc);
  }
  store_partial(acc, sq.nq, partial + blockIdx.x * (int64_t)sq.nq);
}

// Token blocks: a lane owns two adjacent channels of one 32-token block, as in
// k_quantize_tokens; tokens past N are +0.
template <int D, int DTYPE>
__global__ __launch_bounds__(256) void k_sweep_tokens(const uint16_t* __restrict__ x, int H, int N, int64_t sB,
                                                      int64_t sH, int64_t sN, int chunks, SweepQ sq,
                                                      double* __restrict__ partial) {
  constexpr int LPB = D / 2;
  const int64_t bh = blockIdx.x / chunks;
  const int chunk = (int)(blockIdx.x % chunks);
  const int64_t b = bh / H, h = bh % H;
  const int NB = (N + 31) / 32;
  const int64_t units = (int64_t)NB * LPB;
  double acc[kSweepMax];
#pragma unroll
  for (int j = 0; j < kSweepMax; ++j) acc[j] = 0.0;
  for (int i = 0; i < kSweepUnits; ++i) {
    const int64_t u = (int64_t)chunk * (256 * kSweepUnits) + i * 256 + threadIdx.x;
    float v0[32], v1[32];
    const int kb = (int)(u / LPB), cp = (int)(u % LPB);
    const uint16_t* base = x + b * sB + h * sH + (int64_t)(32 * kb) * sN + 2 * cp;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const uint32_t w = (u < units && 32 * kb + t < N) ? *reinterpret_cast<const uint32_t*>(base + t * sN) : 0u;
      unpack2<DTYPE>(w, v0[t], v1[t]);
    }
    float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      m0 = fmaxf(m0, fabsf(v0[t]));
      m1 = fmaxf(m1, fabsf(v1[t]));
    }
    accumulate_block(v0, m0, sq, acc);
    accumulate_block(v1, m1, sq, acc);
  }
  store_partial(acc, sq.nq, partial + blockIdx.x * (int64_t)sq.nq);
}

// sse[bh][j] = sum over the head's chunks, in chunk order
__global__ __launch_bounds__(256) void k_sweep_reduce(const double* __restrict__ partial, int chunks, int nq,
                                                      int64_t n_out, double* __restrict__ sse) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_out) return;
  const int64_t bh = t / nq;
  const int j = (int)(t % nq);
  const double* p = partial + bh * chunks * (int64_t)nq + j;
  double s = 0.0;
  for (int c = 0; c < chunks; ++c) s = __dadd_rn(s, p[(int64_t)c * nq]);
  sse[t] = s;
}

template <int D, int DTYPE>
hipError_t launch_sweep_typed(const SweepArgs& a, const SweepQ& sq, hipStream_t s) {
  const int64_t groups = (int64_t)a.B * a.H * a.chunks;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  if (a.axis == 1)
    hipLaunchKernelGGL((k_sweep_tokens<D, DTYPE>), dim3((unsigned)groups), dim3(256), 0, s, x, a.H, a.N, a.sB, a.sH,
                       a.sN, a.chunks, sq, a.partial);
  else if (a.rotate)
    hipLaunchKernelGGL((k_sweep_headdim<D, DTYPE, true>), dim3((unsigned)groups), dim3(256), 0, s, x, a.H, a.N,
                       a.sB, a.sH, a.sN, a.chunks, sq, a.partial);
  else
    hipLaunchKernelGGL((k_sweep_headdim<D, DTYPE, false>), dim3((unsigned)groups), dim3(256), 0, s, x, a.H, a.N,
                       a.sB, a.sH, a.sN, a.chunks, sq, a.partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n_out = (int64_t)a.B * a.H * a.nq;
  hipLaunchKernelGGL(k_sweep_reduce, dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, s, a.partial, a.chunks,
                     a.nq, n_out, a.sse);
  return hipGetLastError();
}

QTensor headdim_tensor(const QuantArgs& a) {
  QTensor t;
  t.x = static_cast<const uint16_t*>(a.x);
  t.H = a.H;
  t.N = a.N;
  t.Np = (int)padded_tokens(a.N);
  t.sB = a.sB; t.sH = a.sH; t.sN = a.sN;
  t.total = (int64_t)a.B * a.H * t.Np * (a.d / 32);
  t.codes = a.codes;
  t.scales = a.scales;
  return t;
}

QTensor tokens_tensor(const QuantArgs& a) {
  QTensor t = headdim_tensor(a);
  t.total = (int64_t)a.B * a.H * (t.Np / 32);
  return t;
}

int64_t headdim_groups(const QTensor& t) { return (t.total + 256 * kHdUnitsPerThread - 1) / (256 * kHdUnitsPerThread); }
template <int D>
int64_t tokens_groups(const QTensor& t) { return (t.total * (D / 2) + 255) / 256; }

template <int D, int DTYPE, bool ROTATE, int RULE>
hipError_t launch_hd(const QuantArgs& a, hipStream_t stream) {
  const QTensor t = headdim_tensor(a);
  hipLaunchKernelGGL((k_quantize_headdim<D, DTYPE, ROTATE, RULE>), dim3((unsigned)headdim_groups(t)), dim3(256), 0,
                     stream, t, a.qbits);
  return hipGetLastError();
}

template <int D, int DTYPE, int RULE>
hipError_t launch_tok(const QuantArgs& a, hipStream_t stream) {
  const QTensor t = tokens_tensor(a);
  hipLaunchKernelGGL((k_quantize_tokens<D, DTYPE, RULE>), dim3((unsigned)tokens_groups<D>(t)), dim3(256), 0, stream,
                     t, a.qbits);
  return hipGetLastError();
}

template <int D, int DTYPE, bool ROTATE, int RULE>
hipError_t launch_qkv(const QuantArgs& q, const QuantArgs& k, const QuantArgs& v, hipStream_t stream) {
  const QTensor tq = headdim_tensor(q), tk = headdim_tensor(k), tv = tokens_tensor(v);
  const int64_t gq = headdim_groups(tq), gk = headdim_groups(tk), gv = tokens_groups<D>(tv);
  hipLaunchKernelGGL((k_quantize_qkv<D, DTYPE, ROTATE, RULE>), dim3((unsigned)(gq + gk + gv)), dim3(256), 0, stream,
                     tq, tk, tv, gq, gk, q.qbits);
  return hipGetLastError();
}

template <int D, int DTYPE, bool ROTATE>
hipError_t dispatch_qkv_rule(const QuantArgs& q, const QuantArgs& k, const QuantArgs& v, hipStream_t s) {
  if (q.rule == kRuleOcp) return launch_qkv<D, DTYPE, ROTATE, kRuleOcp>(q, k, v, s);
  return launch_qkv<D, DTYPE, ROTATE, kRuleUos>(q, k, v, s);
}

template <int D, int DTYPE>
hipError_t dispatch_qkv(const QuantArgs& q, const QuantArgs& k, const QuantArgs& v, hipStream_t s) {
  return q.rotate ? dispatch_qkv_rule<D, DTYPE, true>(q, k, v, s) : dispatch_qkv_rule<D, DTYPE, false>(q, k, v, s);
}

template <int D, int DTYPE, bool ROTATE>
hipError_t dispatch_hd_rot(const QuantArgs& a, hipStream_t s) {
  if (a.rule == kRuleOcp) return launch_hd<D, DTYPE, ROTATE, kRuleOcp>(a, s);
  if (a.rule == kRuleCeilQ) return launch_hd<D, DTYPE, ROTATE, kRuleCeilQ>(a, s);
  return launch_hd<D, DTYPE, ROTATE, kRuleUos>(a, s);
}

template <int D, int DTYPE>
hipError_t dispatch_hd_rule(const QuantArgs& a, hipStream_t s) {
  return a.rotate ? dispatch_hd_rot<D, DTYPE, true>(a, s) : dispatch_hd_rot<D, DTYPE, false>(a, s);
}

template <int D, int DTYPE>
hipError_t dispatch_tok_rule(const QuantArgs& a, hipStream_t s) {
  if (a.rule == kRuleOcp) return launch_tok<D, DTYPE, kRuleOcp>(a, s);
  if (a.rule == kRuleCeilQ) return launch_tok<D, DTYPE, kRuleCeilQ>(a, s);
  return launch_tok<D, DTYPE, kRuleUos>(a, s);
}

}  // namespace

hipError_t launch_quantize_headdim(const QuantArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.dtype == 1 ? dispatch_hd_rule<128, 1>(a, stream) : dispatch_hd_rule<128, 0>(a, stream);
  return a.dtype == 1 ? dispatch_hd_rule<64, 1>(a, stream) : dispatch_hd_rule<64, 0>(a, stream);
}

hipError_t launch_quantize_tokens(const QuantArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.dtype == 1 ? dispatch_tok_rule<128, 1>(a, stream) : dispatch_tok_rule<128, 0>(a, stream);
  return a.dtype == 1 ? dispatch_tok_rule<64, 1>(a, stream) : dispatch_tok_rule<64, 0>(a, stream);
}

hipError_t launch_quantize_qkv(const QuantArgs& q, const QuantArgs& k, const QuantArgs& v, hipStream_t stream) {
  if (q.d == 128) return q.dtype == 1 ? dispatch_qkv<128, 1>(q, k, v, stream) : dispatch_qkv<128, 0>(q, k, v, stream);
  return q.dtype == 1 ? dispatch_qkv<64, 1>(q, k, v, stream) : dispatch_qkv<64, 0>(q, k, v, stream);
}

int sweep_chunks(int axis, int N, int d) {
  const int64_t units = axis == 1 ? (int64_t)((N + 31) / 32) * (d / 2) : (int64_t)N * (d / 32);
  return (int)((units + 256 * kSweepUnits - 1) / (256 * kSweepUnits));
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of this device's `scratch`, looked up once per device with
// that device current (the caller's current device is the launch device).
hipError_t sweep_scratch_ptr(double** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<double*>(g_scratch_ptr[dev]);
  return hipSuccess;
}
}  // namespace

hipError_t launch_scale_sweep_static(const SweepArgs& a, hipStream_t stream) {
  SweepArgs b = a;
  hipError_t err = sweep_scratch_ptr(&b.partial);
  if (err != hipSuccess) return err;
  return launch_scale_sweep(b, stream);
}

hipError_t launch_scale_sweep(const SweepArgs& a, hipStream_t stream) {
  SweepQ sq;
  for (int j = 0; j < kSweepMax; ++j) sq.qb[j] = j < a.nq ? a.qbits[j] : 0u;
  sq.qmin = a.qmin_bits;
  sq.nq = a.nq;
  if (a.d == 128) return a.dtype == 1 ? launch_sweep_typed<128, 1>(a, sq, stream) : launch_sweep_typed<128, 0>(a, sq, stream);
  return a.dtype == 1 ? launch_sweep_typed<64, 1>(a, sq, stream) : launch_sweep_typed<64, 0>(a, sq, stream);
}

}  // namespace mxattn_internal
