// Quantize-on-append for fp16 keys and values, gfx950: the bulk path.
//
// Same encoding as the exact kernel in kvq_append.hip (sign flip, unnormalised
// Sylvester Walsh-Hadamard transform, fp16 norm, code = number of decision
// midpoints at or below z_j / (sqrt(D) ||x||), LSB-first packing; fp8 far-tier
// keys = E4M3FN(RNE, saturating)(z_j / sqrt(D))), organised so that a lane owns
// a whole vector:
//   * each lane holds 64 coordinates of a vector (lanes v + 64/LPV h, h <
//     LPV = D/64, hold one vector); each wave takes batches of 64/LPV
//     vectors of one stream (keys or values) of one (b, KV head); a work-group
//     serves one stream; a batch is one contiguous run of input rows, staged into
//     the wave's LDS buffer by direct-to-LDS 16-byte loads (each load
//     instruction one contiguous 1 KB, its vectors interleaved chunk by
//     chunk in LDS, so that the lanes' later 16-byte LDS reads of their own
//     vector's chunks fall in distinct banks);
//   * the next batch's loads are issued as soon as the current batch sits in
//     registers, so they overlap the arithmetic (four waves per SIMD cover
//     each other's waits);
//   * the transform runs in fp32 registers (the first stage straight from
//     the fp16 pairs with mixed-precision FMAs, six stages inside the lane,
//     the last one or two between the lanes of a vector through
//     v_permlane16_swap / v_permlane32_swap);
//   * a Lloyd-Max code is one 256-bin table read (bin = round(7.5 t + 127.5)
//     by v_cvt_pk_u8_f32, t = z / ||x||), one FMA against the bin's decision
//     midpoint and a sign test; an fp8 code is v_cvt_pk_fp8_f32 of the
//     clamped coordinate;
//   * each result carries a rigorous bound on its fp32 error (transform
//     rounding <= stages * 2^-24 * sum|x| <= stages * 2^-24 * sqrt(D) ||x||,
//     the norm's and the scaling's roundings; the fp16 norm is decided in
//     fp32 against the rounding midpoints around it); a vector with any
//     code, or its fp16 norm, within that bound of a decision is queued and
//     recomputed in float64 with other queued vectors of the wave (16
//     coordinates per lane, butterflies across lanes by DPP moves and
//     ds_swizzle; what is left at the end is pooled over the work-group), so
//     codes and norms equal the exact encoding everywhere outside the 1e-6
//     window of the parity contract;
//   * a key outlier stream ("Outlier Two-Stream Cache") is taken from the
//     staged rows before the lanes read them: each lane reads its share of
//     the vector's 8 channels, the vector's lanes reduce the largest
//     magnitude, scale = that / 127 in fp32 and code = RNE(x / scale) in
//     float64 (exact: an fp16 over an fp32 is a half-integer or at least
//     2^-25 of itself away from one, far past float64's rounding), the codes
//     and scale are stored, and the channels are zeroed in LDS so the
//     encoding above sees the inlier key.
// Sources: "The Engineering Behind AdapTQ", "The Math Fix" (sign flip + FWHT,
// add/sub only); VeloxQuant-MLX "Stage 2" (normalise, fp16 norm, nearest
// centroid) and "The Bit-Packing Problem" (LSB-first layout); "FoveatedKV",
// "The VR headset thing" (fp8 E4M3 far-tier keys).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"
#include "kvq_lane.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;                  // waves per work-group, each with its own batches
constexpr int kThreads = 64 * kWaves;
constexpr int kBins = 256;
constexpr float kBinScale = 7.5f;          // bins per unit of t; 256 bins span t in [-17.07, 17.07)
constexpr float kBinOffset = 127.5f;       // v_cvt_pk_u8_f32 rounds to nearest: bin = floor(7.5 t + 128)
constexpr double kBinSlack = 1e-3;         // each bin's rule also holds this far (in t) past its edges
constexpr float kU = 5.9604645e-8f;        // 2^-24, unit roundoff of fp32

template <int D>
struct Shape {
  static constexpr int LPV = D / 64;                   // lanes per vector: lane v + VPB h holds part h
  static constexpr int CPL = D / LPV;                  // coordinates per lane (64)
  static constexpr int VPB = 64 / LPV;                 // vectors per batch
  static constexpr int CH = D * 2 / 16;                // 16-byte chunks per fp16 vector
  static constexpr int CHL = CH / LPV;                 // chunks per lane
  static constexpr int VPI = 64 / CH;                  // vectors per 1 KB load instruction
  static constexpr int NI = VPB / VPI;                 // load instructions per batch
  static constexpr int PAD = D == 64 ? 128 : D == 128 ? 64 : 32;   // bytes after each kilobyte (bank spread)
  static constexpr int STRIDE = 1024 + PAD;
  static constexpr int BUF = NI * STRIDE;              // LDS bytes of one batch
  static constexpr int EPL = D / 64;                   // coordinates per lane on the exact path
  static constexpr int STAGES = __builtin_ctz(D);
};

typedef unsigned int uint4_t __attribute__((ext_vector_type(4)));
typedef unsigned int uint2_t __attribute__((ext_vector_type(2)));
constexpr int kRawBufferFlags = 0x00020000;     // 32-bit data format, untyped raw access
constexpr uint32_t kDrop = 0x80000000u;         // buffer offset past every descriptor's size: store dropped

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBufferFlags);
}

struct TableEntry {
  float negbnd;      // minus the decision midpoint inside the bin (t scale); +inf if none
  uint32_t code_hi;  // code of t at or past that midpoint (of the whole bin if none)
};

struct StreamArgs {
  const uint16_t *in;        // [pairs][n_new][D] fp16
  uint8_t *codes;            // [pairs][capacity][row]
  uint16_t *norms;           // [pairs][capacity] (Lloyd-Max formats)
  const float *centroids;    // [2^bits] (Lloyd-Max formats)
  // key outlier stream (OUT kernels, keys only): channels [pairs][8],
  // int8 codes [pairs][capacity][8], scales [pairs][capacity]
  const int32_t *out_idx;
  int8_t *out_codes;
  float *out_scales;
};

struct BulkArgs {
  StreamArgs s[2];           // keys, values
  const int8_t *signs;
  int pairs, n_new, capacity, start_pos;
  int batches_per_stream;    // pairs * ceil(n_new / VPB)
};

// ---- fp16 norm: RNE_fp16(sqrt(S)) decided exactly for a given S ----
__device__ inline double half_value(uint32_t bits) {
  if (bits >= 0x7C00u) return 65536.0;    // one step past the largest finite fp16
  return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ inline uint16_t norm_fp16(double S) {
  if (!(S > 0.0)) return 0;
  if (S >= 65520.0 * 65520.0) return 0x7C00;
  const float rf = (float)sqrt(S);
  uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)rf);
  if (h > 0x7BFFu) h = 0x7BFFu;
  if (h == 0u) h = 1u;
  const double v = half_value(h);
  const double lo = 0.5 * (half_value(h - 1) + v);
  const double hi = 0.5 * (v + half_value(h + 1));
  if (S < lo * lo || (S == lo * lo && (h & 1u))) h -= 1;
  else if (S > hi * hi || (S == hi * hi && (h & 1u))) h += 1;
  return (uint16_t)h;
}

// The fast path's fp16 norm, in fp32: RNE_fp16 of n = sqrt(S) (v_sqrt_f32,
// within 1 ulp) for an fp32 S whose relative error is at most eps, and
// whether the exact root could lie on the other side of one of the two
// rounding midpoints around that fp16 value: n within (eps/2 + 3u) n of one
// (the root halves S's relative error, v_sqrt_f32 adds at most 2u, the
// distance one more), with a quarter of headroom.  The midpoints of two
// adjacent fp16 values are exact in fp32.  Zero, subnormal-rounded and
// overflowing results are flagged too.
__device__ inline float half_f(uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); }

__device__ inline uint16_t norm_fp16_fast(float S, float eps, bool &near) {
  const float n = __builtin_amdgcn_sqrtf(S);
  const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)n);
  const float v = half_f(h);
  const float mlo = 0.5f * (half_f(h - 1u) + v), mhi = 0.5f * (v + half_f(h + 1u));
  const float d = fminf(fabsf(n - mlo), fabsf(n - mhi));
  near = near || h == 0u || h >= 0x7BFFu || !(d > 1.25f * (0.5f * eps + 3.f * kU) * n);
  return (uint16_t)h;
}

// ---- the code table of one Lloyd-Max stream (t = z / ||x||, N(0,1) scale) ----
template <int D>
__device__ void build_table(const float *centroids, int bits, TableEntry *table, uint32_t *ambiguous) {
  const int L = 1 << bits;
  const double root_d = sqrt((double)D);
  for (int bn = threadIdx.x; bn < kBins; bn += kThreads) {
    const double lo = ((double)bn - 128.0) / kBinScale - kBinSlack;
    const double hi = ((double)bn - 127.0) / kBinScale + kBinSlack;
    uint32_t below = 0, inside = 0;
    double mid_in = 0.0;
    for (int i = 0; i + 1 < L; ++i) {
      const double m = 0.5 * ((double)centroids[i] + (double)centroids[i + 1]) * root_d;
      if (m < lo) ++below;
      else if (m <= hi) { ++inside; mid_in = m; }
    }
    TableEntry e;
    if (inside == 0) e = TableEntry{INFINITY, below};
    else if (inside == 1) e = TableEntry{-(float)mid_in, below + 1};
    else {
      e = TableEntry{INFINITY, below};
      *ambiguous = 1u;                      // midpoints closer than a bin: every vector takes the exact path
    }
    table[bn] = e;
  }
}

// Bound on |t| wherever a bin holds a decision midpoint: the largest
// |centroid| on the t scale plus one bin width (bounds the relative part of
// the error of t near a decision).
template <int D>
__device__ inline float max_mid(const float *centroids, int bits) {
  const int L = 1 << bits;
  const float a = fabsf(centroids[0]), b = fabsf(centroids[L - 1]);
  return fmaxf(a, b) * sqrtf((float)D) + 0.2f;
}

// ---- staging: one batch of fp16 rows into the wave's LDS buffer ----
// Load instruction j covers the contiguous kilobyte of vectors VPI j ..
// VPI j + VPI - 1 (VPI = 64 / CH); its lane L = a + VPI c fetches chunk c of
// vector VPI j + a and lands at slot L of LDS block j (blocks STRIDE bytes
// apart).  Vector (j, a) thus reads its chunk c at j STRIDE + 16 a + 16 VPI c:
// one base per lane plus an immediate per chunk, and the bases of 16
// consecutive lanes fall in 16 distinct bank groups (the padding makes
// STRIDE / 16 = 8, 4, 2 mod 16 for D = 64, 128, 256).
template <int D>
__device__ inline void stage_batch(const StreamArgs &st, int pair, int t0, int n_new, uint8_t *buf) {
  using S = Shape<D>;
  const int lane = threadIdx.x & 63;
  const int a = lane % S::VPI, c = lane / S::VPI;
  const uint8_t *pbase = reinterpret_cast<const uint8_t *>(st.in) + (size_t)pair * n_new * (D * 2);
  if (t0 + S::VPB <= n_new) {
    const uint8_t *gbase = pbase + (size_t)t0 * (D * 2);
    const uint32_t off = (uint32_t)(a * (D * 2) + 16 * c);
#pragma unroll
    for (int j = 0; j < S::NI; ++j)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(gbase + j * 1024 + off),
                                       (__attribute__((address_space(3))) void *)(buf + j * S::STRIDE), 16, 0, 0);
  } else {
    // the last, partial batch of a (b, KV head): rows past the end repeat the last row
#pragma unroll
    for (int j = 0; j < S::NI; ++j) {
      const int t = min(t0 + j * S::VPI + a, n_new - 1);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(pbase + (size_t)t * (D * 2) + 16 * c),
                                       (__attribute__((address_space(3))) void *)(buf + j * S::STRIDE), 16, 0, 0);
    }
  }
}

// Base of the lane's staged vector (chunk k of the lane's half is at +16 VPI k).
template <int D>
__device__ inline const uint8_t *staged_base(const uint8_t *buf) {
  using S = Shape<D>;
  const int lane = threadIdx.x & 63;
  const int v = lane % S::VPB, h = lane / S::VPB;
  const int j = v / S::VPI, a = v % S::VPI;
  return buf + j * S::STRIDE + 16 * a + 16 * S::VPI * (h * S::CHL);
}

// x_lo + x_hi and x_lo - x_hi of an fp16 pair in fp32 (one rounding each).
__device__ inline void pair_sum_diff(uint32_t w, float &s, float &d) {
  asm volatile("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(s) : "v"(w));
  asm volatile("v_fma_mix_f32 %0, -%1, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w));
}

__device__ inline float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ inline float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// ---- the exact path: flagged vectors in float64, several per wave ----
// A vector the fast path flags is queued (its input row in a per-wave LDS
// list) and encoded later in a round of VPE vectors: lane (k, p) holds
// coordinates 16 p .. 16 p + 15 of queued vector k in float64.  Sums of fp16
// values are exact in float64 (each is an integer multiple of 2^-24 below
// 2^16, and D of them stay below 2^53 such units), so the butterflies are
// exact; the norm's sum of squares and the scaling round only at the level
// of 1e-16, far inside the 1e-6 window.  Kept out of line: it is rare, and
// inlined its constants would be hoisted into registers the fast path needs.
template <int D>
struct Exact {
  static constexpr int CPE = 16;             // coordinates per lane
  static constexpr int LPE = D / CPE;        // lanes per vector
  static constexpr int VPE = 64 / LPE;       // vectors per round
  // queue entries: a round's worth less one can wait, plus a whole batch
  static constexpr int QUEUE = (VPE - 1 + Shape<D>::VPB + 3) & ~3;
};

// v from lane ^ m, for m < 32: row-local DPP moves for m = 1, 2, ds_swizzle
// in xor mode above (no LDS access, no address registers).
__device__ inline uint32_t xor_lane_u32(uint32_t v, int m) {
  const int x = (int)v;
  if (m == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);     // quad_perm [1,0,3,2]
  if (m == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);     // quad_perm [2,3,0,1]
  if (m == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x101F);
  if (m == 8) return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x201F);
  return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x401F);
}

__device__ inline double xor_lane(double v, int m) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = xor_lane_u32((uint32_t)b, m), hi = xor_lane_u32((uint32_t)(b >> 32), m);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int D, int FMT, bool OUT>
__device__ __attribute__((always_inline)) inline void exact_round_body(
    const uint16_t *in, uint8_t *codes, uint16_t *norms, const int32_t *out_idx, const int8_t *signs_g,
    const double *mids_g, const uint32_t *queue_g, int nvec, int n_new, int capacity, int start_pos) {
  // the sign, midpoint and queue arrays live in LDS
  const auto *signs = (const __attribute__((address_space(3))) int8_t *)signs_g;
  const auto *mids = (const __attribute__((address_space(3))) double *)mids_g;
  const auto *queue = (const __attribute__((address_space(3))) uint32_t *)queue_g;
  using E = Exact<D>;
  constexpr int C = E::CPE;
  const int lane = threadIdx.x & 63;
  const int k = lane / E::LPE, p = lane % E::LPE;
  const bool active = k < nvec;
  const uint32_t id = queue[active ? k : 0];                 // input row: pair * n_new + t
  const int pair = (int)(id / (uint32_t)n_new);
  const int t = (int)id - pair * n_new;
  const uint4 *src = reinterpret_cast<const uint4 *>(in + (size_t)id * D + C * p);
  const uint4 w0 = src[0], w1 = src[1];
  const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const auto *sp = (const __attribute__((address_space(3))) uint32_t *)(signs + C * p);
  const uint32_t sw[4] = {sp[0], sp[1], sp[2], sp[3]};
  int32_t oidx[OUT ? kOutlierCount : 1];
  if constexpr (OUT) {
#pragma unroll
    for (int q = 0; q < kOutlierCount; ++q) oidx[q] = out_idx[(size_t)pair * kOutlierCount + q];
  }
  double x[C];
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const uint32_t bits = (wd[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
    double v = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    if constexpr (OUT) {
      // the outlier channels are zero in the inlier key
#pragma unroll
      for (int q = 0; q < kOutlierCount; ++q) v = (oidx[q] == C * p + e) ? 0.0 : v;
    }
    ss = fma(v, v, ss);
    const bool neg = ((sw[e / 4] >> (8 * (e % 4))) & 0x80u) != 0u;
    x[e] = neg ? -v : v;
  }
  // butterflies inside the lane (coordinate bits 0-3), then across the
  // vector's lanes (coordinate bit 4 + log2 m pairs lanes p and p ^ m)
#pragma unroll
  for (int h = 1; h < C; h <<= 1) {
#pragma unroll
    for (int e = 0; e < C; ++e) {
      if (!(e & h)) {
        const double a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < E::LPE; m <<= 1) {
    const bool upper = (p & m) != 0;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      const double o = xor_lane(x[e], m);
      x[e] = upper ? o - x[e] : x[e] + o;
    }
    ss += xor_lane(ss, m);
  }
  const size_t slot = (size_t)pair * capacity + start_pos + t;
  constexpr int ROW = FMT == 8 ? D : D * FMT / 8;
  uint8_t *row = codes + slot * ROW;
  if constexpr (FMT == 8) {
    const double rs = 1.0 / sqrt((double)D);
    uint32_t cw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < C; ++e) {
      // y rounded once to fp32, then to E4M3 (the two roundings can differ
      // from one only within 2^-24 |y| of an E4M3 midpoint: inside the window)
      const float y = fminf(fmaxf((float)(x[e] * rs), -448.f), 448.f);
      const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
      cw[e / 4] |= c << (8 * (e % 4));
    }
    if (active) *reinterpret_cast<uint4 *>(row + C * p) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
  } else {
    constexpr int L = 1 << FMT;
    const uint16_t n16 = norm_fp16(ss);
    if (active && p == 0) norms[slot] = n16;
    const double inv = ss > 0.0 ? 1.0 / sqrt((double)D * ss) : 0.0;
    uint32_t cw[2] = {0u, 0u};                              // 16 codes, LSB first
#pragma unroll
    for (int e = 0; e < C; ++e) {
      // number of midpoints at or below u, by binary search over the
      // ascending midpoints; a zero vector takes the middle code
      const double u = x[e] * inv;
      uint32_t code = 0;
#pragma unroll
      for (int step = L / 2; step >= 1; step >>= 1) code += (u >= mids[code + step - 1]) ? (uint32_t)step : 0u;
      code = ss > 0.0 ? code : (uint32_t)(L / 2);
      const int bit = FMT * e;
      cw[bit / 32] |= code << (bit % 32);
      if ((bit % 32) + FMT > 32) cw[bit / 32 + 1] |= code >> (32 - bit % 32);
    }
    if (active) {
      uint8_t *dst = row + 2 * FMT * p;                    // 16 codes = 2 FMT bytes
      if constexpr (FMT == 4) *reinterpret_cast<uint2 *>(dst) = make_uint2(cw[0], cw[1]);
      else if constexpr (FMT == 2) *reinterpret_cast<uint32_t *>(dst) = cw[0];
      else {
        reinterpret_cast<uint16_t *>(dst)[0] = (uint16_t)(cw[0] & 0xFFFFu);
        reinterpret_cast<uint16_t *>(dst)[1] = (uint16_t)(cw[0] >> 16);
        reinterpret_cast<uint16_t *>(dst)[2] = (uint16_t)(cw[1] & 0xFFFFu);
      }
    }
  }
}

// Out of line for the rounds inside the batch loop (inlined there, its
// constants would be hoisted out of the loop into registers the fast path
// needs); the end-of-launch rounds take the body inline, which spares the
// call's register saves to scratch memory on the launch's critical path.
template <int D, int FMT, bool OUT>
__device__ __attribute__((noinline)) void exact_round(const uint16_t *in, uint8_t *codes, uint16_t *norms,
                                                      const int32_t *out_idx, const int8_t *signs_g,
                                                      const double *mids_g, const uint32_t *queue_g, int nvec,
                                                      int n_new, int capacity, int start_pos) {
  exact_round_body<D, FMT, OUT>(in, codes, norms, out_idx, signs_g, mids_g, queue_g, nvec, n_new, capacity,
                                start_pos);
}

// ---- the fast path: one batch of one stream ----
// The outlier stream of one staged batch (see the file comment): lane
// (v, h) takes channels k = KPL h .. KPL h + KPL-1 of vector v.
template <int D>
__device__ inline void outlier_batch(const StreamArgs &st, int pair, int t0, int n_new, int capacity, int start_pos,
                                     uint8_t *buf, uint32_t drop) {
  using S = Shape<D>;
  constexpr int KPL = kOutlierCount / S::LPV;
  const int lane = threadIdx.x & 63;
  const int v = lane % S::VPB, h = lane / S::VPB;
  const int j = v / S::VPI, a = v % S::VPI;
  uint8_t *vb = buf + j * S::STRIDE + 16 * a;
  const int32_t *idx = st.out_idx + (size_t)pair * kOutlierCount;
  float xk[KPL];
  uint32_t addr[KPL];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const uint32_t c = (uint32_t)idx[KPL * h + k] & (uint32_t)(D - 1);
    addr[k] = 16u * S::VPI * (c >> 3) + 2u * (c & 7u);
    xk[k] = (float)*reinterpret_cast<const _Float16 *>(vb + addr[k]);
    amax = fmaxf(amax, fabsf(xk[k]));
  }
#pragma unroll
  for (int hb = 1; hb < S::LPV; hb <<= 1) amax = fmaxf(amax, __shfl_xor(amax, hb * S::VPB));
  const float scale = amax / 127.f;              // one float32 rounding
  uint32_t cw[2] = {0u, 0u};                     // the lane's codes, four per word
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const double u = (scale > 0.f) ? (double)xk[k] / (double)scale : 0.0;
    const int c = (int)fmin(fmax(rint(u), -127.0), 127.0);
    cw[k / 4] |= ((uint32_t)c & 0xFFu) << (8 * (k % 4));
    *reinterpret_cast<uint16_t *>(vb + addr[k]) = 0;   // the inlier key has the channel zeroed
  }
  const __amdgpu_buffer_rsrc_t cr =
      make_rsrc(st.out_codes + (size_t)pair * capacity * kOutlierCount, (uint32_t)capacity * kOutlierCount);
  const uint32_t coff = ((uint32_t)(start_pos + t0 + v) * kOutlierCount + KPL * h) | drop;
  if constexpr (KPL == 8) __builtin_amdgcn_raw_buffer_store_b64((uint2_t){cw[0], cw[1]}, cr, coff, 0, 0);
  else if constexpr (KPL == 4) __builtin_amdgcn_raw_buffer_store_b32(cw[0], cr, coff, 0, 0);
  else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)cw[0], cr, coff, 0, 0);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(st.out_scales + (size_t)pair * capacity, (uint32_t)capacity * 4u);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, scale), sr,
                                        ((uint32_t)(start_pos + t0 + v) * 4u) | drop | ((uint32_t)-h & kDrop), 0, 0);
}

template <int D, int FMT, bool OUT>
__device__ void encode_batch(const StreamArgs &st, const int8_t *signs, const double *mids, int pair, int t0,
                             int n_new, int capacity, int start_pos, uint8_t *buf, const uint32_t *masks,
                             const TableEntry *table, float mmax, bool force_exact, uint32_t *queue, int &count,
                             bool issue_next,
                             const StreamArgs &nst, int npair, int nt0, uint8_t *nbuf) {
  using S = Shape<D>;
  constexpr int CPL = S::CPL;
  const int lane = threadIdx.x & 63;
  const int v = lane % S::VPB;
  const int h = lane / S::VPB;
  const int t = t0 + v;
  const bool valid = t < n_new;
  // store offsets of rows past the context get bit 31 (dropped by the buffer
  // descriptor's size check), computed without a select the compiler could
  // turn into a branch
  const uint32_t drop = (uint32_t)(n_new - 1 - t) & kDrop;
  if constexpr (OUT) outlier_batch<D>(st, pair, t0, n_new, capacity, start_pos, buf, drop);

  // the lane's fp16 pairs, sign-flipped (mask word e covers coordinates 2e, 2e + 1)
  uint32_t w[CPL / 2];
  const uint8_t *sb = staged_base<D>(buf);
#pragma unroll
  for (int k = 0; k < S::CHL; ++k) {
    const uint4 q = *reinterpret_cast<const uint4 *>(sb + 16 * S::VPI * k);
    w[4 * k + 0] = q.x;
    w[4 * k + 1] = q.y;
    w[4 * k + 2] = q.z;
    w[4 * k + 3] = q.w;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): the buffer is in registers
  if (issue_next) stage_batch<D>(nst, npair, nt0, n_new, nbuf);
  __builtin_amdgcn_sched_barrier(0);

  // per chunk: sign flip, squared norm (exact products, eight fp32 partial
  // sums) and the first butterfly stage straight from the fp16 pairs
  float z[CPL];
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint4 *mrow = reinterpret_cast<const uint4 *>(masks + h * (CPL / 2));
  uint4 mnext = mrow[0];
#pragma unroll
  for (int k = 0; k < S::CHL; ++k) {
    const uint4 m = mnext;                 // the next chunk's masks are requested one chunk ahead
    if (k + 1 < S::CHL) mnext = mrow[k + 1];
    const uint32_t mk[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * k + q;
      const uint32_t x = w[e] ^ mk[q];
      const float a = half_lo(x), b = half_hi(x);
      acc[e & 7] = fmaf(a, a, fmaf(b, b, acc[e & 7]));
      pair_sum_diff(x, z[2 * e], z[2 * e + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  float ss = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
#pragma unroll
  for (int hb = 1; hb < S::LPV; hb <<= 1) ss += __shfl_xor(ss, hb * S::VPB);
  // remaining stages inside the lane
#pragma unroll
  for (int hs = 2; hs < CPL; hs <<= 1) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      if (!(i & hs)) {
        const float a = z[i], b = z[i + hs];
        z[i] = a + b;
        z[i + hs] = a - b;
      }
    }
  }
  // the stages across the lanes of a vector: part h pairs with part h ^ hb,
  // VPB hb lanes away (16: v_permlane16_swap, 32: v_permlane32_swap)
#pragma unroll
  for (int hb = 1; hb < S::LPV; hb <<= 1) {
#pragma unroll
    for (int i = 0; i < CPL; i += 2) {
      // after the swap the lower part's lane holds (z_i, partner's z_i) and
      // the upper part's lane (partner's z_i+1, z_i+1); the second swap puts
      // the sums and differences back in place
      float p = z[i], q = z[i + 1];
      if (hb * S::VPB == 16) swap16(p, q);
      else swap32(p, q);
      float s = p + q, d = p - q;
      if (hb * S::VPB == 16) swap16(s, d);
      else swap32(s, d);
      z[i] = s;
      z[i + 1] = d;
    }
  }

  // Error bounds (t scale): transform rounding <= STAGES u sum|x| / ||x|| <=
  // STAGES u sqrt(D); ss has relative error <= (CPL/8 + 5) u, so r = rsq(ss)
  // <= ((CPL/8 + 5)/2 + 1) u, and t = z r one more u: |t~ - t| <= the
  // absolute part plus (CPL/16 + 5) u |t|, |t| <= mmax near a decision; the
  // fp32 midpoint adds u mmax.  25% of headroom on top.
  // zero, tiny or overflowing norms, and codebooks with midpoints closer
  // than a table bin: exact path
  bool near = force_exact || !(ss > 1e-30f && ss < 4.2e9f);
  constexpr int ROW = FMT == 8 ? D : D * FMT / 8;
  constexpr int LB = ROW / S::LPV;               // row bytes per lane
  uint32_t packed[LB / 4];
#pragma unroll
  for (int i = 0; i < LB / 4; ++i) packed[i] = 0;
  uint16_t nstore = 0;
  if constexpr (FMT == 8) {
    constexpr float rs = D == 64 ? 0.125f : D == 128 ? 0.08838834764831845f : 0.0625f;   // RN(1/sqrt(D))
    const float nrm = sqrtf(ss);
    const float m8 = 1.25f * kU * ((float)S::STAGES + 3.f) * nrm * 1.001f + 1e-30f;
    // codes of y and of y -/+ the bound: a code is settled when all three agree
    uint32_t diffbits = 0;
#pragma unroll
    for (int i = 0; i < CPL; i += 4) {
      float y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = __builtin_amdgcn_fmed3f(z[i + k] * rs, -448.f, 448.f);
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c, true);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] - m8, y[1] - m8, 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] - m8, y[3] - m8, lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] + m8, y[1] + m8, 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] + m8, y[3] + m8, hi, true);
      diffbits |= (uint32_t)(lo ^ hi);
      packed[i / 4] = (uint32_t)c;
    }
    near |= diffbits != 0;
  } else {
    const float r = __builtin_amdgcn_rsqf(ss);
    const float rb = r * kBinScale;
    const float margin = 1.25f * kU * ((float)S::STAGES * sqrtf((float)D) + ((float)CPL / 16.f + 6.f) * mmax) + 1e-7f;
    nstore = norm_fp16_fast(ss, (float)(CPL / 8 + 6) * kU, near);
    float nmin = INFINITY;                  // smallest |t - midpoint| over the lane's codes
    // 16 coordinates at a time (bounds the table reads in flight)
#pragma unroll
    for (int g = 0; g < CPL; g += 16) {
#pragma unroll
      for (int i = g; i < g + 16; ++i) {
        const uint32_t bin = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(z[i], rb, kBinOffset), 0, 0u);
        const TableEntry te = table[bin];
        const float diff = fmaf(z[i], r, te.negbnd);
        const uint32_t code = te.code_hi - (__builtin_bit_cast(uint32_t, diff) >> 31);
        nmin = fminf(nmin, fabsf(diff));
        constexpr int B = FMT;
        const int bit = B * i;
        packed[bit / 32] |= code << (bit % 32);
        if ((bit % 32) + B > 32) packed[bit / 32 + 1] |= code >> (32 - bit % 32);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    near |= !(nmin > margin);
  }
  // both halves of a vector agree on the path (the shuffle runs in every
  // lane: under a short-circuit || the flagged lanes would sit it out)
  {
    int any = near ? 1 : 0;
#pragma unroll
    for (int hb = 1; hb < S::LPV; hb <<= 1) any |= __shfl_xor(any, hb * S::VPB);
    near = any != 0;
  }
  // Every lane stores, with bit 31 set in the offset (past the descriptor's
  // size: the hardware drops the store) for rows past the context and for
  // flagged vectors, which the exact path writes instead: no branch for the
  // compiler to sink the code computation behind.
  const uint32_t skip = drop | (near ? kDrop : 0u);
  if constexpr (FMT != 8) {
    const __amdgpu_buffer_rsrc_t nrs = make_rsrc(st.norms + (size_t)pair * capacity, (uint32_t)capacity * 2u);
    __builtin_amdgcn_raw_buffer_store_b16(nstore, nrs, ((uint32_t)(start_pos + t) * 2u) | skip | ((uint32_t)-h & kDrop),
                                          0, 0);
  }
  {
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(st.codes + (size_t)pair * capacity * ROW, (uint32_t)capacity * ROW);
    const uint32_t off = ((uint32_t)(start_pos + t) * ROW + h * LB) | skip;
    if constexpr (LB % 16 == 0) {
#pragma unroll
      for (int i = 0; i < LB / 16; ++i) {
        const uint4_t q = {packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(q, crs, off + 16 * i, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LB / 8; ++i) {
        const uint2_t q = {packed[2 * i], packed[2 * i + 1]};
        __builtin_amdgcn_raw_buffer_store_b64(q, crs, off + 8 * i, 0, 0);
      }
    }
  }
  // flagged vectors join the wave's queue for the exact path
  const bool queued = valid && near && h == 0;
  const uint64_t flagged = __ballot(queued);
  if (flagged) {
    const uint32_t rank =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(flagged >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)flagged, 0u));
    if (queued) queue[count + (int)rank] = (uint32_t)(pair * n_new + t);
    count += __popcll(flagged);
  }
}

// One stream (keys or values) per work-group: the batch loop of one format,
// run by every wave of the work-group over its own batches.
template <int D, int FMT, bool OUT>
__device__ void run_stream(const StreamArgs &st, const BulkArgs &A, uint8_t *smem) {
  using S = Shape<D>;
  uint8_t *bufs = smem;                                                    // kWaves * BUF
  TableEntry *table = reinterpret_cast<TableEntry *>(smem + kWaves * S::BUF);
  uint32_t *masks = reinterpret_cast<uint32_t *>(table + kBins);          // D / 2 words
  double *mids = reinterpret_cast<double *>(masks + D / 2);               // float64 decision midpoints
  int8_t *lsigns = reinterpret_cast<int8_t *>(mids + 16);                  // D signs
  uint32_t *queues = reinterpret_cast<uint32_t *>(lsigns + D);           // kWaves * QUEUE entries

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // uniform: batch math in SGPRs
  uint8_t *buf = bufs + wave * S::BUF;
  uint32_t *queue = queues + wave * Exact<D>::QUEUE;
  int count = 0;                            // wave-uniform: entries waiting in the queue
  const int chunks = (A.n_new + S::VPB - 1) / S::VPB;
  const int total = A.batches_per_stream;
  const int gw = blockIdx.x * kWaves + wave, nw = gridDim.x * kWaves;

  // the first batch's loads go out before the tables are built
  int pair = gw / chunks, t0 = (gw - (gw / chunks) * chunks) * S::VPB;
  if (gw < total) stage_batch<D>(st, pair, t0, A.n_new, buf);
  __shared__ uint32_t ambiguous;
  if (threadIdx.x == 0) ambiguous = 0u;
  __syncthreads();
  if constexpr (FMT != 8) build_table<D>(st.centroids, FMT, table, &ambiguous);
  for (int e = threadIdx.x; e < D / 2; e += kThreads)
    masks[e] = (A.signs[2 * e] < 0 ? 0x8000u : 0u) | (A.signs[2 * e + 1] < 0 ? 0x80000000u : 0u);
  for (int e = threadIdx.x; e < D; e += kThreads) lsigns[e] = A.signs[e];
  if constexpr (FMT != 8) {
    if (threadIdx.x + 1 < (1 << FMT))
      mids[threadIdx.x] = 0.5 * ((double)st.centroids[threadIdx.x] + (double)st.centroids[threadIdx.x + 1]);
  }
  __syncthreads();
  const float mmax = FMT == 8 ? 0.f : max_mid<D>(st.centroids, FMT);
  const bool force_exact = __builtin_amdgcn_readfirstlane((int)ambiguous) != 0;

  for (int id = gw; id < total; id += nw) {
    const int nid = id + nw;
    const bool next = nid < total;
    const int npair = next ? nid / chunks : 0;
    const int nt0 = next ? (nid - npair * chunks) * S::VPB : 0;
    __builtin_amdgcn_s_waitcnt(0);          // vmcnt(0): this batch has landed in LDS
    encode_batch<D, FMT, OUT>(st, lsigns, mids, pair, t0, A.n_new, A.capacity, A.start_pos, buf, masks, table, mmax,
                              force_exact, queue, count, next, st, npair, nt0, buf);
    // a full round of queued vectors goes through the exact path (the queue
    // entries were written by other lanes of this wave)
    while (count >= Exact<D>::VPE) {
      count -= Exact<D>::VPE;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      exact_round<D, FMT, OUT>(st.in, st.codes, st.norms, st.out_idx, lsigns, mids, queue + count, Exact<D>::VPE,
                               A.n_new, A.capacity, A.start_pos);
    }
    pair = npair;
    t0 = nt0;
  }
  // What is left in the waves' queues is pooled over the work-group (the
  // staging buffers are free once every batch is done) and shared out in
  // full rounds: every wave running its own, mostly empty, round at the end
  // of the launch would cost more than the rounds the launch needs.
  __shared__ int left[kWaves];
  const int lane = threadIdx.x & 63;
  if (lane == 0) left[wave] = count;
  __syncthreads();
  int base = 0, pooled = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = left[w];
    base += w < wave ? c : 0;
    pooled += c;
  }
  uint32_t *pool = reinterpret_cast<uint32_t *>(bufs);
  for (int j = lane; j < count; j += 64) pool[base + j] = queue[j];
  __syncthreads();
  for (int r = wave * Exact<D>::VPE; r < pooled; r += kWaves * Exact<D>::VPE)
    exact_round_body<D, FMT, OUT>(st.in, st.codes, st.norms, st.out_idx, lsigns, mids, pool + r,
                                  min(Exact<D>::VPE, pooled - r), A.n_new, A.capacity, A.start_pos);
}

template <int D>
constexpr int kLdsBytes = kWaves * Shape<D>::BUF + kBins * (int)sizeof(TableEntry) + D / 2 * 4 + 16 * 8 + D +
                          kWaves * Exact<D>::QUEUE * 4;

template <int D, int KF, int VF, bool OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void append_bulk_kernel(BulkArgs A) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes<D>];
  if (blockIdx.y == 0) run_stream<D, KF, OUT>(A.s[0], A, smem);
  else run_stream<D, VF, false>(A.s[1], A, smem);
}

template <int D, int KF, int VF>
hipError_t go(const AppendArgs &a, hipStream_t stream) {
  using S = Shape<D>;
  BulkArgs A;
  A.s[0] = StreamArgs{static_cast<const uint16_t *>(a.k), a.k_codes, a.k_norms, a.k_centroids, a.outlier_idx,
                      a.outlier_codes, a.outlier_scales};
  A.s[1] = StreamArgs{static_cast<const uint16_t *>(a.v), a.v_codes, a.v_norms, a.v_centroids, nullptr, nullptr,
                      nullptr};
  A.signs = a.signs;
  A.pairs = a.batch * a.kv_heads;
  A.n_new = a.n_new;
  A.capacity = a.capacity;
  A.start_pos = a.start_pos;
  const int chunks = (a.n_new + S::VPB - 1) / S::VPB;
  A.batches_per_stream = A.pairs * chunks;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess)
    cus = 256;
  // persistent work-groups: as many as stay resident (four per compute
  // unit), half of them per stream
  const long long total = A.batches_per_stream;
  const int blocks = (int)std::min<long long>((total + kWaves - 1) / kWaves, 2ll * cus);
  if constexpr (KF != 8) {
    if (a.outlier_idx) {
      hipLaunchKernelGGL((append_bulk_kernel<D, KF, VF, true>), dim3(blocks, 2), dim3(kThreads), 0, stream, A);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((append_bulk_kernel<D, KF, VF, false>), dim3(blocks, 2), dim3(kThreads), 0, stream, A);
  return hipGetLastError();
}

template <int D, int KF>
hipError_t go_v(const AppendArgs &a, hipStream_t stream, bool *ok) {
  switch (a.v_format) {
    case 2: return go<D, KF, 2>(a, stream);
    case 3: return go<D, KF, 3>(a, stream);
    case 4: return go<D, KF, 4>(a, stream);
  }
  *ok = false;
  return hipSuccess;
}

template <int D>
hipError_t go_k(const AppendArgs &a, hipStream_t stream, bool *ok) {
  switch (a.k_format) {
    case 2: return go_v<D, 2>(a, stream, ok);
    case 3: return go_v<D, 3>(a, stream, ok);
    case 4: return go_v<D, 4>(a, stream, ok);
    case 8: return go_v<D, 8>(a, stream, ok);
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

bool bulk_append_supported(const AppendArgs &a) {
  const bool vf = a.v_format >= 2 && a.v_format <= 4;
  const bool kf = (a.k_format >= 2 && a.k_format <= 4) || a.k_format == 8;
  return a.in_f16 && vf && kf && (a.head_dim == 64 || a.head_dim == 128 || a.head_dim == 256) && a.n_new >= 64 &&
         (a.outlier_idx == nullptr || a.k_format != 8) && a.qjl_proj == nullptr &&
         (long long)a.capacity * kOutlierCount < (1ll << 31) &&
         (long long)a.batch * a.kv_heads * a.n_new < (1ll << 31) &&     // exact-path queue entries: input rows
         (long long)a.batch * a.kv_heads * ((a.n_new + 63) / 64) * 2 < (1ll << 31) &&
         (long long)a.capacity * a.head_dim < (1ll << 31);    // one (b, KV head) slice of codes within a buffer descriptor
}

hipError_t launch_append_bulk(const AppendArgs &a, hipStream_t stream) {
  bool ok = true;
  hipError_t e = hipSuccess;
  switch (a.head_dim) {
    case 64: e = go_k<64>(a, stream, &ok); break;
    case 128: e = go_k<128>(a, stream, &ok); break;
    case 256: e = go_k<256>(a, stream, &ok); break;
    default: ok = false;
  }
  return ok ? e : hipErrorInvalidValue;
}

}  // namespace kvq
