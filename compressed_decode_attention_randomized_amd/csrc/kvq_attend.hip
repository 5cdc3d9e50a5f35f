// Fused split-K GQA decode attention on the compressed cache, gfx950.
//
// Grid: x = split (near-tier splits first, then far-tier splits), y = (b, kv head).
// A 256-thread work-group serves the G query heads that share one KV head, so
// every code row is read from HBM once for all G heads.
//
// Per work-group:
//   1. every lane requests its row of the first block of tokens; meanwhile
//      wave 0 loads the G queries and, for far splits, sign-flips and
//      Walsh-Hadamard transforms them in registers (the query is rotated
//      once, keys are never rotated back) and stores them to LDS, one
//      barrier; each lane takes its coordinates pre-scaled by
//      log2(e)/sqrt(d) (near) or log2(e)/d (far: rotation normalisation
//      times the softmax scale);
//   2. each token row is processed by D/DPL lanes, each lane owning DPL
//      consecutive coordinates: the lane reads its slice of the packed key row
//      (nontemporal vector loads), looks its codes up in LDS (two 2- or 3-bit
//      codes per read from a pair table, 4-bit codes one per read at offsets
//      taken with SDWA byte selects; fp8 keys are converted in hardware, two
//      per instruction) and accumulates q~ . c[code] for the G heads; the
//      slice sums are combined by DPP adds and multiplied by the fp16 norm;
//   3. online softmax per lane slot in base 2 (one exp2 per score; the state
//      is rescaled only when a score passes the reference point by kSlack);
//      values are accumulated in the rotated domain straight from their codes;
//   4. the slot states are merged by xor-shuffles inside the wave and through
//      LDS across the four waves; the split writes (m, l) and sum p v / l.
// Key side streams (far tier), both folded into each lane's partial score
// before the cross-lane reduction: an outlier stream adds
// q[idx] . (code * scale), its 8 channels shared out over the lanes of a
// token; a QJL sketch adds ||r|| sqrt(pi/2)/m sum_i (2 z_i - 1) (S q~)_i,
// with S q~ formed once per work-group into LDS and each lane scoring its
// slice of the sketch bits.
// Near-tier splits run the same loop on fp16 rows in the original domain.
// Sources: "The Engineering Behind AdapTQ", "Engineering the Hot Path" (rotate
// q once, score from codes through a table, no dequantize pass); "FoveatedKV",
// "Making it fast" (fused split-K dispatch over both tiers, q pre-scaled,
// online softmax with one exp per score, fp8 keys for the far tier);
// VeloxQuant-MLX, "Stage 3: QJL Residual Correction" and "Outlier Two-Stream
// Cache" (the two key side streams).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"
#include "kvq_lane.h"

namespace kvq {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
  const void *q;
  int q_f16;
  int kv_heads, q_heads, capacity, seq_len, num_splits, num_near_splits, near_len;
  const uint8_t *k_codes, *v_codes;
  const uint16_t *k_norms, *v_norms;
  const int8_t *signs;
  const float *k_centroids, *v_centroids;
  const uint16_t *near_k, *near_v;
  float *part_o, *part_ml;
  const float *gate_ref, *spike_ref;   // [B][Hq] natural-log references or NULL (gated launches)
  uint32_t *spike_bits;                // [B][Hq][spike_words]
  int spike_words;
  const int32_t *out_idx;              // key outlier stream ([B][Hkv][8] channels) or NULL
  const int8_t *out_codes;             // [B][Hkv][capacity][8]
  const float *out_scales;             // [B][Hkv][capacity]
  const float *qjl_proj;               // QJL sketch: S^T [D][D] or NULL
  const uint8_t *qjl_signs;            // [B][Hkv][capacity][D/8]
  const uint16_t *qjl_norms;           // [B][Hkv][capacity] fp16
};

// Key side streams of the far tier.
constexpr int kNoExtra = 0, kOutliers = 1, kQjl = 2;

// Score gate and spike flags of the far tier for one block of tokens, the G
// heads of one KV head (log2 score units, as the kernel keeps them).
template <int G>
struct FarGate {
  float gate[G], spike[G];              // thresholds: -inf gate / +inf spike when not asked for
  uint32_t *bits;                       // this (b, KV head)'s first head row of flag words, or NULL
  int words;
};

// Loads NB bytes (NB a multiple of 2) at p into 32-bit words, using the widest
// access the slice alignment allows.  Cache rows are read once per launch, so
// the loads carry the nontemporal hint (streamed past the caches instead of
// allocated in them: a plain read of a 947 MB buffer by 4864 work-groups
// measured 5.94 TB/s with ordinary 16-byte loads and 6.43 TB/s with these).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int NB>
__device__ inline void load_slice(const uint8_t *p, uint32_t (&w)[(NB + 3) / 4]) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + i);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (NB % 8 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 8; ++i) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p) + i);
      w[2 * i] = v.x; w[2 * i + 1] = v.y;
    }
  } else if constexpr (NB % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) w[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p) + i);
  } else {
#pragma unroll
    for (int i = 0; i < (NB + 3) / 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < NB / 2; ++i) {
      const uint32_t h = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p) + i);
      w[i >> 1] |= h << (16 * (i & 1));
    }
  }
}
__device__ inline uint32_t load_u16(const uint16_t *p) { return __builtin_nontemporal_load(p); }

// Code e of an LSB-first bit stream held in 32-bit words.
template <int B>
__device__ inline uint32_t code_at(const uint32_t *w, int e) {
  const int o = e * B, wi = o >> 5, sh = o & 31;
  if (sh + B <= 32) return (w[wi] >> sh) & ((1u << B) - 1u);
  return ((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) & ((1u << B) - 1u);
}

// Table offsets (4 c) of the eight 4-bit codes of w, code e at bits 4e..4e+3:
// byte k of w << 2 holds code 2k at bits 2..5 and byte k of w >> 2 code
// 2k + 1, so each offset is one v_and_b32 with an SDWA byte select (the
// compiler would fold the pre-shifts back into a shift and a mask per code).
template <int K>
__device__ inline uint32_t masked_byte(uint32_t w) {
  uint32_t r;
  if constexpr (K == 0) r = w & 0x3Cu;
  if constexpr (K == 1) asm("v_and_b32_sdwa %0, 60, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(w));
  if constexpr (K == 2) asm("v_and_b32_sdwa %0, 60, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(w));
  if constexpr (K == 3) asm("v_and_b32_sdwa %0, 60, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(w));
  return r;
}
__device__ inline void nibble_offsets(uint32_t w, uint32_t (&o)[8]) {
  const uint32_t a = w << 2, b = w >> 2;
  o[0] = masked_byte<0>(a); o[1] = masked_byte<0>(b);
  o[2] = masked_byte<1>(a); o[3] = masked_byte<1>(b);
  o[4] = masked_byte<2>(a); o[5] = masked_byte<2>(b);
  o[6] = masked_byte<3>(a); o[7] = masked_byte<3>(b);
}
__device__ inline float table_at(const float *lut, uint32_t off) {
  return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(lut) + off);
}

__device__ inline float half_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Running softmax state of one lane slot for G heads (base-2 logits).
// m is a reference point, not necessarily the running maximum: the state is
// rescaled only when a score exceeds m by more than kSlack, so weights
// 2^(s - m) stay below 2^kSlack and l, acc hold sum 2^(s - m) (v) for that m.
// The quotient acc / l is the same for any m; the rescale, a branch a wave
// takes whenever one of its slots needs it, then runs a few times per slot
// instead of at every new maximum.  mx tracks the true maximum (one max per
// score), and the split's l is restated against it when it is written, so
// (m, l) keeps its meaning (split maximum, sum of exp(s - maximum)); m never
// exceeds mx and mx never exceeds m + kSlack.
constexpr float kSlack = 8.f;
template <int G, int DPL>
struct State {
  float m[G], mx[G], l[G], acc[G][DPL];
  __device__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      mx[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
    }
  }
  // Adds one token with scores s[h] (already -inf if the token is absent);
  // returns the weights p[h] for the value accumulation.  For G >= 2 the
  // exponentials are the hardware's v_exp_f32 (weights are at most 2^kSlack;
  // one that would be below 2^-126 becomes 0, which no fp32 sum of weights
  // would notice): 3-6% on those launches; the G = 1 launches measured
  // slower with it (two_tier 171.9 -> 184.4 us) and keep exp2f.
  __device__ static float exp2w(float x) {
    if constexpr (G >= 2) return __builtin_amdgcn_exp2f(x);
    else return exp2f(x);
  }
  __device__ void add_scores(const float (&s)[G], float (&p)[G]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (s[h] > m[h] + kSlack) {
        const float alpha = exp2w(m[h] - s[h]);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] *= alpha;
        m[h] = s[h];
      }
      p[h] = (s[h] == -INFINITY) ? 0.f : exp2w(s[h] - m[h]);
      l[h] += p[h];
      mx[h] = fmaxf(mx[h], s[h]);
    }
  }
  // Merge with the state held by lane (lane ^ mask).
  __device__ void merge_xor(int mask) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], mask);
      const float lo = __shfl_xor(l[h], mask);
      mx[h] = fmaxf(mx[h], __shfl_xor(mx[h], mask));
      const float M = fmaxf(m[h], mo);
      const float a = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - M);
      const float b = (mo == -INFINITY) ? 0.f : exp2f(mo - M);
      l[h] = l[h] * a + lo * b;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float ao = __shfl_xor(acc[h][e], mask);
        acc[h][e] = acc[h][e] * a + ao * b;
      }
      m[h] = M;
    }
  }
};

// Sum of x over the LPT consecutive lanes that share a token (LPT a power of
// two), in every one of them.  Groups of up to 16 lanes reduce with DPP
// moves folded into the adds: quad permutations [1,0,3,2] and [2,3,0,1],
// then the row half-mirror (lane i with 7 - i) and the row mirror (i with
// 15 - i), which after the earlier stages pair lanes holding the two halves'
// sums; wider groups finish with shuffles.  Each stage adds the same two
// values in either order, so all lanes of a group end with the same bits.
template <int CTRL>
__device__ inline float add_dpp(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

template <int LPT>
__device__ inline float lane_sum(float x) {
  if constexpr (LPT >= 2) x = add_dpp<0xB1>(x);
  if constexpr (LPT >= 4) x = add_dpp<0x4E>(x);
  if constexpr (LPT >= 8) x = add_dpp<0x141>(x);
  if constexpr (LPT >= 16) x = add_dpp<0x140>(x);
  if constexpr (LPT >= 32) x += __shfl_xor(x, 16);
  if constexpr (LPT >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Codes 2p and 2p+1 (one 2B-bit field) of an LSB-first bit stream.
template <int B>
__device__ inline uint32_t pair_at(const uint32_t *w, int p) {
  constexpr uint32_t kMask = (1u << (2 * B)) - 1u;
  const int o = 2 * B * p, wi = o >> 5, sh = o & 31;
  if (sh + 2 * B <= 32) return (w[wi] >> sh) & kMask;
  return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & kMask;
}

// 2- and 3-bit codes are looked up two at a time: a pair table maps the
// 2B-bit field f of two consecutive codes to (c[f & (2^B - 1)], c[f >> B]),
// replicated over 32 lane slots (entry f of slot s at byte (32 f + s) * 8,
// so the 32 lanes an LDS cycle serves never share a bank).
template <int B>
constexpr int pair_table_bytes() { return (B == 2 || B == 3) ? (1 << (2 * B)) * 32 * 8 : 0; }

typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ inline float2_t pair_entry(const uint8_t *tab, uint32_t f, uint32_t slot8) {
  return *reinterpret_cast<const float2_t *>(tab + ((f << 8) | slot8));
}

// Far tier: packed Lloyd-Max (KB in 2..4) or fp8 (KB = 8) keys, Lloyd-Max values.
// fp8 keys decode in hardware (v_cvt_pk_f32_fp8: OCP E4M3FN, exact in fp32),
// 2- and 3-bit codes through pair tables, 4-bit codes one table read each.
// X = kOutliers: the keys carry an outlier stream; every score gains
// q[idx] . (code * scale) / sqrt(d).  The channels are shared out over the
// token's lanes (channel k on lane k % LPT; qo holds q[idx[k]] pre-scaled
// for the lane's channels, osel their bit offsets in the 8 code bytes), and
// each lane folds scale * sum q . code into its partial before the
// reduction, so the key scale is applied in the lane (key_scale() = 1).
// X = kQjl: the keys carry a QJL sketch; the lane's partial score becomes
// nk * (its codec part) + rho * sum_e (2 z_e - 1) p_e over its DPL sketch
// bits, rho = ||r||_16 sqrt(pi/2)/D and p = S q~ pre-scaled (pq holds 2 p,
// psum the slice's sum of p), so the reduced partial is the whole score.
template <int D, int KB, int VB, int G, int DPL, int X = kNoExtra>
struct FarTier {
  static constexpr bool OUT = X == kOutliers, QJL = X == kQjl;
  static constexpr int kLPT = D / DPL, kOPL = (kOutlierCount + kLPT - 1) / kLPT;   // outlier channels per lane
  static constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  static constexpr int KNB = DPL * KB / 8, VNB = DPL * VB / 8;
  static constexpr bool kKeyPairs = KB == 2 || KB == 3, kValPairs = VB == 2 || VB == 3;
  static constexpr bool kFar = true;
  const uint8_t *krow0, *vrow0;
  const uint16_t *kn0, *vn0;
  const float *lutk, *lutv;
  const uint8_t *pairk, *pairv;
  uint32_t slot8;
  uint32_t kw[(KNB + 3) / 4], vw[(VNB + 3) / 4];
  float nk, nv;
  // outlier stream (OUT only)
  const int8_t *oc0;
  const float *os0;
  float qo[G][OUT ? kOPL : 1];
  uint32_t osel[OUT ? kOPL : 1];
  uint2 oc;
  float osc;
  // QJL sketch (QJL only)
  const uint8_t *zs0;
  const uint16_t *zn0;
  float pq[QJL ? G : 1][QJL ? DPL : 1], psum[QJL ? G : 1];
  uint32_t zw;
  float rho;

  __device__ void load(int t, int ds) {
    load_keys(t, ds);
    load_values(t, ds);
  }
  __device__ void load_keys(int t, int ds) {
    load_slice<KNB>(krow0 + (size_t)t * KROW + ds * KNB, kw);
    nk = (KB == 8) ? 1.f : half_to_float(load_u16(kn0 + t));
    if constexpr (OUT) {
      oc = *reinterpret_cast<const uint2 *>(oc0 + (size_t)t * kOutlierCount);
      osc = os0[t];
    }
    if constexpr (QJL) {
      const uint8_t *zr = zs0 + (size_t)t * (D / 8);
      zw = (DPL == 32) ? reinterpret_cast<const uint32_t *>(zr)[ds]
                       : (DPL == 16) ? (uint32_t)reinterpret_cast<const uint16_t *>(zr)[ds] : (uint32_t)zr[ds];
      rho = half_to_float(zn0[t]) * (1.2533141373155003f / (float)D);   // sqrt(pi/2) / m, m = D
    }
  }
  __device__ void load_values(int t, int ds) {
    load_slice<VNB>(vrow0 + (size_t)t * VROW + ds * VNB, vw);
    nv = half_to_float(load_u16(vn0 + t));
  }
  __device__ void score(const float (&qr)[G][DPL], float (&part)[G]) const {
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = 0.f;
    if constexpr (KB == 8) {
#pragma unroll
      for (int e = 0; e < DPL; e += 2) {
        const float2_t c = (e & 2) ? __builtin_amdgcn_cvt_pk_f32_fp8((int)kw[e >> 2], true)
                                   : __builtin_amdgcn_cvt_pk_f32_fp8((int)kw[e >> 2], false);
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = fmaf(qr[h][e + 1], c.y, fmaf(qr[h][e], c.x, part[h]));
      }
    } else if constexpr (kKeyPairs) {
#pragma unroll
      for (int e = 0; e < DPL; e += 2) {
        const float2_t c = pair_entry(pairk, pair_at<KB>(kw, e >> 1), slot8);
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = fmaf(qr[h][e + 1], c.y, fmaf(qr[h][e], c.x, part[h]));
      }
    } else if constexpr (KB == 4 && DPL % 8 == 0) {
#pragma unroll
      for (int i = 0; i < DPL / 8; ++i) {
        uint32_t o[8];
        nibble_offsets(kw[i], o);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float c = table_at(lutk, o[u]);
#pragma unroll
          for (int h = 0; h < G; ++h) part[h] = fmaf(qr[h][8 * i + u], c, part[h]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float c = lutk[code_at<KB>(kw, e)];
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = fmaf(qr[h][e], c, part[h]);
      }
    }
    if constexpr (QJL) {
      float a[G];
#pragma unroll
      for (int h = 0; h < G; ++h) a[h] = -psum[h];
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float b = (float)((zw >> e) & 1u);
#pragma unroll
        for (int h = 0; h < G; ++h) a[h] = fmaf(pq[h][e], b, a[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] = fmaf(rho, a[h], part[h] * nk);
    }
    if constexpr (OUT) {
      float c[kOPL];
#pragma unroll
      for (int u = 0; u < kOPL; ++u) {
        const uint32_t w = (osel[u] < 32u) ? oc.x : oc.y;
        c[u] = (float)(int8_t)((w >> (osel[u] & 31u)) & 0xFFu);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < kOPL; ++u) a = fmaf(qo[h][u], c[u], a);
        part[h] = fmaf(osc, a, part[h] * nk);
      }
    }
  }
  __device__ float key_scale() const { return (QJL || OUT) ? 1.f : nk; }
  __device__ void accumulate(const float (&p)[G], State<G, DPL> &st) const {
    float w[G];
#pragma unroll
    for (int h = 0; h < G; ++h) w[h] = p[h] * nv;
    if constexpr (kValPairs) {
#pragma unroll
      for (int e = 0; e < DPL; e += 2) {
        const float2_t c = pair_entry(pairv, pair_at<VB>(vw, e >> 1), slot8);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          st.acc[h][e] = fmaf(w[h], c.x, st.acc[h][e]);
          st.acc[h][e + 1] = fmaf(w[h], c.y, st.acc[h][e + 1]);
        }
      }
    } else if constexpr (VB == 4 && DPL % 8 == 0) {
#pragma unroll
      for (int i = 0; i < DPL / 8; ++i) {
        uint32_t o[8];
        nibble_offsets(vw[i], o);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float c = table_at(lutv, o[u]);
#pragma unroll
          for (int h = 0; h < G; ++h) st.acc[h][8 * i + u] = fmaf(w[h], c, st.acc[h][8 * i + u]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float c = lutv[code_at<VB>(vw, e)];
#pragma unroll
        for (int h = 0; h < G; ++h) st.acc[h][e] = fmaf(w[h], c, st.acc[h][e]);
      }
    }
  }
};

// Near tier: exact fp16 rows in the original domain.
template <int D, int G, int DPL>
struct NearTier {
  static constexpr bool kFar = false;
  static constexpr int NB = DPL * 2;
  const uint8_t *krow0, *vrow0;
  uint32_t kw[NB / 4], vw[NB / 4];

  __device__ void load(int t, int ds) {
    load_slice<NB>(krow0 + (size_t)t * D * 2 + ds * NB, kw);
    load_slice<NB>(vrow0 + (size_t)t * D * 2 + ds * NB, vw);
  }
  __device__ static float elem(const uint32_t *w, int e) { return half_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu); }
  __device__ void score(const float (&qr)[G][DPL], float (&part)[G]) const {
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float k = elem(kw, e);
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] = fmaf(qr[h][e], k, part[h]);
    }
  }
  __device__ float key_scale() const { return 1.f; }
  __device__ void accumulate(const float (&p)[G], State<G, DPL> &st) const {
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float v = elem(vw, e);
#pragma unroll
      for (int h = 0; h < G; ++h) st.acc[h][e] = fmaf(p[h], v, st.acc[h][e]);
    }
  }
};

// Online softmax over tokens [t0, t1): each lane slot takes every TPB-th
// token.  On entry cur holds the lane's row of the first block (first_block,
// issued before the query prologue so that round trip overlaps it); the
// next block's rows are requested before this block's arithmetic, so one
// block is in flight while a wave computes.  (Buffers kept in fixed
// registers by unrolling two blocks per iteration need no copies, but the
// scheduler then interleaves the two blocks and the kernel needs 20-30 more
// VGPRs, a wave per SIMD fewer.)
template <int G, int DPL, int LPT, typename Tier>
__device__ void token_loop(Tier &cur, const float (&qr)[G][DPL], State<G, DPL> &st, int t0, int t1) {
  constexpr int TPW = 64 / LPT;
  constexpr int TPB = TPW * kWaves;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ds = lane % LPT, ts = lane / LPT;
  int t = t0 + wave * TPW + ts;
  for (int base = t0; base < t1; base += TPB) {
    const bool valid = t < t1;
    const int tn = t + TPB;
    Tier nxt = cur;
    nxt.load(tn < t1 ? tn : t0, ds);
    float part[G];
    cur.score(qr, part);
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = lane_sum<LPT>(part[h]);
    float s[G], p[G];
    const float ks = cur.key_scale();
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = valid ? part[h] * ks : -INFINITY;
    st.add_scores(s, p);
    cur.accumulate(p, st);
    cur = nxt;
    t = tn;
  }
}

// Loads the lane's row of the first block of [t0, t1) into X (see token_loop).
template <int LPT, typename Tier>
__device__ void first_block(Tier &X, int t0, int t1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = t0 + wave * (64 / LPT) + lane / LPT;
  if (t0 < t1) X.load(t < t1 ? t : t0, lane % LPT);
}

// Spike flags of one block: head h's bit of each of the wave's TPW tokens
// (tw its first) whose score is above fg.spike[h], or-ed into the head's
// flag words.
template <int G, int LPT>
__device__ inline void spike_flags(const FarGate<G> &fg, const float (&s)[G], int tw, int ds, int lane) {
  constexpr int TPW = 64 / LPT;
  if (!fg.bits) return;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint64_t ball = __builtin_amdgcn_ballot_w64(ds == 0 && s[h] > fg.spike[h]);
    uint32_t m = 0u;
#pragma unroll
    for (int k = 0; k < TPW; ++k) m |= (uint32_t)((ball >> (k * LPT)) & 1ull) << k;
    if (m != 0u && lane == 0) atomicOr(fg.bits + (size_t)h * fg.words + (tw >> 5), m << (tw & 31));
  }
}

// Gated pass while nothing is gated: the ungated loop's schedule (a block's
// key and value rows requested together, one block ahead of its
// arithmetic), with the gate applied to the weights and the spike flags
// set.  A wave leaves it after the first block in which some lane slot's
// token is gated for every head, and returns where the rest of its range
// starts (t1 if it got through): from there token_loop_gated requests only
// the value rows some head keeps.  A pass that gates nothing so streams
// like the ungated one.
template <int G, int DPL, int LPT, typename Tier>
__device__ int token_loop_spec(Tier &cur, const float (&qr)[G][DPL], State<G, DPL> &st, int t0, int t1,
                               const FarGate<G> &fg) {
  constexpr int TPW = 64 / LPT;
  constexpr int TPB = TPW * kWaves;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ds = lane % LPT, ts = lane / LPT;
  int t = t0 + wave * TPW + ts;
  for (int base = t0; base < t1; base += TPB) {
    const bool valid = t < t1;
    const int tn = t + TPB;
    Tier nxt = cur;
    nxt.load(tn < t1 ? tn : t0, ds);
    float part[G];
    cur.score(qr, part);
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = lane_sum<LPT>(part[h]);
    float s[G], p[G];
    const float ks = cur.key_scale();
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = valid ? part[h] * ks : -INFINITY;
    spike_flags<G, LPT>(fg, s, t - ts, ds, lane);
    st.add_scores(s, p);
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool keep = s[h] >= fg.gate[h];
      p[h] = keep ? p[h] : 0.f;
      any = any || keep;
    }
    cur.accumulate(p, st);
    cur = nxt;
    t = tn;
    if (__builtin_amdgcn_ballot_w64(valid && !any) != 0ull) return base + TPB;
  }
  return t1;
}

// Far-tier loop with the score gate and spike flags.  A token whose score is
// below fg.gate[h] keeps its weight in l but adds nothing to head h's
// values; a lane slot whose token every head gates does not even load its
// value row (the value loads of a block go out after the block's scores,
// and are accumulated one block later, before the next block's softmax
// update, so the running state they were weighted against still holds).
// Flags of tokens scoring above fg.spike[h] are or-ed into head h's words
// (a wave's TPW consecutive tokens never straddle a 32-token word: blocks
// start at multiples of 32).  Two tier buffers alternate so no register
// with a load in flight is ever copied.
template <int G, int DPL, int LPT, typename Tier>
__device__ void token_loop_gated(const Tier &proto, const float (&qr)[G][DPL], State<G, DPL> &st, int t0, int t1,
                                 const FarGate<G> &fg) {
  constexpr int TPW = 64 / LPT;
  constexpr int TPB = TPW * kWaves;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ds = lane % LPT, ts = lane / LPT;
  if (t0 >= t1) return;
  auto row = [&](int t) { return t < t1 ? t : t0; };
  // one block: X has its keys loaded; Y holds the previous block's values
  // (pending, weights py) and takes the next block's keys
  auto block = [&](Tier &X, Tier &Y, float (&px)[G], const float (&py)[G], bool &vx, bool vy, int t) {
    Y.load_keys(row(t + TPB), ds);
    float part[G];
    X.score(qr, part);
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = lane_sum<LPT>(part[h]);
    const bool valid = t < t1;
    float s[G];
    const float ks = X.key_scale();
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = valid ? part[h] * ks : -INFINITY;
    if (vy) Y.accumulate(py, st);
    spike_flags<G, LPT>(fg, s, t - ts, ds, lane);
    st.add_scores(s, px);
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool keep = s[h] >= fg.gate[h];
      px[h] = keep ? px[h] : 0.f;
      any = any || keep;
    }
    if (any) X.load_values(row(t), ds);
    vx = any;
  };
  Tier A = proto, B = proto;
  float pa[G], pb[G];
#pragma unroll
  for (int h = 0; h < G; ++h) pa[h] = pb[h] = 0.f;
  bool va = false, vb = false;
  int t = t0 + wave * TPW + ts;
  A.load_keys(row(t), ds);
  for (int base = t0; base < t1; base += 2 * TPB) {
    block(A, B, pa, pb, va, vb, t);
    t += TPB;
    if (base + TPB >= t1) {
      if (va) A.accumulate(pa, st);
      return;
    }
    block(B, A, pb, pa, vb, va, t);
    t += TPB;
  }
  if (vb) B.accumulate(pb, st);
}

// Query rows hkv*G .. hkv*G+G-1 of batch entry b into qs, sign-flipped and
// Walsh-Hadamard transformed when `rotate` (far splits).  Wave 0 does it in
// registers: lane i holds coordinates i*E .. i*E+E-1 (E = D/64) of each
// row, the butterflies of stride below E run inside the lane and the others
// across lanes by DPP and permlane swaps (no LDS round trip, no barrier per
// stage); the other waves go on with their own prologue work.  The caller's
// barrier publishes qs.
template <int D, int G>
__device__ void query_rows(const Params &P, int b, int hkv, bool rotate, float (*qs)[D]) {
  constexpr int E = D / 64;
  if ((threadIdx.x >> 6) != 0) return;
  const int lane = threadIdx.x & 63;
  float v[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t row = ((size_t)b * P.q_heads + hkv * G + h) * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e)
      v[h][e] = P.q_f16 ? half_to_float(static_cast<const uint16_t *>(P.q)[row + e])
                        : static_cast<const float *>(P.q)[row + e];
  }
  if (rotate) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool neg = P.signs[lane * E + e] < 0;
#pragma unroll
      for (int h = 0; h < G; ++h) v[h][e] = neg ? -v[h][e] : v[h][e];
    }
#pragma unroll
    for (int len = 1; len < E; len <<= 1) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (e & len) continue;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float x = v[h][e], y = v[h][e + len];
          v[h][e] = x + y;
          v[h][e + len] = x - y;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) v[h][e] = fwht_lanes(v[h][e], lane);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < E; ++e) qs[h][lane * E + e] = v[h][e];
  }
}

// The lane's DPL query coordinates (slice ds), pre-scaled.
template <int D, int G, int DPL>
__device__ void lane_query(const float (*qs)[D], float scale, float (&qr)[G][DPL]) {
  const int ds = (threadIdx.x & 63) % (D / DPL);
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) qr[h][e] = qs[h][ds * DPL + e] * scale;
  }
}

// Merges the lane slots of each wave, then the four waves, and writes the
// split's normalised partial output and its (m, l).
template <int D, int G, int DPL>
__device__ void write_split(const Params &P, State<G, DPL> &st, int b, int hkv, int split,
                            float (*red_ml)[G][3], float (*red_acc)[G][D]) {
  constexpr int LPT = D / DPL;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ds = lane % LPT;
  const int total_splits = P.num_near_splits + P.num_splits;
#pragma unroll
  for (int m = LPT; m < 64; m <<= 1) st.merge_xor(m);
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) red_acc[wave][h][ds * DPL + e] = st.acc[h][e];
      if (lane == 0) {
        red_ml[wave][h][0] = st.m[h];
        red_ml[wave][h][1] = st.l[h];
        red_ml[wave][h][2] = st.mx[h];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kBlock) {
    const int h = i / D, j = i - (i / D) * D;
    float M = -INFINITY, MX = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      M = fmaxf(M, red_ml[w][h][0]);
      MX = fmaxf(MX, red_ml[w][h][2]);
    }
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = red_ml[w][h][0];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      l += red_ml[w][h][1] * f;
      o += red_acc[w][h][j] * f;
    }
    const size_t row = ((size_t)b * P.q_heads + hkv * G + h) * total_splits + split;
    P.part_o[row * D + j] = (l > 0.f) ? o / l : 0.f;
    if (j == 0) {
      // l restated against the split maximum: M <= MX <= M + kSlack
      P.part_ml[row * 2 + 0] = (MX == -INFINITY) ? -INFINITY : MX * kLn2;
      P.part_ml[row * 2 + 1] = (MX == -INFINITY) ? 0.f : l * exp2f(M - MX);
    }
  }
}

// NEAR: the launch has near-tier splits (without them the kernel carries no
// registers for the near path).
// GATED: score gate and spike flags; X: key side stream (none, outliers, QJL).
// WPE: waves per SIMD the register allocation must leave room for (1: no
// constraint).
template <int D, int KB, int VB, int G, bool NEAR, bool GATED, int X = kNoExtra, int WPE = 1>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(WPE))) void attend_kernel(Params P) {
  constexpr bool OUT = X == kOutliers, QJL = X == kQjl;
  // Coordinates per lane.  G = 1 without a near tier: 32 (two 16-byte fp8
  // or 32-bit-code slices per token, half the per-token softmax lanes of
  // 16); with one, 16 on both tiers (near-tier fp16 rows would double the
  // buffered registers at 32, and 32 on the far splits alone measured slower
  // on the two-tier cache, 163.7 against 158.3 us); G >= 4 with a near tier
  // (where the far codes allow whole-word slices): 8 on both, so the near
  // rows' fp16 slices and the G x DPL arrays leave room for three or four
  // waves per SIMD (the decode-buffer launch: 27.5 -> 25.5 us; on far-only
  // launches the extra reduction round and the softmax repeated over twice
  // the lanes cost more than the occupancy gains); 16 otherwise.
  constexpr int DPLN = (NEAR && G >= 4 && KB != 3 && VB != 3) ? 8 : 16;
  constexpr int DPLF = (G == 1 && !NEAR) ? 32 : DPLN;
  constexpr int LPTN = D / DPLN, LPTF = D / DPLF;
  static_assert(LPTF >= 1 && LPTN <= 64, "lane mapping");

  __shared__ float qs[G][D];
  constexpr int kPairK = pair_table_bytes<KB>(), kPairV = pair_table_bytes<VB>();
  __shared__ float lutk[16];
  __shared__ float lutv[16];
  __shared__ __attribute__((aligned(16))) uint8_t pairtab[(kPairK + kPairV) > 0 ? kPairK + kPairV : 16];
  __shared__ float red_ml[kWaves][G][3];
  __shared__ float red_acc[kWaves][G][D];
  __shared__ float ps[QJL ? G : 1][QJL ? D : 1];

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / P.kv_heads, hkv = bh - b * P.kv_heads;

  if constexpr (NEAR) {
    if (split < P.num_near_splits) {
      const int chunk = ((P.near_len + P.num_near_splits - 1) / P.num_near_splits + 31) / 32 * 32;
      const int t0 = min(P.near_len, split * chunk), t1 = min(P.near_len, t0 + chunk);
      NearTier<D, G, DPLN> tier;
      const size_t base = (size_t)bh * P.near_len * D * 2;
      tier.krow0 = reinterpret_cast<const uint8_t *>(P.near_k) + base;
      tier.vrow0 = reinterpret_cast<const uint8_t *>(P.near_v) + base;
      first_block<LPTN>(tier, t0, t1);
      query_rows<D, G>(P, b, hkv, false, qs);
      __syncthreads();
      float qr[G][DPLN];
      lane_query<D, G, DPLN>(qs, kLog2e / sqrtf((float)D), qr);
      State<G, DPLN> st;
      st.init();
      token_loop<G, DPLN, LPTN>(tier, qr, st, t0, t1);
      write_split<D, G, DPLN>(P, st, b, hkv, split, red_ml, red_acc);
      return;
    }
  }

  // ---- far split ----
  const int fs = split - P.num_near_splits;
  const int chunk = ((P.seq_len + P.num_splits - 1) / P.num_splits + 31) / 32 * 32;
  const int t0 = min(P.seq_len, fs * chunk), t1 = min(P.seq_len, t0 + chunk);
  using Far = FarTier<D, KB, VB, G, DPLF, X>;
  Far tier;
  tier.krow0 = P.k_codes + (size_t)bh * P.capacity * (D * KB / 8);
  tier.vrow0 = P.v_codes + (size_t)bh * P.capacity * (D * VB / 8);
  tier.kn0 = P.k_norms + (size_t)bh * P.capacity;
  tier.vn0 = P.v_norms + (size_t)bh * P.capacity;
  tier.lutk = lutk;
  tier.lutv = lutv;
  tier.pairk = pairtab;
  tier.pairv = pairtab + kPairK;
  tier.slot8 = (uint32_t)(tid & 31) * 8;
  if constexpr (OUT) {
    tier.oc0 = P.out_codes + (size_t)bh * P.capacity * kOutlierCount;
    tier.os0 = P.out_scales + (size_t)bh * P.capacity;
  }
  if constexpr (QJL) {
    tier.zs0 = P.qjl_signs + (size_t)bh * P.capacity * (D / 8);
    tier.zn0 = P.qjl_norms + (size_t)bh * P.capacity;
  }
  first_block<LPTF>(tier, t0, t1);

  // ---- rotated query into LDS, centroid tables ----
  query_rows<D, G>(P, b, hkv, true, qs);
  if (KB != 8 && tid < (1 << KB)) lutk[tid] = P.k_centroids[tid];
  if (tid < (1 << VB)) lutv[tid] = P.v_centroids[tid];
  // pair tables: entry (c[f & m], c[f >> B]) of field f in 32 slots
  if constexpr (kPairK > 0) {
    for (int i = tid; i < kPairK / 8; i += kBlock) {
      const int f = i >> 5;
      *reinterpret_cast<float2_t *>(pairtab + i * 8) =
          (float2_t){P.k_centroids[f & ((1 << KB) - 1)], P.k_centroids[f >> KB]};
    }
  }
  if constexpr (kPairV > 0) {
    for (int i = tid; i < kPairV / 8; i += kBlock) {
      const int f = i >> 5;
      *reinterpret_cast<float2_t *>(pairtab + kPairK + i * 8) =
          (float2_t){P.v_centroids[f & ((1 << VB) - 1)], P.v_centroids[f >> VB]};
    }
  }
  __syncthreads();

  const float prescale = kLog2e / (float)D;
  if constexpr (QJL) {
    // p = S (q~ pre-scaled) per head.  Thread t takes the four columns
    // 4c..4c+3 of S^T (c = t % (D/4), one 16-byte load per row) over its
    // range of rows (t / (D/4)), sixteen loads in flight; the ranges of a
    // wave are summed by shuffles, the four waves' sums through red_acc
    // (unused until the epilogue), in a fixed order.
    constexpr int CG = D / 4, R = kBlock / CG, JR = D / R, JC = JR < 16 ? JR : 16;
    const int c = tid % CG, r = tid / CG;
    float acc[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.f;
    const float4 *col = reinterpret_cast<const float4 *>(P.qjl_proj) + c;
    for (int j0 = r * JR; j0 < (r + 1) * JR; j0 += JC) {
      float4 sv[JC];
#pragma unroll
      for (int u = 0; u < JC; ++u) sv[u] = col[(size_t)(j0 + u) * CG];
#pragma unroll
      for (int u = 0; u < JC; ++u) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float qv = qs[h][j0 + u];
          acc[h][0] = fmaf(sv[u].x, qv, acc[h][0]);
          acc[h][1] = fmaf(sv[u].y, qv, acc[h][1]);
          acc[h][2] = fmaf(sv[u].z, qv, acc[h][2]);
          acc[h][3] = fmaf(sv[u].w, qv, acc[h][3]);
        }
      }
    }
    const int lane0 = tid & 63, wave0 = tid >> 6;
#pragma unroll
    for (int m = CG; m < 64; m <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[h][e] += __shfl_xor(acc[h][e], m);
      }
    }
    if (lane0 < CG) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        *reinterpret_cast<float4 *>(&red_acc[wave0][h][4 * c]) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
    }
    __syncthreads();
    for (int o = tid; o < G * D; o += kBlock) {
      const int h = o / D, i = o - (o / D) * D;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red_acc[w][h][i];
      ps[h][i] = v * prescale;
    }
    __syncthreads();
  }

  const int ds = (tid & 63) % LPTF;
  float qr[G][DPLF];
  lane_query<D, G, DPLF>(qs, prescale, qr);
  if constexpr (QJL) {
    float pq[G][DPLF], psum[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < DPLF; ++e) {
        const float v = ps[h][ds * DPLF + e];
        pq[h][e] = 2.f * v;
        sum += v;
      }
      psum[h] = sum;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      tier.psum[h] = psum[h];
#pragma unroll
      for (int e = 0; e < DPLF; ++e) tier.pq[h][e] = pq[h][e];
    }
  }
  if constexpr (OUT) {
    // the query at the outlier channels (original domain), scaled to log2 units of s
    // the lane's channels k = ds + LPT u (< 8); others get q = 0
    const float sc = kLog2e / sqrtf((float)D);
    const int32_t *oi = P.out_idx + (size_t)bh * kOutlierCount;
    constexpr int kOPL = Far::kOPL;
#pragma unroll
    for (int u = 0; u < kOPL; ++u) {
      const int k = ds + LPTF * u;
      const bool has = k < kOutlierCount;
      const int c = has ? oi[k] : 0;
      const uint32_t sel = has ? (uint32_t)(8 * k) : 0u;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const size_t qrow = ((size_t)b * P.q_heads + hkv * G + h) * D;
        const float v = P.q_f16 ? half_to_float(static_cast<const uint16_t *>(P.q)[qrow + c])
                                : static_cast<const float *>(P.q)[qrow + c];
        tier.qo[h][u] = has ? v * sc : 0.f;
      }
      tier.osel[u] = sel;
    }
  }

  State<G, DPLF> st;
  st.init();
  if constexpr (GATED) {
    constexpr float kGate2 = 16.f * kLog2e;     // e^-16 in log2 units
    FarGate<G> fg;
    const size_t row0 = (size_t)b * P.q_heads + (size_t)hkv * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      fg.gate[h] = P.gate_ref ? P.gate_ref[row0 + h] * kLog2e - kGate2 : -INFINITY;
      fg.spike[h] = P.spike_ref ? P.spike_ref[row0 + h] * kLog2e : INFINITY;
    }
    fg.bits = P.spike_ref ? P.spike_bits + row0 * P.spike_words : nullptr;
    fg.words = P.spike_words;
    const int resume = token_loop_spec<G, DPLF, LPTF>(tier, qr, st, t0, t1, fg);
    if (resume < t1) token_loop_gated<G, DPLF, LPTF>(tier, qr, st, resume, t1, fg);
  } else {
    token_loop<G, DPLF, LPTF>(tier, qr, st, t0, t1);
  }
  write_split<D, G, DPLF>(P, st, b, hkv, split, red_ml, red_acc);
}

template <int D, int KB, int VB, int G>
hipError_t go(const AttendArgs &a, hipStream_t stream) {
  Params P{a.q, a.q_f16, a.kv_heads, a.q_heads, a.capacity, a.seq_len, a.num_splits, a.num_near_splits,
           a.near_len, a.k_codes, a.v_codes, a.k_norms, a.v_norms, a.signs, a.k_centroids, a.v_centroids,
           a.near_k, a.near_v, a.part_o, a.part_ml, a.gate_ref, a.spike_ref, a.spike_bits, (a.seq_len + 31) / 32,
           a.outlier_idx, a.outlier_codes, a.outlier_scales, a.qjl_proj, a.qjl_signs, a.qjl_norms};
  dim3 grid(a.near_only ? a.num_near_splits : a.num_near_splits + a.num_splits, a.batch * a.kv_heads);
  const bool near = a.num_near_splits > 0, gated = a.gated != 0;
  if constexpr (KB != 8) {
    if (a.qjl_proj) {
      if (near) hipLaunchKernelGGL((attend_kernel<D, KB, VB, G, true, false, kQjl>), grid, dim3(kBlock), 0, stream, P);
      else hipLaunchKernelGGL((attend_kernel<D, KB, VB, G, false, false, kQjl>), grid, dim3(kBlock), 0, stream, P);
      return hipGetLastError();
    }
    if (a.outlier_idx) {
      if (near) {
        hipLaunchKernelGGL((attend_kernel<D, KB, VB, G, true, false, kOutliers>), grid, dim3(kBlock), 0, stream, P);
      } else {
        hipLaunchKernelGGL((attend_kernel<D, KB, VB, G, false, false, kOutliers>), grid, dim3(kBlock), 0, stream, P);
      }
      return hipGetLastError();
    }
  }
  // G = 1 with a near tier (8 or 16 coordinates per lane), ungated, fits six
  // waves per SIMD in 80 registers without spilling (two_tier 155.7 ->
  // 153.4 us); its natural allocation, 88 registers, leaves room for five.
  // The gated loop would spill there and keeps its allocation.
  constexpr int kNearWaves = G == 1 ? 6 : 1;
  if (near && gated) hipLaunchKernelGGL((attend_kernel<D, KB, VB, G, true, true>), grid, dim3(kBlock), 0, stream, P);
  else if (near)
    hipLaunchKernelGGL((attend_kernel<D, KB, VB, G, true, false, kNoExtra, kNearWaves>), grid, dim3(kBlock), 0, stream,
                       P);
  else if (gated) hipLaunchKernelGGL((attend_kernel<D, KB, VB, G, false, true>), grid, dim3(kBlock), 0, stream, P);
  else hipLaunchKernelGGL((attend_kernel<D, KB, VB, G, false, false>), grid, dim3(kBlock), 0, stream, P);
  return hipGetLastError();
}

// Query groups the VALU kernel is instantiated for: 1, 2 and 4 (3-bit
// values: 1 only).
bool valu_group_built(int G, int v_format) { return G == 1 || (v_format != 3 && (G == 2 || G == 4)); }

bool valu_formats_built(int kf, int vf) {
  return (kf == 2 && vf == 2) || (kf == 3 && vf == 3) || (kf == 4 && vf == 4) || (kf == 3 && vf == 4) ||
         (kf == 8 && vf == 4);
}

bool valu_attend_supported(const AttendArgs &a) {
  return (a.head_dim == 64 || a.head_dim == 128 || a.head_dim == 256) && a.q_heads % a.kv_heads == 0 &&
         valu_group_built(a.q_heads / a.kv_heads, a.v_format) && valu_formats_built(a.k_format, a.v_format);
}

template <int D, int KB, int VB>
hipError_t by_group(const AttendArgs &a, hipStream_t stream, bool *ok) {
  const int G = a.q_heads / a.kv_heads;
  if (G == 1) return go<D, KB, VB, 1>(a, stream);
  if constexpr (VB != 3) {
    if (G == 2) return go<D, KB, VB, 2>(a, stream);
    if (G == 4) return go<D, KB, VB, 4>(a, stream);
  }
  *ok = false;
  return hipSuccess;
}

template <int D>
hipError_t by_format(const AttendArgs &a, hipStream_t stream, bool *ok) {
  const int kf = a.k_format, vf = a.v_format;
  if (kf == 2 && vf == 2) return by_group<D, 2, 2>(a, stream, ok);
  if (kf == 3 && vf == 3) return by_group<D, 3, 3>(a, stream, ok);
  if (kf == 4 && vf == 4) return by_group<D, 4, 4>(a, stream, ok);
  if (kf == 3 && vf == 4) return by_group<D, 3, 4>(a, stream, ok);
  if (kf == 8 && vf == 4) return by_group<D, 8, 4>(a, stream, ok);
  *ok = false;
  return hipSuccess;
}

hipError_t launch_valu(const AttendArgs &a, hipStream_t stream, bool *supported) {
  *supported = true;
  switch (a.head_dim) {
    case 64: return by_format<64>(a, stream, supported);
    case 128: return by_format<128>(a, stream, supported);
    case 256: return by_format<256>(a, stream, supported);
  }
  *supported = false;
  return hipSuccess;
}

// The far tier of a cache with a near tier, as a launch of its own: no near
// splits, partial rows starting at the first far split.
AttendArgs far_part(const AttendArgs &a) {
  AttendArgs f = a;
  f.num_near_splits = 0;
  f.near_len = 0;
  f.near_k = f.near_v = nullptr;
  return f;
}

}  // namespace

const char *attend_kernel_name(const AttendArgs &a) {
  // NULL where launch_attend would return KVQ_EUNSUPPORTED
  const char *valu = valu_attend_supported(a) ? "attend_kernel" : nullptr;
  if (a.qjl_proj || a.outlier_idx)
    return (a.num_near_splits == 0 && wide_attend_supported(a)) ? "attend_wide_kernel" : valu;
  if (a.num_near_splits > 0) {
    if (pair_near_supported(a)) return "attend_pair_kernel";
    const AttendArgs f = far_part(a);
    if (pair_attend_supported(f)) return valu ? "attend_pair_kernel+attend_kernel" : nullptr;
    if (wide_attend_supported(f)) return valu ? "attend_wide_kernel+attend_kernel" : nullptr;
  }
  if (pair_attend_supported(a)) return "attend_pair_kernel";
  if (wide_attend_supported(a)) return "attend_wide_kernel";
  if (mfma_attend_supported(a)) return "attend_mfma_kernel";
  return valu;
}

hipError_t launch_attend_gated(const AttendArgs &a, hipStream_t stream, bool *supported) {
  AttendArgs g = a;
  g.gated = 1;
  return launch_valu(g, stream, supported);
}

hipError_t launch_attend(const AttendArgs &a, hipStream_t stream, bool *supported) {
  // Key side streams: the outlier stream beside 4-bit codes and the QJL
  // sketch beside 3-bit keys and 4-bit values (G >= 2), both at d = 128
  // without a near tier, on the two-wave-per-SIMD matrix-core kernel;
  // otherwise on the VALU kernel.
  if (a.qjl_proj || a.outlier_idx) {
    if (a.num_near_splits == 0 && wide_attend_supported(a)) {
      *supported = true;
      return launch_attend_wide(a, stream);
    }
    return launch_valu(a, stream, supported);
  }
  // A near tier (fp16 rows, original domain) beside 4-bit codes at d = 128:
  // both tiers in one launch of the pair-table kernel.  Beside other codes
  // that a pair-table kernel covers: the near splits run on the VALU kernel
  // and the far splits on the pair-table kernel, two launches on the stream
  // writing disjoint partial rows.
  if (a.num_near_splits > 0) {
    if (pair_near_supported(a)) {
      *supported = true;
      return launch_attend_pair(a, stream);
    }
    const AttendArgs f = far_part(a);
    const bool pair = pair_attend_supported(f), wide = !pair && wide_attend_supported(f);
    if (pair || wide) {
      AttendArgs n = a;
      n.near_only = 1;
      const hipError_t e = launch_valu(n, stream, supported);
      if (e != hipSuccess || !*supported) return e;
      return pair ? launch_attend_pair(f, stream, a.num_near_splits) : launch_attend_wide(f, stream, a.num_near_splits);
    }
  }
  if (pair_attend_supported(a)) {
    *supported = true;
    return launch_attend_pair(a, stream);
  }
  if (wide_attend_supported(a)) {
    *supported = true;
    return launch_attend_wide(a, stream);
  }
  if (mfma_attend_supported(a)) return launch_attend_mfma(a, stream, supported);
  return launch_valu(a, stream, supported);
}

}  // namespace kvq
