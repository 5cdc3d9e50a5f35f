// Split-K GQA decode attention on packed Lloyd-Max codes, matrix-core version
// for gfx950 (v_mfma_f32_16x16x32_f16, fp32 accumulation).
//
// Why matrix cores: one KV head serves G query heads, so scoring a tile of
// tokens is a [16 tokens x d] x [d x G] product and the value update a
// [G x 16 tokens] x [16 tokens x d] product.  Done with fp32 vector FMAs
// that is 2*G multiply-adds per 4-bit code, more than the vector units can
// issue at HBM rate; on the matrix cores the remaining vector work per code is
// one table address and one LDS read.
//
// Exactness: every fp32 factor enters as a pair of fp16 halves (hi = RN(x),
// lo = RN(x - hi)), giving about 22 significant bits:
//   keys    A operand k-slot pair (2p, 2p+1) = (c_hi, c_lo) of one coordinate,
//           B columns 0..7 = (z_hi, z_hi) per head, columns 8..15 = (z_lo, 0),
//           so column h + column h+8 = c_hi z_hi + c_lo z_hi + c_hi z_lo;
//   values  B operand k-slot pair = (c_hi, c_lo) of one token's coordinate,
//           A rows 0..7 = (w_hi, w_hi) per head, rows 8..15 = (w_lo, w_lo),
//           row h + row h+8 = (w_hi + w_lo)(c_hi + c_lo),
// where z is the query after sign flip and Walsh-Hadamard transform, c the
// centroid, w = exp2(score - max) * value norm.  Each LDS table entry holds a
// centroid's (hi, lo) pair, so one 32-bit lookup is one operand register.
//
// Work mapping: grid (split, b * Hkv); 4 waves per work-group, each wave
// walking 16-token tiles of the split; one tile = 1 KB of key codes loaded as
// one 16-byte slice per lane (d=128, 4-bit).  Lane (g, n) = (lane / 16,
// lane % 16): its key slice is token n, coordinates [g*d/4, (g+1)*d/4); its
// scores are tokens 4g..4g+3 for head n % 8; its value codes are tokens
// 4g..4g+3, coordinates [n*d/16, (n+1)*d/16).
// Sources: "The Engineering Behind AdapTQ", "Engineering the Hot Path"
// (rotate q once, score from codes through a table, no dequantize pass);
// "FoveatedKV", "Making it fast" (split-K, q pre-scaled, online softmax with
// one exp per score).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kTile = 16;
constexpr int kGMax = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kCodeScale = 256.f;   // centroid scale: keeps the low fp16 half a normal number

struct MParams {
  const void *q;
  int q_f16;
  int kv_heads, q_heads, capacity, seq_len, num_splits;
  const uint8_t *k_codes, *v_codes;
  const uint16_t *k_norms, *v_norms;
  const int8_t *signs;
  const float *k_centroids, *v_centroids;
  float *part_o, *part_ml;
};

__device__ inline uint32_t pack2(_Float16 a, _Float16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ inline half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint4_t v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

// (hi, lo) fp16 split of x: hi = RN(x), lo = RN(x - hi).
__device__ inline uint32_t split_entry(float x) {
  const _Float16 hi = (_Float16)x;
  return pack2(hi, (_Float16)(x - (float)hi));
}

__device__ inline float half_value(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }

template <int NB>
__device__ inline void load_bytes(const uint8_t *p, uint32_t (&w)[(NB + 3) / 4]) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (NB % 8 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 8; ++i) {
      const uint2 v = reinterpret_cast<const uint2 *>(p)[i];
      w[2 * i] = v.x; w[2 * i + 1] = v.y;
    }
  } else if constexpr (NB % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) w[i] = reinterpret_cast<const uint32_t *>(p)[i];
  } else {
    static_assert(NB == 2, "slice size");
    w[0] = *reinterpret_cast<const uint16_t *>(p);
  }
}

// (byte K of v) * 4 in one VALU op: SDWA selects the byte as the shifted
// operand.  Used to turn a byte holding one code into an LDS table offset.
template <int K>
__device__ inline uint32_t byte_x4(uint32_t v) {
  uint32_t r;
  if constexpr (K == 0) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(v));
  if constexpr (K == 1) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(v));
  if constexpr (K == 2) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(v));
  if constexpr (K == 3) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(v));
  return r;
}

// The codes of one 32-bit word split into byte planes: plane k holds codes
// k, k+P, k+2P, k+3P (P = codes per byte), one per byte, so each code's table
// offset is a single byte_x4.
template <int B>
struct CodePlanes {
  static constexpr int P = 8 / B;
  uint32_t pl[P];
  __device__ void set(uint32_t w) {
    constexpr uint32_t M = (B == 4) ? 0x0F0F0F0Fu : 0x03030303u;
#pragma unroll
    for (int k = 0; k < P; ++k) pl[k] = (w >> (B * k)) & M;
  }
  template <int E>
  __device__ uint32_t addr() const { return byte_x4<E / P>(pl[E % P]); }
};

__device__ inline uint32_t lut_read(const uint32_t *lut, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lut) + byte_addr);
}

// xor-8 exchange inside a row of 16 lanes (DPP row rotate by 8).
__device__ inline float row_swap8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

template <int KB, int NW, int E = 0>
__device__ inline void key_scores_word(const CodePlanes<KB> &cp, const uint32_t (*bk)[4], const uint32_t *lutk,
                                       float4_t &dk, int kb0) {
  constexpr int KCW = 32 / KB;
  if constexpr (E < KCW) {
    const half8_t a = as_half8(lut_read(lutk, cp.template addr<E + 0>()), lut_read(lutk, cp.template addr<E + 1>()),
                               lut_read(lutk, cp.template addr<E + 2>()), lut_read(lutk, cp.template addr<E + 3>()));
    const int kb = kb0 + E / 4;
    const half8_t bq = as_half8(bk[kb][0], bk[kb][1], bk[kb][2], bk[kb][3]);
    dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq, dk, 0, 0, 0);
    key_scores_word<KB, NW, E + 4>(cp, bk, lutk, dk, kb0);
  }
}

// Key tile product: lane's NW code words (4 coordinates per MFMA k-block).
template <int KB, int NW>
__device__ inline void key_scores(const uint32_t *kw, const uint32_t (*bk)[4], const uint32_t *lutk, float4_t &dk) {
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    CodePlanes<KB> cp;
    cp.set(kw[w]);
    key_scores_word<KB, NW>(cp, bk, lutk, dk, w * (32 / KB) / 4);
  }
}

template <int VB, int VDL, int NW, int DT = 0>
__device__ inline void value_update_dt(const CodePlanes<VB> (&vp)[4][NW], const uint32_t *lutv, const half8_t &aw,
                                       float4_t (&dv)[VDL]) {
  if constexpr (DT < VDL) {
    constexpr int VCW = 32 / VB, W = DT / VCW, E = DT % VCW;
    const half8_t bv = as_half8(lut_read(lutv, vp[0][W].template addr<E>()), lut_read(lutv, vp[1][W].template addr<E>()),
                                lut_read(lutv, vp[2][W].template addr<E>()), lut_read(lutv, vp[3][W].template addr<E>()));
    dv[DT] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, bv, dv[DT], 0, 0, 0);
    value_update_dt<VB, VDL, NW, DT + 1>(vp, lutv, aw, dv);
  }
}

// Value tile product: tokens ts..ts+3 (one code word set each), VDL coordinate tiles.
template <int VB, int VDL, int NW>
__device__ inline void value_update(const uint32_t (*vw)[NW], const uint32_t *lutv, const half8_t &aw,
                                    float4_t (&dv)[VDL]) {
  CodePlanes<VB> vp[4][NW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int w = 0; w < NW; ++w) vp[i][w].set(vw[i][w]);
  }
  value_update_dt<VB, VDL, NW>(vp, lutv, aw, dv);
}

// Reductions across the four 16-lane rows of the wave.
__device__ inline float max_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float sum_rows(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int D, int KB, int VB>
struct Tile {
  static constexpr int KSL = D * KB / 32, VDL = D / 16, VSL = VDL * VB / 8;
  uint32_t kw[(KSL + 3) / 4];
  uint32_t vw[4][(VSL + 3) / 4];
  uint2 kn, vn;                                   // fp16 norms of tokens ts..ts+3
};

template <int D, int KB, int VB>
__device__ inline void load_tile(Tile<D, KB, VB> &t, const uint8_t *krow, const uint8_t *vrow, const uint16_t *kn,
                                 const uint16_t *vn, int tb, int g, int n) {
  using T = Tile<D, KB, VB>;
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  load_bytes<T::KSL>(krow + (size_t)(tb + n) * KROW, t.kw);
  const int ts = tb + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) load_bytes<T::VSL>(vrow + (size_t)(ts + i) * VROW, t.vw[i]);
  t.kn = *reinterpret_cast<const uint2 *>(kn + ts);
  t.vn = *reinterpret_cast<const uint2 *>(vn + ts);
}

constexpr int kBatch = 2;          // 16-token tiles per wave iteration

template <int D, int KB, int VB>
__global__ __launch_bounds__(kBlock) void attend_mfma_kernel(MParams P) {
  constexpr int NKB = D / 16;                 // key MFMAs per tile (16 coordinates each)
  constexpr int KSL = D * KB / 32;            // key bytes per lane slice (d/4 coordinates)
  constexpr int VDL = D / 16;                 // value coordinates per lane
  constexpr int VSL = VDL * VB / 8;           // value bytes per lane per token
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  constexpr int QP = D + 4;                   // padded query row (LDS banks)
  constexpr int STEP = kWaves * kBatch * kTile;
  static_assert(KB == 2 || KB == 4, "key bits");
  static_assert(VB == 2 || VB == 4, "value bits");

  __shared__ uint32_t lutk[16], lutv[16];
  __shared__ float qz[kGMax * QP];
  __shared__ float qmax[kGMax];
  __shared__ float red_ml[kWaves][kGMax][2];
  __shared__ float red_acc[kWaves][16][D + 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int G = P.q_heads / P.kv_heads;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / P.kv_heads, hkv = bh - b * P.kv_heads;

  // chunks of ceil(T/S) tokens rounded up to a multiple of the tile
  const int chunk = ((P.seq_len + P.num_splits - 1) / P.num_splits + kTile - 1) / kTile * kTile;
  const int t0 = min(P.seq_len, split * chunk), t1 = min(P.seq_len, t0 + chunk);
  const uint8_t *krow = P.k_codes + (size_t)bh * P.capacity * KROW + g * KSL;
  const uint8_t *vrow = P.v_codes + (size_t)bh * P.capacity * VROW + n * VSL;
  const uint16_t *kn = P.k_norms + (size_t)bh * P.capacity;
  const uint16_t *vn = P.v_norms + (size_t)bh * P.capacity;

  // first batch in flight before the prologue; a tile that starts past the
  // split end reloads the batch's first tile (all its tokens are masked)
  Tile<D, KB, VB> cur[kBatch], nxt[kBatch];
  int tb = t0 + wave * kBatch * kTile;
  if (tb < t1) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) load_tile(cur[u], krow, vrow, kn, vn, (tb + u * kTile < t1) ? tb + u * kTile : tb, g, n);
  }

  // ---- centroid tables and the sign-flipped queries ----
  if (tid < (1 << KB)) lutk[tid] = split_entry(P.k_centroids[tid] * kCodeScale);
  if (tid >= 64 && tid < 64 + (1 << VB)) lutv[tid - 64] = split_entry(P.v_centroids[tid - 64] * kCodeScale);
  for (int i = tid; i < kGMax * D; i += kBlock) {
    const int h = i / D, j = i - (i / D) * D;
    float v = 0.f;
    if (h < G) {
      const size_t qi = ((size_t)b * P.q_heads + hkv * G + h) * D + j;
      v = P.q_f16 ? half_value(static_cast<const uint16_t *>(P.q)[qi]) : static_cast<const float *>(P.q)[qi];
      if (P.signs[j] < 0) v = -v;
    }
    qz[h * QP + j] = v;
  }
  __syncthreads();
  // unnormalised Walsh-Hadamard transform of each query (Sylvester order)
  for (int len = 1; len < D; len <<= 1) {
    for (int i = tid; i < G * (D / 2); i += kBlock) {
      const int h = i / (D / 2), k = i - h * (D / 2);
      const int lo = (k / len) * 2 * len + (k % len);
      const float a = qz[h * QP + lo], c = qz[h * QP + lo + len];
      qz[h * QP + lo] = a + c;
      qz[h * QP + lo + len] = a - c;
    }
    __syncthreads();
  }
  if (wave == 0) {
    for (int h = 0; h < G; ++h) {
      float m = 0.f;
      for (int j = lane; j < D; j += 64) m = fmaxf(m, fabsf(qz[h * QP + j]));
      m = max_rows(m);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) qmax[h] = m;
    }
  }
  __syncthreads();

  // ---- key-side B operand: column n serves head n % 8 ----
  const int hq = n & 7;
  const bool col_live = hq < G;
  float qscale = 1.f;
  if (col_live && qmax[hq] > 0.f) qscale = exp2f(7.f - ceilf(log2f(qmax[hq])));   // max |z * qscale| in (64, 128]
  uint32_t bk[NKB][4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float z = col_live ? qz[hq * QP + g * (D / 4) + 4 * kb + p] * qscale : 0.f;
      const _Float16 hi = (_Float16)z;
      const _Float16 lo = (_Float16)(z - (float)hi);
      bk[kb][p] = (n < 8) ? pack2(hi, hi) : pack2(lo, (_Float16)0.f);
    }
  }
  // score in base-2 units = norm * (column h + column h+8) * sfac
  const float sfac = col_live ? kLog2e / ((float)D * kCodeScale * qscale) : 0.f;

  float4_t dv[VDL];
#pragma unroll
  for (int dt = 0; dt < VDL; ++dt) dv[dt] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (; tb < t1; tb += STEP) {
    const int tn = tb + STEP;
    if (tn < t1) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) load_tile(nxt[u], krow, vrow, kn, vn, (tn + u * kTile < t1) ? tn + u * kTile : tn, g, n);
    }

    // ---- scores of tokens ts..ts+3 of each tile for head hq ----
    float4_t dk[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      dk[u] = (float4_t){0.f, 0.f, 0.f, 0.f};
      key_scores<KB, KSL / 4>(cur[u].kw, bk, lutk, dk[u]);
    }
    float s[kBatch][4];
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int ts = tb + u * kTile + 4 * g;
      const uint32_t knw[2] = {cur[u].kn.x, cur[u].kn.y};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float nk = half_value((knw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        const float v = (dk[u][i] + row_swap8(dk[u][i])) * (nk * sfac);
        s[u][i] = (col_live && ts + i < t1) ? v : -INFINITY;
        mt = fmaxf(mt, s[u][i]);
      }
    }
    mt = max_rows(mt);

    if (__builtin_amdgcn_ballot_w64(mt > m_run) != 0) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
      l_run *= alpha;
      m_run = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, (4 * g + i) & 7);
#pragma unroll
        for (int dt = 0; dt < VDL; ++dt) dv[dt][i] *= ai;
      }
    }

#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t vnw[2] = {cur[u].vn.x, cur[u].vn.y};
      uint32_t av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (s[u][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[u][i] - m_run);
        l_run += p;
        const float nv = half_value((vnw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        const float w = (p > 0.f) ? p * nv : 0.f;
        const _Float16 hi = (_Float16)w;
        const _Float16 part = (n < 8) ? hi : (_Float16)(w - (float)hi);
        av[i] = pack2(part, part);
      }
      const half8_t aw = as_half8(av[0], av[1], av[2], av[3]);
      value_update<VB, VDL, (VSL + 3) / 4>(cur[u].vw, lutv, aw, dv);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) cur[u] = nxt[u];
  }

  // ---- wave epilogue: l per head over the 4 lane groups; value tile rows to LDS ----
  l_run = sum_rows(l_run);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int dt = 0; dt < VDL; ++dt) red_acc[wave][4 * g + i][n * VDL + dt] = dv[dt][i];
  }
  if (lane < kGMax) {
    red_ml[wave][lane][0] = m_run;
    red_ml[wave][lane][1] = l_run;
  }
  __syncthreads();

  // ---- merge the four waves (rows h and h+8 carry the high and low weight halves) ----
  const int total = P.num_splits;
  for (int i = tid; i < G * D; i += kBlock) {
    const int h = i / D, j = i - (i / D) * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_ml[w][h][0]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = red_ml[w][h][0];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      l += red_ml[w][h][1] * f;
      o += (red_acc[w][h][j] + red_acc[w][h + 8][j]) * f;
    }
    const size_t row = ((size_t)b * P.q_heads + hkv * G + h) * total + split;
    P.part_o[row * D + j] = (l > 0.f) ? o / (l * kCodeScale) : 0.f;
    if (j == 0) {
      P.part_ml[row * 2 + 0] = (M == -INFINITY) ? -INFINITY : M * kLn2;
      P.part_ml[row * 2 + 1] = l;
    }
  }
}

template <int D, int KB, int VB>
hipError_t go(const AttendArgs &a, hipStream_t stream) {
  MParams P{a.q, a.q_f16, a.kv_heads, a.q_heads, a.capacity, a.seq_len, a.num_splits, a.k_codes, a.v_codes,
            a.k_norms, a.v_norms, a.signs, a.k_centroids, a.v_centroids, a.part_o, a.part_ml};
  dim3 grid(a.num_splits, a.batch * a.kv_heads);
  hipLaunchKernelGGL((attend_mfma_kernel<D, KB, VB>), grid, dim3(kBlock), 0, stream, P);
  return hipGetLastError();
}

template <int D>
hipError_t by_format(const AttendArgs &a, hipStream_t stream, bool *ok) {
  if (a.k_format == 4 && a.v_format == 4) return go<D, 4, 4>(a, stream);
  if (a.k_format == 2 && a.v_format == 2) return go<D, 2, 2>(a, stream);
  *ok = false;
  return hipSuccess;
}

}  // namespace

bool mfma_attend_supported(const AttendArgs &a) {
  const int G = a.q_heads / a.kv_heads;
  const bool fmt = (a.k_format == 4 && a.v_format == 4) || (a.k_format == 2 && a.v_format == 2);
  return fmt && a.num_near_splits == 0 && G >= 1 && G <= kGMax && (a.head_dim == 128 || a.head_dim == 256);
}

hipError_t launch_attend_mfma(const AttendArgs &a, hipStream_t stream, bool *supported) {
  *supported = true;
  switch (a.head_dim) {
    case 128: return by_format<128>(a, stream, supported);
    case 256: return by_format<256>(a, stream, supported);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace kvq
