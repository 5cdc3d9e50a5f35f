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
// walking batches of two 16-token tiles of the split.  Lane (g, n) =
// (lane / 16, lane % 16): its key slice is token n of the tile, coordinates
// [g*d/4, (g+1)*d/4) (one 16-byte load at d=128, 4-bit); its scores are
// tokens 4g..4g+3 for head n % 8; its value codes are tokens 4g..4g+3,
// coordinates [n*d/16, (n+1)*d/16).  All loads are buffer loads with the
// cache arrays as SGPR resources and 32-bit lane offsets.
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
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kTile = 16;
constexpr int kGMax = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kCodeScale = 256.f;            // centroid scale: keeps the low fp16 half a normal number
constexpr int kRawBufferFlags = 0x00020000;    // 32-bit data format, untyped raw access

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

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBufferFlags);
}

// NB bytes at byte offset off of a buffer into 32-bit words (NB in {2,4,8,16,32}).
template <int NB>
__device__ inline void buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[(NB + 3) / 4]) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const uint4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (NB == 8) {
    const uint2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (NB == 4) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else {
    static_assert(NB == 2, "slice size");
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
}

// (byte K of v) * 4: turns a byte holding one code into an LDS table
// offset (the compiler selects a byte-select shift where it can).
template <int K>
__device__ inline uint32_t byte_x4(uint32_t v) {
  return ((v >> (8 * K)) & 0xFFu) << 2;
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

// Max / sum over the four 16-lane rows that hold one column, with the gfx950
// row swaps (VALU, no LDS): after v_permlane16_swap on two copies of x, each
// lane holds its own value in one copy and its xor-16 partner's in the other;
// v_permlane32_swap does the same for xor 32.
// (Compiler builtins, so that the compiler pads their hazards, matrix-core
// operands included.)
__device__ inline void swap16(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b), false, false);
  const unsigned r0 = r[0], r1 = r[1];   // (copied out first: a bit cast of r[1] itself reads element 0)
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ inline void swap32(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b), false, false);
  const unsigned r0 = r[0], r1 = r[1];   // (copied out first: a bit cast of r[1] itself reads element 0)
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ inline float max_rows(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = fmaxf(a, b);
  a = x;
  b = x;
  swap32(a, b);
  return fmaxf(a, b);
}
__device__ inline float sum_rows(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = a + b;
  a = x;
  b = x;
  swap32(a, b);
  return a + b;
}

template <int D, int KB, int VB>
struct Geometry {
  static constexpr int NKB = D / 16;          // key MFMAs per tile (16 coordinates each)
  static constexpr int KSL = D * KB / 32;     // key bytes per lane slice (d/4 coordinates)
  static constexpr int VDL = D / 16;          // value coordinates per lane
  static constexpr int VSL = VDL * VB / 8;    // value bytes per lane per token
  static constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  static constexpr int KW = (KSL + 3) / 4, VW = (VSL + 3) / 4;
};

template <int D, int KB, int VB>
struct Tile {
  using Gm = Geometry<D, KB, VB>;
  uint32_t kw[Gm::KW];
  uint32_t vw[4][Gm::VW];
  uint32_t kn[2], vn[2];                       // fp16 norms of tokens ts..ts+3
};

struct Sources {
  __amdgpu_buffer_rsrc_t kc, vc, kn, vn;
};

// Loads of the tile at token tb.  With skip set every offset is moved past
// the end of its buffer, where buffer loads return zeros without touching
// memory; loads are thus issued unconditionally, which keeps the wait for a
// tile at its first use instead of at a control-flow join.
template <int D, int KB, int VB>
__device__ inline void load_tile(Tile<D, KB, VB> &t, const Sources &src, int tb, bool skip, int g, int n) {
  using Gm = Geometry<D, KB, VB>;
  const uint32_t far = skip ? 0x80000000u : 0u;
  buf_load<Gm::KSL>(src.kc, far + (uint32_t)(tb + n) * Gm::KROW + g * Gm::KSL, t.kw);
  const int ts = tb + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) buf_load<Gm::VSL>(src.vc, far + (uint32_t)(ts + i) * Gm::VROW + n * Gm::VSL, t.vw[i]);
  buf_load<8>(src.kn, far + (uint32_t)ts * 2, t.kn);
  buf_load<8>(src.vn, far + (uint32_t)ts * 2, t.vn);
}

template <int KB, int E>
__device__ inline half8_t key_operand(const CodePlanes<KB> &c, const uint32_t *lutk) {
  return as_half8(lut_read(lutk, c.template addr<E>()), lut_read(lutk, c.template addr<E + 1>()),
                  lut_read(lutk, c.template addr<E + 2>()), lut_read(lutk, c.template addr<E + 3>()));
}

template <int KB, int W, int E = 0>
__device__ inline void key_word(const CodePlanes<KB> &c0, const uint32_t (*bk)[4], const uint32_t *lutk, float4_t &d0) {
  constexpr int KCW = 32 / KB;
  if constexpr (E < KCW) {
    constexpr int kb = (W * KCW + E) / 4;
    const half8_t bq = as_half8(bk[kb][0], bk[kb][1], bk[kb][2], bk[kb][3]);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand<KB, E>(c0, lutk), bq, d0, 0, 0, 0);
    key_word<KB, W, E + 4>(c0, bk, lutk, d0);
  }
}

template <int KB, int KW, int W = 0>
__device__ inline void key_scores(const uint32_t (&kw0)[KW], const uint32_t (*bk)[4], const uint32_t *lutk, float4_t &d0) {
  if constexpr (W < KW) {
    CodePlanes<KB> c0;
    c0.set(kw0[W]);
    key_word<KB, W>(c0, bk, lutk, d0);
    key_scores<KB, KW, W + 1>(kw0, bk, lutk, d0);
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
__device__ inline void value_update(const uint32_t (&vw)[4][NW], const uint32_t *lutv, const half8_t &aw,
                                    float4_t (&dv)[VDL]) {
  CodePlanes<VB> vp[4][NW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int w = 0; w < NW; ++w) vp[i][w].set(vw[i][w]);
  }
  value_update_dt<VB, VDL, NW>(vp, lutv, aw, dv);
}

// One 16-token tile of the online softmax.  TAIL masks tokens at or past t1;
// full tiles skip every per-token test.
template <bool TAIL, int D, int KB, int VB>
__device__ inline void process_tile(const Tile<D, KB, VB> &t, const uint32_t (*bk)[4], const uint32_t *lutk,
                                    const uint32_t *lutv, float sfac, int tb, int t1, int g, int n,
                                    float4_t (&dv)[Geometry<D, KB, VB>::VDL], float &m_run, float &l_run) {
  using Gm = Geometry<D, KB, VB>;
  float4_t dk = {0.f, 0.f, 0.f, 0.f};
  key_scores<KB, Gm::KW>(t.kw, bk, lutk, dk);

  float s[4];
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float nk = half_value((t.kn[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
    float v = (dk[i] + row_swap8(dk[i])) * (nk * sfac);
    if constexpr (TAIL) v = (tb + 4 * g + i < t1) ? v : -INFINITY;
    s[i] = v;
    mt = fmaxf(mt, v);
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
      for (int dt = 0; dt < Gm::VDL; ++dt) dv[dt][i] *= ai;
    }
  }

  uint32_t av[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float p = __builtin_amdgcn_exp2f(s[i] - m_run);
    if constexpr (TAIL) p = (s[i] == -INFINITY) ? 0.f : p;
    l_run += p;
    const float nv = half_value((t.vn[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
    float w = p * nv;
    if constexpr (TAIL) w = (p > 0.f) ? w : 0.f;
    const _Float16 hi = (_Float16)w;
    const _Float16 part = (n < 8) ? hi : (_Float16)(w - (float)hi);
    av[i] = pack2(part, part);
  }
  value_update<VB, Gm::VDL, Gm::VW>(t.vw, lutv, as_half8(av[0], av[1], av[2], av[3]), dv);
}

template <int D, int KB, int VB>
// d = 256 keeps two work-groups per SIMD row (at most 256 registers per lane)
__global__ __launch_bounds__(kBlock, D == 256 ? 2 : 3) void attend_mfma_kernel(MParams P) {
  using Gm = Geometry<D, KB, VB>;
  constexpr int NKB = Gm::NKB, VDL = Gm::VDL;
  constexpr int STEP = kWaves * kTile;
  static_assert(KB == 2 || KB == 4, "key bits");
  static_assert(VB == 2 || VB == 4, "value bits");

  __shared__ uint32_t lutk[16], lutv[16];
  __shared__ float red_ml[kWaves][kGMax][2];
  __shared__ float red_acc[kWaves][16][D + 4];
  __shared__ __attribute__((aligned(16))) uint32_t qent[kGMax][D + 4];
  __shared__ float qfac[kGMax];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int G = P.q_heads / P.kv_heads;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / P.kv_heads, hkv = bh - b * P.kv_heads;

  // chunks of ceil(T/S) tokens rounded up to a multiple of 32 (two tiles)
  const int chunk = ((P.seq_len + P.num_splits - 1) / P.num_splits + 2 * kTile - 1) / (2 * kTile) * (2 * kTile);
  const int t0 = min(P.seq_len, split * chunk), t1 = min(P.seq_len, t0 + chunk);
  const uint32_t cap = (uint32_t)P.capacity;
  Sources src;
  src.kc = make_rsrc(P.k_codes + (size_t)bh * cap * Gm::KROW, cap * Gm::KROW);
  src.vc = make_rsrc(P.v_codes + (size_t)bh * cap * Gm::VROW, cap * Gm::VROW);
  src.kn = make_rsrc(P.k_norms + (size_t)bh * cap, cap * 2);
  src.vn = make_rsrc(P.v_norms + (size_t)bh * cap, cap * 2);

  // Full tiles [t0, t1f) go through the main loop; a partial last tile (only
  // the last split can have one) is handled after it.  Tiles stay inside the
  // cache: t0 and the capacity are multiples of 16.
  const int t1f = t0 + ((t1 - t0) & ~(kTile - 1));
  Tile<D, KB, VB> ta, tc;
  int tb = t0 + wave * kTile;
  load_tile(ta, src, tb, tb >= t1f, g, n);        // in flight during the prologue

  // ---- rotated queries, shared by the work-group ----
  // Wave w rotates heads w and w+4: lane l holds coordinates [l*E1, (l+1)*E1);
  // sign flip, Walsh-Hadamard stages of stride < E1 inside the lane, strides
  // E1..32*E1 across lanes (xor 1..32).  Each rotated coordinate z, scaled so
  // that max |z| of its head lies in (64, 128], is stored as an fp16 (hi, lo)
  // pair; the row stride D+4 keeps the later 16-byte reads conflict-free.
  constexpr int E1 = D / 64;
  for (int h = wave; h < G; h += kWaves) {
    float z[E1];
    const size_t qoff = ((size_t)b * P.q_heads + hkv * G + h) * D + lane * E1;
    if (P.q_f16) {
      const uint16_t *qs = static_cast<const uint16_t *>(P.q) + qoff;
#pragma unroll
      for (int e = 0; e < E1; ++e) z[e] = half_value(qs[e]);
    } else {
      const float *qs = static_cast<const float *>(P.q) + qoff;
#pragma unroll
      for (int e = 0; e < E1; ++e) z[e] = qs[e];
    }
#pragma unroll
    for (int e = 0; e < E1; ++e) z[e] = (P.signs[lane * E1 + e] < 0) ? -z[e] : z[e];
#pragma unroll
    for (int st = 1; st < E1; st <<= 1) {
#pragma unroll
      for (int e = 0; e < E1; ++e) {
        if (!(e & st)) {
          const float a = z[e], c = z[e + st];
          z[e] = a + c;
          z[e + st] = a - c;
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int e = 0; e < E1; ++e) {
        const float o = __shfl_xor(z[e], m);
        z[e] = upper ? (o - z[e]) : (z[e] + o);
      }
    }
    float zmax = 0.f;
#pragma unroll
    for (int e = 0; e < E1; ++e) zmax = fmaxf(zmax, fabsf(z[e]));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, m));
    const float qscale = (zmax > 0.f) ? exp2f(7.f - ceilf(log2f(zmax))) : 1.f;
#pragma unroll
    for (int e = 0; e < E1; ++e) qent[h][lane * E1 + e] = split_entry(z[e] * qscale);
    if (lane == 0) qfac[h] = kLog2e / ((float)D * kCodeScale * qscale);
  }
  if (tid < (1 << KB)) lutk[tid] = split_entry(P.k_centroids[tid] * kCodeScale);
  if (tid >= 64 && tid < 64 + (1 << VB)) lutv[tid - 64] = split_entry(P.v_centroids[tid - 64] * kCodeScale);
  __syncthreads();

  // ---- key-side B operand: column n serves head n % 8 ----
  // columns 0..7 take (z_hi, z_hi), columns 8..15 take (z_lo, 0); columns of
  // heads >= G carry zeros and feed only value rows that are never read
  const int hq = n & 7;
  const bool col_live = hq < G;
  const uint32_t sel = (n < 8) ? 0x01000100u : 0x0C0C0302u;   // v_perm byte selectors
  uint32_t bk[NKB][4];
#pragma unroll
  for (int k4 = 0; k4 < NKB; ++k4) {
    uint4_t e = {0u, 0u, 0u, 0u};
    if (col_live) e = *reinterpret_cast<const uint4_t *>(&qent[hq][g * (D / 4) + 4 * k4]);
#pragma unroll
    for (int p = 0; p < 4; ++p) bk[k4][p] = __builtin_amdgcn_perm(e[p], e[p], sel);
  }
  const float sfac = col_live ? qfac[hq] : 0.f;

  float4_t dv[VDL];
#pragma unroll
  for (int dt = 0; dt < VDL; ++dt) dv[dt] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Two tiles used in turn (no register copies between iterations, so the
  // wait for a tile's loads sits at its first use and the next tile's loads
  // stay in flight meanwhile).
  for (; tb < t1f; tb += 2 * STEP) {
    load_tile(tc, src, tb + STEP, tb + STEP >= t1f, g, n);
    process_tile<false>(ta, bk, lutk, lutv, sfac, tb, t1, g, n, dv, m_run, l_run);
    if (tb + STEP >= t1f) break;
    load_tile(ta, src, tb + 2 * STEP, tb + 2 * STEP >= t1f, g, n);
    process_tile<false>(tc, bk, lutk, lutv, sfac, tb + STEP, t1, g, n, dv, m_run, l_run);
  }
  if (t1f < t1 && wave == ((t1f - t0) / kTile) % kWaves) {
    load_tile(ta, src, t1f, false, g, n);
    process_tile<true>(ta, bk, lutk, lutv, sfac, t1f, t1, g, n, dv, m_run, l_run);
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
  // buffer resources address one (b, kv head) slice with 32-bit offsets
  const bool fits = (int64_t)a.capacity * a.head_dim / 2 < (1ll << 31);
  return fmt && fits && a.num_near_splits == 0 && G >= 1 && G <= kGMax && (a.head_dim == 128 || a.head_dim == 256);
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
