// Split-K GQA decode attention on 4-, 3- or 2-bit Lloyd-Max keys and values,
// head dimension 256, and on 4-bit keys with a key outlier stream at head
// dimension 128: the pair-table matrix-core tile of the head-dimension-128
// kernel (shared tile code; quad-table entries for 2-bit codes, tables
// indexed by 6-bit fields of two codes for 3-bit ones) at two waves per
// SIMD, which leaves registers for the larger tiles and the side stream.
//
// Outlier stream ("Outlier Two-Stream Cache": the keys' largest-variance
// channels kept as int8 codes with a per-token scale, beside the codes of
// the keys with those channels zeroed): each lane adds
// scale * sum_k q[idx_k] code_k / sqrt(d) to its two tokens' scores before
// the softmax update, the int8 codes and scales of its tokens loaded with
// the tile and q at the 8 channels held in registers.
//
// Work mapping: a work-group of 8 waves (two per SIMD: at d = 256 the query
// operand and the value accumulator take 128 registers) fills a compute
// unit and shares one pair table.  Its wave groups serve 2^lg
// consecutive units of the flattened (b * Hkv + KV head, split) space, so
// with few query heads per KV head a work-group covers splits of several
// (b, KV head) pairs and the grid needs no second round of work-groups; a
// group of several waves takes 16-token tiles from an LDS counter, two tiles
// in flight per wave.  The group's rotated queries sit in LDS, one row pair
// per head (hi and lo fp16 forms), at most 8 rows per work-group.
// Sources: "The Engineering Behind AdapTQ", "Engineering the Hot Path"
// (rotate q once, score from codes through a table, no dequantize pass);
// "FoveatedKV", "Making it fast" (split-K, pre-scaled q, online softmax with
// one exp per score, split merge); "I Ported a Google Research Paper to Apple
// Silicon", "The Bit-Packing Problem" (4-bit codes, low nibble first).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"
#include "kvq_lane.h"
#include "kvq_pair.h"

namespace kvq {
namespace {

using namespace pair;

constexpr int kWaves = 8;
constexpr int kMinWaves = 2;                   // waves per SIMD the register budget is sized for
constexpr int kBlock = kWaves * 64;
constexpr int kZeroRow = 2 * kGMax;             // all-zero query row for the unused B columns
constexpr int kSetupWaves = 4;                  // waves that build the tables and the rotated queries

struct WParams {
  const void *q;
  int q_f16;
  int kv_heads, capacity, seq_len, num_splits;
  int group_size;                  // query heads per KV head
  int chunk;                       // tokens per split (a multiple of 32)
  int group_log2;                  // log2 of the units one work-group covers (its wave groups)
  int units;                       // (b, KV head) pairs times splits
  int part_stride;                 // splits per (b, query head) row of the partial buffers
  const uint8_t *k_codes, *v_codes;
  const uint16_t *k_norms, *v_norms;
  const int8_t *signs;
  const float *k_centroids, *v_centroids;
  float *part_o, *part_ml;
  // key outlier stream: [b * Hkv + KV head][8] channels,
  // [..][capacity][8] int8 codes, [..][capacity] scales
  const int32_t *out_idx;
  const int8_t *out_codes;
  const float *out_scales;
  // QJL residual sketch (QJL kernels): S^T [D][D], sketch bits
  // [b * Hkv + KV head][capacity][D / 8], residual norms [..][capacity] fp16
  const float *qjl_proj;
  const uint8_t *qjl_signs;
  const uint16_t *qjl_norms;
};

// Key side streams of a tile.
constexpr int kSideNone = 0, kSideOut = 1, kSideQjl = 2;
constexpr float kQjlRho = 1.2533141373155003f;   // sqrt(pi / 2): the sketch estimate's factor (over m = D)
constexpr int kSketchTab = 16384;                 // byte offset of the sketch operand table in `tab` (3-bit keys)
constexpr int kSketchPart = 32768;                // byte offset of the S q partial sums in `tab` during set-up

// Per-tile registers: outlier stream: the int8 codes (two 8-byte rows) and
// scales of the lane's two tokens 4g + 2 (n & 1) + {0, 1}; QJL sketch: the
// sketch bits 32g..32g+31 of token n and the fp16 residual norms of the
// lane's two tokens.
template <int X>
struct SideTile {};
template <>
struct SideTile<kSideOut> {
  uint4_t oc;
  uint2_t os;
};
template <>
struct SideTile<kSideQjl> {
  uint32_t zw;
  uint32_t rn;
};

// Slices of the side stream's two arrays (outliers: codes, scales; QJL:
// sketch bits, residual norms) for one (b, KV head).
struct SideSources {
  const uint8_t *a, *b;
  uint32_t a_bytes, b_bytes;
  uint32_t ao, bo;                     // per-lane offsets
};

template <int D, int X>
constexpr int kSideLoads = (X == kSideNone) ? 0 : 2;

template <int D, int X>
__device__ inline void load_side(SideTile<X> &t, const SideSources &src, int tb, bool skip) {
  if constexpr (X != kSideNone) {
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(src.a, skip ? 0u : src.a_bytes);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(src.b, skip ? 0u : src.b_bytes);
    if constexpr (X == kSideOut) {
      t.oc = __builtin_amdgcn_raw_buffer_load_b128(ar, src.ao, tb * kOutlierCount, kStream);
      t.os = __builtin_amdgcn_raw_buffer_load_b64(br, src.bo, tb * 4, kStream);
    } else {
      t.zw = __builtin_amdgcn_raw_buffer_load_b32(ar, src.ao, tb * (D / 8), kStream);
      t.rn = __builtin_amdgcn_raw_buffer_load_b32(br, src.bo, tb * 2, kStream);
    }
  }
}

// The partial last tile: descriptors from the tile to the slice's end.
template <int D, int X>
__device__ inline void load_side_tail(SideTile<X> &t, const SideSources &src, int tb) {
  if constexpr (X != kSideNone) {
    constexpr uint32_t ar = (X == kSideOut) ? kOutlierCount : D / 8, br = (X == kSideOut) ? 4 : 2;
    SideSources s = src;
    s.a += (size_t)tb * ar;
    s.b += (size_t)tb * br;
    s.a_bytes -= (uint32_t)tb * ar;
    s.b_bytes -= (uint32_t)tb * br;
    load_side<D, X>(t, s, 0, false);
  }
}

// Per-lane state of the side stream for the lane's head (zero for columns
// past the group): outliers: qo = q at the 8 channels times log2(e)/sqrt(d);
// QJL: the sketch B operand (2 p pscale split hi / lo, one column each),
// 1 / pscale, sum p, and the sketch table address of the lane's slot.
template <int X>
struct SideState {
  float qo[X == kSideOut ? kOutlierCount : 1];
  uint4_t bq[X == kSideQjl ? 4 : 1];
  float pf, ps;
  uint32_t zslot;
};

// Adds the side stream's term to the lane's two raw scores (log2 units).
//   outliers: scale * sum_k qo_k code_k;
//   QJL: rho (sum_i (2 z_i - 1) p_i) with rho = ||r||_16 sqrt(pi/2) / D and
//        p = S q~ log2(e) / D, as rho (sum_i z_i 2 p_i - sum_i p_i): the first
//        sum is a second contraction per tile, the sketch bits as fp16 0/1 A
//        operands (one table read per byte of bits: 8 indices, two per
//        32-bit word) against 2 p pscale split hi (column 2h) and lo
//        (column 2h+1).
template <int D, int X>
__device__ inline void side_terms(const SideTile<X> &t, const SideState<X> &st, const uint8_t *tab, int n,
                                  float (&s)[2]) {
  if constexpr (X == kSideOut) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t w0 = u ? t.oc.z : t.oc.x, w1 = u ? t.oc.w : t.oc.y;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < kOutlierCount; ++k) {
        const uint32_t w = (k < 4) ? w0 : w1;
        const float c = (float)(int8_t)(uint8_t)(w >> (8 * (k & 3)));
        acc = __builtin_fmaf(st.qo[k], c, acc);
      }
      s[u] = __builtin_fmaf(__builtin_bit_cast(float, u ? t.os.y : t.os.x), acc, s[u]);
    }
  } else if constexpr (X == kSideQjl) {
    float4_t dq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t addr = (((t.zw >> (8 * kb)) & 0xFFu) << 6) | st.zslot;
      dq = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, quad_read(tab, addr)),
                                                   __builtin_bit_cast(half8_t, st.bq[kb]), dq, 0, 0, 0);
    }
    const bool odd = n & 1;
    const float f0 = add_swap1(dq[0]), f1 = add_swap1(dq[1]), f2 = add_swap1(dq[2]), f3 = add_swap1(dq[3]);
    const float d0 = odd ? f2 : f0, d1 = odd ? f3 : f1;
    const float r0 = half_value(t.rn & 0xFFFFu) * (kQjlRho / (float)D), r1 = half_value(t.rn >> 16) * (kQjlRho / (float)D);
    s[0] = __builtin_fmaf(r0, __builtin_fmaf(d0, st.pf, -st.ps), s[0]);
    s[1] = __builtin_fmaf(r1, __builtin_fmaf(d1, st.pf, -st.ps), s[1]);
  }
}

// process_tile with the side stream's term added before the softmax update
// (so the rescale decision sees the whole score).
template <int D, int KB, int VB, int X, bool TAIL>
__device__ inline void process_tile_side(const Tile<D, KB, VB> &t, const SideTile<X> &sd, const SideState<X> &st,
                                         const uint4_t (&bk)[D / 16], const uint8_t *tab, uint32_t kslot,
                                         uint32_t vslot, float sfac, float m1, int tb, int t1, int g, int n,
                                         float4_t (&dv)[D / 16], float &m_run, float &l_run, float &m_top) {
  float4_t dk = {0.f, 0.f, 0.f, 0.f};
  key_scores<D, KB>(t.kw, bk, tab, kslot, dk);
  const bool odd = n & 1;
  const uint32_t knp = odd ? t.kn.y : t.kn.x;
  const uint32_t vnp = odd ? t.vn.y : t.vn.x;
  float s[2];
  raw_scores<true>(dk, knp, sfac, n, s);
  side_terms<D, X>(sd, st, tab, n, s);
  tile_update<D, TAIL>(s, tb, t1, g, n, dv, m_run, l_run, m_top);
  ValueBytes<D, VB> vb;
  value_bytes<D, VB>(t, vb, n);
  const half8_t aw = tile_weights<TAIL, true>(s, vnp, m1, n, m_run, l_run);
  value_update<D, VB>(vb, tab, vslot, aw, dv);
}

// Pair tables (4-bit, 3-bit) or quad tables (2-bit) of the key codebook in
// the first 64 KB of `tab` and, when the value codebook differs (another
// width or other centroids), of the value codebook in the next 64 KB; run
// by the four set-up waves.  Thread t < 256 writes the 16-byte chunks
// t + 256k, k = 0..15 (0..3 for the 64 rows of a 3-bit table): row (code
// byte or field) t/16 + 16k, so the low four bits of the row,
// t/16 = 4 wave + lane/16, are the same for every k and the high bits are k.
//   4-bit: a row holds 32 slots of (e(c[r % 16]), e(c[r / 16])), a chunk two
//          slots;
//   3-bit: a row holds 32 slots of (e(c[r & 7]), e(c[r >> 3])), a chunk two
//          slots; r & 7 is lane/16 + 4 (wave & 1) and r >> 3 is
//          wave/2 + 2k;
//   2-bit: a row holds 16 slots of (e(c[r & 3]), e(c[(r >> 2) & 3]),
//          e(c[(r >> 4) & 3]), e(c[r >> 6])), a chunk one slot.
// Centroids come through uniform addresses (scalar loads: every index below
// is a constant or depends on the wave only).
template <int BITS>
__device__ inline void fill_table(uint8_t *t, const float *c, int wave, int lane, int tid) {
  const int r4 = lane >> 4;
  // entries of the row's low four bits: code t/16 = 4 wave + lane/16
  // (4-bit), lane/16 + 4 (wave & 1) (3-bit), or codes r4 and wave (2-bit)
  const int base = (BITS == 4) ? 4 * wave : (BITS == 3) ? 4 * (wave & 1) : 0;
  float lo = c[base];
#pragma unroll
  for (int u = 1; u < 4; ++u) lo = (r4 == u) ? c[base + u] : lo;
  const uint32_t le = split_entry(lo * kCodeScale);
  if constexpr (BITS == 3) {
    const int upper = wave >> 1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t hi = split_entry(c[2 * k + upper] * kCodeScale);
      *reinterpret_cast<uint4_t *>(t + (tid + 256 * k) * 16) = (uint4_t){le, hi, le, hi};
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t hi = split_entry(c[k] * kCodeScale);
      *reinterpret_cast<uint4_t *>(t + (tid + 256 * k) * 16) = (uint4_t){le, hi, le, hi};
    }
  } else {
    const uint32_t m = split_entry(c[wave] * kCodeScale);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t e2 = split_entry(c[k & 3] * kCodeScale), e3 = split_entry(c[k >> 2] * kCodeScale);
      *reinterpret_cast<uint4_t *>(t + (tid + 256 * k) * 16) = (uint4_t){le, m, e2, e3};
    }
  }
}

template <int KB, int VB>
__device__ inline void fill_tables(uint8_t *tab, const float *kcen, const float *vcen, int wave, int lane, int tid,
                                   uint32_t *v_table) {
  bool same = KB == VB;
#pragma unroll
  for (int i = 0; i < (1 << VB); ++i) same = same && (kcen[i] == vcen[i]);
  fill_table<KB>(tab, kcen, wave, lane, tid);
  if (!same) fill_table<VB>(tab + 65536, vcen, wave, lane, tid);
  if (tid == 0) v_table[0] = same ? 0u : 0x10000u;
}

template <int D, int KB, int VB, int X>
__global__ __launch_bounds__(kBlock, kMinWaves) void attend_wide_kernel(WParams P) {
  constexpr bool OUT = X == kSideOut, QJL = X == kSideQjl;
  static_assert(!QJL || (D == 128 && KB == 3 && VB == 4), "the QJL sketch beside 3-bit keys and 4-bit values at d = 128");
  static_assert(D == 256 || (D == 128 && VB == 4 && KB >= 3), "head dimension 256, or 128 with 4-bit values");
  static_assert(!OUT || (D == 128 && KB == 4 && VB == 4), "the outlier stream beside 4-bit codes at d = 128");
  using TileT = Tile<D, KB, VB>;
  constexpr int kKRow = TileT::kKRow, kVRow = TileT::kVRow;
  constexpr int kVDL = D / 16;                    // value coordinates per lane
  constexpr int kRowPad = D + 4;                  // query table row stride (words)
  constexpr int kLoads = kTileLoads<D, KB, VB> + kSideLoads<D, X>;
  // s_waitcnt vmcnt(loads of one tile) expcnt(7) lgkmcnt(15)
  constexpr int kWaitOlderTile = 0x0F70 | kLoads;
  static_assert(kLoads <= 15, "tile loads");
  // pair tables during the loop, the waves' value rows afterwards
  __shared__ __attribute__((aligned(16))) uint8_t tab[2 * 65536];
  __shared__ __attribute__((aligned(16))) uint32_t qtab[2 * kGMax + 1][kRowPad];
  __shared__ float red_ml[kWaves][kGMax][3];      // (reference, sum, largest score) per wave and head
  __shared__ float qfac[kGMax];
  __shared__ float wfac[kWaves][kGMax];
  __shared__ uint32_t next_tile[kWaves];
  __shared__ uint32_t ready;                         // set-up waves done
  __shared__ uint32_t v_table[1];                    // offset of the value table: 0 when shared with the keys
  __shared__ float qout[OUT ? kGMax : 1][kOutlierCount];   // q at the outlier channels, in log2 units of s
  // QJL: the rotated queries (fp32, before scaling) and the sketch B operand
  // rows (2 p pscale: hi halves in row 2r, lo halves in row 2r+1; a zero row last)
  __shared__ float qrot[QJL ? kGMax : 1][QJL ? D : 1];
  __shared__ __attribute__((aligned(16))) uint32_t ptab[QJL ? 2 * kGMax + 1 : 1][QJL ? D / 2 + 4 : 1];
  __shared__ float pfac[QJL ? kGMax : 1], psumr[QJL ? kGMax : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int G = P.group_size, S = P.num_splits;
  const int lg = P.group_log2;                       // group_size << group_log2 <= 8 (host)
  const int gw = kWaves >> lg;
  const int grp = wave >> (3 - lg), gwave = wave & (gw - 1);
  // this wave group's unit: pair index b * Hkv + KV head, and split; its
  // query heads are rows pr * G + h of q, since Hq = Hkv * G
  const int unit = (blockIdx.x << lg) + grp;
  const bool active = unit < P.units;
  const int pr = active ? unit / S : 0;
  const int split = active ? unit - pr * S : 0;

  // chunks of ceil(T/S) tokens rounded up to a multiple of 32 (from the
  // host); full tiles [t0, t1f) go through the main loop, a partial last
  // tile (only the last split can have one) after it
  const int chunk = P.chunk;
  const int t0 = active ? min(P.seq_len, split * chunk) : 0;
  const int t1 = active ? min(P.seq_len, t0 + chunk) : 0;
  const int ntiles = (t1 - t0) / kTile;
  const int t1f = t0 + ntiles * kTile;
  const uint32_t cap = (uint32_t)P.capacity;
  Sources src;
  src.kc = P.k_codes + (size_t)pr * cap * kKRow;
  src.vc = P.v_codes + (size_t)pr * cap * kVRow;
  src.kn = P.k_norms + (size_t)pr * cap;
  src.vn = P.v_norms + (size_t)pr * cap;
  src.kcode_bytes = cap * kKRow;
  src.vcode_bytes = cap * kVRow;
  src.norm_bytes = cap * 2;
  set_offsets<D, KB, VB>(src, g, n);
  SideSources side_src;
  if constexpr (OUT) {
    side_src.a = reinterpret_cast<const uint8_t *>(P.out_codes + (size_t)pr * cap * kOutlierCount);
    side_src.b = reinterpret_cast<const uint8_t *>(P.out_scales + (size_t)pr * cap);
    side_src.a_bytes = cap * kOutlierCount;
    side_src.b_bytes = cap * 4;
    side_src.ao = (uint32_t)(4 * g + 2 * (n & 1)) * kOutlierCount;
    side_src.bo = (uint32_t)(4 * g + 2 * (n & 1)) * 4;
  }
  if constexpr (QJL) {
    side_src.a = P.qjl_signs + (size_t)pr * cap * (D / 8);
    side_src.b = reinterpret_cast<const uint8_t *>(P.qjl_norms + (size_t)pr * cap);
    side_src.a_bytes = cap * (D / 8);
    side_src.b_bytes = cap * 2;
    side_src.ao = (uint32_t)n * (D / 8) + 4 * g;
    side_src.bo = (uint32_t)(4 * g + 2 * (n & 1)) * 2;
  }

  // ---- set-up ----
  // Waves 0-3 build the code tables and the rotated queries; waves 4-7 first
  // request their first two tiles (so the set-up waves' own requests do not
  // sit ahead of the table work in their issue queues).  Readiness is an LDS
  // count the set-up waves bump, not a barrier.
  static_assert(kSetupWaves * 64 * 16 * 16 == 65536, "table fill layout");
  if (tid < kWaves) next_tile[tid] = 2 * gw;
  if (tid == 0) ready = 0u;
  __syncthreads();                                   // cheap here: no wave has memory requests yet

  int ia = gwave, ic = gwave + gw;                   // first tiles of this wave; later ones from its group's counter
  TileT ta, tc;
  SideTile<X> sa, sc;
  if (wave < kSetupWaves) {
    fill_tables<KB, VB>(tab, P.k_centroids, P.v_centroids, wave, lane, tid, v_table);
    if (tid < D) qtab[kZeroRow][tid] = 0u;
    if constexpr (QJL) {
      if (tid < D / 2 + 4) ptab[2 * kGMax][tid] = 0u;
      // sketch operand table: entry (byte b, slot s) at kSketchTab + 64 b +
      // 16 s holds the 8 bits of b as fp16 0/1, two per word (bit 2j in the
      // low half of word j); 4 slots (lane % 4) spread a wave's reads over
      // the banks
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t c = (uint32_t)tid + 256u * k, b = c >> 2;
        uint4_t e;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          e[j] = (((b >> (2 * j)) & 1u) ? 0x3C00u : 0u) | (((b >> (2 * j + 1)) & 1u) ? 0x3C000000u : 0u);
        *reinterpret_cast<uint4_t *>(tab + kSketchTab + c * 16) = e;
      }
    }

    // ---- rotated queries: rows r = wave and wave + 4 (head r % G of the
    // unit r / G of this work-group) ----
    // Lane l holds coordinates E l .. E l + E-1 (E = D / 64): sign flip, the
    // butterflies of strides below E in the lane, strides E..D/2 across
    // lanes (xor 1..32).  The rotated vector is scaled so that its largest
    // |z| lies in (64, 128] and stored in the two B-operand forms
    // (z_hi, z_hi) (row 2r) and (z_lo, 0) (row 2r+1).
    const int q_f16 = P.q_f16;
    const uint32_t q_es = q_f16 ? 2u : 4u;
    for (int rr = 0; rr < 2; ++rr) {
      const int r = wave + kSetupWaves * rr;
      if (r >= (G << lg)) break;
      const int gr = r / G, h = r - gr * G;
      const int u = (blockIdx.x << lg) + gr;
      const bool has_q = u < P.units;
      const size_t q_row = (size_t)(has_q ? u / S : 0) * G + h;
      const __amdgpu_buffer_rsrc_t qsrc = make_rsrc(static_cast<const uint8_t *>(P.q) + q_row * D * q_es,
                                                    has_q ? (uint32_t)D * q_es : 0u);
      const __amdgpu_buffer_rsrc_t ssrc = make_rsrc(P.signs, has_q ? (uint32_t)D : 0u);
      constexpr int E = D / 64;
      float z[E];
      // fp32 elements come one 4-byte load each: a 16- or 8-byte load whose
      // words are picked against the fp16 form was compiled to one 4-byte
      // load feeding every word (an fp32 query then reads one coordinate
      // per lane); fp16 rows come as one packed load.  Both forms are read,
      // the one of the other element size goes unused (past the row's end
      // it reads as zero).
      float v32[E];
#pragma unroll
      for (int e = 0; e < E; ++e)
        v32[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qsrc, (uint32_t)(E * lane + e) * 4u, 0, 0));
      if constexpr (E == 4) {
        const uint2_t qh = __builtin_amdgcn_raw_buffer_load_b64(qsrc, lane * 8, 0, 0);
        const uint32_t sg = __builtin_amdgcn_raw_buffer_load_b32(ssrc, lane * 4, 0, 0);   // signs of 4l..4l+3
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t hw = (e < 2) ? qh.x : qh.y;
          const float v = q_f16 ? half_value((hw >> (16 * (e & 1))) & 0xFFFFu) : v32[e];
          z[e] = ((sg >> (8 * e + 7)) & 1u) ? -v : v;
        }
        const float a0 = z[0] + z[1], a1 = z[0] - z[1], a2 = z[2] + z[3], a3 = z[2] - z[3];
        z[0] = a0 + a2;
        z[1] = a1 + a3;
        z[2] = a0 - a2;
        z[3] = a1 - a3;
      } else {
        const uint32_t qh = __builtin_amdgcn_raw_buffer_load_b32(qsrc, lane * 4, 0, 0);
        const uint32_t sg = __builtin_amdgcn_raw_buffer_load_b16(ssrc, lane * 2, 0, 0);   // signs of 2l, 2l+1
        const float v0 = q_f16 ? half_value(qh & 0xFFFFu) : v32[0];
        const float v1 = q_f16 ? half_value(qh >> 16) : v32[1];
        const float w0 = (sg & 0x80u) ? -v0 : v0, w1 = (sg & 0x8000u) ? -v1 : v1;
        z[0] = w0 + w1;
        z[1] = w0 - w1;
      }
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        z[e] = fwht_lanes(z[e], lane);
        am = fmaxf(am, fabsf(z[e]));
      }
      if constexpr (QJL) {
#pragma unroll
        for (int e = 0; e < E; ++e) qrot[r][E * lane + e] = has_q ? z[e] : 0.f;
      }
      const float zmax = wave_max(am, lane);
      const float qscale = (zmax > 0.f) ? exp2f(7.f - ceilf(log2f(zmax))) : 1.f;
      uint32_t f0[E], f1[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float zs = z[e] * qscale;
        const _Float16 hs = (_Float16)zs;
        f0[e] = pack2(hs, hs);
        f1[e] = pack2((_Float16)(zs - (float)hs), (_Float16)0.f);
      }
      if constexpr (E == 4) {
        *reinterpret_cast<uint4_t *>(&qtab[2 * r][lane * 4]) = (uint4_t){f0[0], f0[1], f0[2], f0[3]};
        *reinterpret_cast<uint4_t *>(&qtab[2 * r + 1][lane * 4]) = (uint4_t){f1[0], f1[1], f1[2], f1[3]};
      } else {
        *reinterpret_cast<uint2_t *>(&qtab[2 * r][lane * 2]) = (uint2_t){f0[0], f0[1]};
        *reinterpret_cast<uint2_t *>(&qtab[2 * r + 1][lane * 2]) = (uint2_t){f1[0], f1[1]};
      }
      if constexpr (OUT) {
        // q at the unit's outlier channels (original domain), in log2 units of s
        if (lane < kOutlierCount) {
          const int32_t *oi = P.out_idx + (size_t)(has_q ? u / S : 0) * kOutlierCount;
          const int c = has_q ? oi[lane] : 0;
          const float v = q_f16 ? half_value(__builtin_amdgcn_raw_buffer_load_b16(qsrc, (uint32_t)c * 2, 0, 0))
                                : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qsrc, (uint32_t)c * 4, 0, 0));
          qout[r][lane] = has_q ? v * (kLog2e / sqrtf((float)D)) : 0.f;
        }
      }
      if (lane == 0) qfac[r] = has_q ? kLog2e / ((float)D * kCodeScale * qscale) : 0.f;
    }
    // this wave's table, query and factor writes complete before its count
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(&ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_tile<D, KB, VB>(ta, src, t0 + ia * kTile, ia >= ntiles);
  load_side<D, X>(sa, side_src, t0 + ia * kTile, ia >= ntiles);
  __builtin_amdgcn_sched_barrier(0);
  load_tile<D, KB, VB>(tc, src, t0 + ic * kTile, ic >= ntiles);
  load_side<D, X>(sc, side_src, t0 + ic * kTile, ic >= ntiles);
  __builtin_amdgcn_sched_barrier(0);

  // QJL: thread t takes column i = t % D of S^T (row i of S) over rows
  // j in [32 (t / D), +32) of S^T; its 32 loads go out before the wait
  constexpr int kJ = QJL ? 32 : 1;
  float sv[kJ];
  if constexpr (QJL) {
    static_assert(kBlock == 4 * D && 4 * kJ == D, "S q~ thread mapping");
    const int i = tid & (D - 1), j0 = (tid / D) * kJ;
#pragma unroll
    for (int j = 0; j < kJ; ++j) sv[j] = P.qjl_proj[(size_t)(j0 + j) * D + i];
  }

  // Wait for the set-up counts (bounded: every set-up wave reaches its count
  // without waiting on anything but its own loads).
  for (int spin = 0; spin < kSpinLimit; ++spin) {
    const uint32_t r = __hip_atomic_load(&ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(r) >= (uint32_t)kSetupWaves) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  SideState<X> side;
  if constexpr (QJL) {
    // p = S q~ log2(e) / D for the work-group's R query rows: partial sums
    // over each thread's 32 rows of S^T to LDS at kSketchPart (free space
    // between the sketch table and the value table), then wave r < R sums
    // its row's four partials for coordinates 2l, 2l+1 and writes the B
    // operand rows
    const int R = G << lg;
    const int i = tid & (D - 1), jq = tid / D;
    float *part = reinterpret_cast<float *>(tab + kSketchPart);      // [4][kGMax][D]
    for (int r = 0; r < R; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kJ; ++j) acc = __builtin_fmaf(sv[j], qrot[r][jq * kJ + j], acc);
      part[(jq * kGMax + r) * D + i] = acc;
    }
    __syncthreads();                                 // waits on LDS only: the tile loads stay in flight
    if (wave < R) {
      const int r = wave;
      float p2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 2 * lane + e;
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) v += part[(q * kGMax + r) * D + c];
        p2[e] = v * (kLog2e / (float)D);
      }
      const float amax = wave_max(2.f * fmaxf(fabsf(p2[0]), fabsf(p2[1])), lane);
      const float total = wave_sum(p2[0] + p2[1], lane);
      const float pscale = (amax > 0.f) ? exp2f(7.f - ceilf(log2f(amax))) : 1.f;
      const float a = 2.f * p2[0] * pscale, c = 2.f * p2[1] * pscale;
      const _Float16 ha = (_Float16)a, hc = (_Float16)c;
      ptab[2 * r][lane] = pack2(ha, hc);
      ptab[2 * r + 1][lane] = pack2((_Float16)(a - (float)ha), (_Float16)(c - (float)hc));
      if (lane == 0) {
        pfac[r] = 1.f / pscale;
        psumr[r] = total;
      }
    }
    __syncthreads();
    // B operand of sketch block kb for column n: row n (head n / 2, hi or lo
    // halves), sketch indices 32g + 8kb .. +7
    const bool scol = n < 2 * G;
    const int prow = scol ? grp * 2 * G + n : 2 * kGMax;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) side.bq[kb] = *reinterpret_cast<const uint4_t *>(&ptab[prow][16 * g + 4 * kb]);
    side.pf = scol ? pfac[grp * G + (n >> 1)] : 0.f;
    side.ps = scol ? psumr[grp * G + (n >> 1)] : 0.f;
    side.zslot = (uint32_t)kSketchTab + (uint32_t)(lane & 3) * 16;
  }

  // B operand of key block kb for column n: the group's query row 2h + form
  // for n = 2h + form < 2G (the zero row otherwise), coordinates
  // 64g + 4kb .. +3
  const bool col = n < 2 * G;
  const int qrow = col ? grp * 2 * G + n : kZeroRow;
  uint4_t bk[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) bk[kb] = *reinterpret_cast<const uint4_t *>(&qtab[qrow][g * (D / 4) + 4 * kb]);
  const float sfac = col ? qfac[grp * G + (n >> 1)] : 0.f;
  if constexpr (OUT) {
#pragma unroll
    for (int k = 0; k < kOutlierCount; ++k) side.qo[k] = col ? qout[grp * G + (n >> 1)][k] : 0.f;
  }
  // table slot: lane % 32 of 8-byte pair entries, lane % 16 of 16-byte quad entries
  const uint32_t kslot = (KB != 2) ? (uint32_t)(lane & 31) * 8 : (uint32_t)(lane & 15) * 16;
  const uint32_t vslot = ((VB != 2) ? (uint32_t)(lane & 31) * 8 : (uint32_t)(lane & 15) * 16) | v_table[0];
  float m1 = -1.f;
  asm volatile("" : "+s"(m1));                       // no instruction: keeps -1 from being folded

  float4_t dv[kVDL];
#pragma unroll
  for (int dt = 0; dt < kVDL; ++dt) dv[dt] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;             // softmax reference and sum for this lane's column
  float m_top = -INFINITY;                           // largest score of this lane's rows

  // Tiles alternate between the two tile buffers, each refilled with a newly
  // claimed tile right after use; the explicit vmcnt (the older tile's
  // loads) is the only wait for a tile's data; loads past the end return
  // zeros.
  while (ia < ntiles) {
    uint32_t nx = 0u;
    if (lane == 0) nx = atomicAdd(&next_tile[grp], 1u);
    __builtin_amdgcn_s_waitcnt(kWaitOlderTile);
    if constexpr (X != kSideNone)
      process_tile_side<D, KB, VB, X, false>(ta, sa, side, bk, tab, kslot, vslot, sfac, m1, t0 + ia * kTile, t1, g, n,
                                             dv, m_run, l_run, m_top);
    else
      process_tile<D, KB, VB, false>(ta, bk, tab, kslot, vslot, sfac, m1, t0 + ia * kTile, t1, g, n, dv, m_run, l_run, m_top);
    asm volatile("" : "+v"(nx));                     // keeps the read of the answer here
    const int na = __builtin_amdgcn_readfirstlane(nx);
    load_tile<D, KB, VB>(ta, src, t0 + na * kTile, na >= ntiles);
    load_side<D, X>(sa, side_src, t0 + na * kTile, na >= ntiles);
    int nc = ntiles;
    if (ic < ntiles) {
      uint32_t ny = 0u;
      if (lane == 0) ny = atomicAdd(&next_tile[grp], 1u);
      __builtin_amdgcn_s_waitcnt(kWaitOlderTile);
      if constexpr (X != kSideNone)
        process_tile_side<D, KB, VB, X, false>(tc, sc, side, bk, tab, kslot, vslot, sfac, m1, t0 + ic * kTile, t1, g, n,
                                               dv, m_run, l_run, m_top);
      else
        process_tile<D, KB, VB, false>(tc, bk, tab, kslot, vslot, sfac, m1, t0 + ic * kTile, t1, g, n, dv, m_run, l_run,
                                     m_top);
      asm volatile("" : "+v"(ny));
      nc = __builtin_amdgcn_readfirstlane(ny);
    }
    load_tile<D, KB, VB>(tc, src, t0 + nc * kTile, nc >= ntiles);
    load_side<D, X>(sc, side_src, t0 + nc * kTile, nc >= ntiles);
    ia = na;
    ic = nc;
  }
  // the last split's partial tile [t1f, t1)
  if (gwave == 0 && t1f < t1) {
    load_tail_tile<D, KB, VB>(ta, src, t1f);
    if constexpr (X != kSideNone) {
      load_side_tail<D, X>(sa, side_src, t1f);
      process_tile_side<D, KB, VB, X, true>(ta, sa, side, bk, tab, kslot, vslot, sfac, m1, t1f, t1, g, n, dv, m_run,
                                            l_run, m_top);
    } else {
      process_tile<D, KB, VB, true>(ta, bk, tab, kslot, vslot, sfac, m1, t1f, t1, g, n, dv, m_run, l_run, m_top);
    }
  }

  // ---- wave epilogue: (m, l) per head to LDS; after the barrier (the
  // tables are dead then) the value rows of the heads in use ----
  l_run = sum_rows(add_swap1(l_run));                // both lanes of a head, all four lane rows
  m_top = max_rows(fmaxf(m_top, lane_swap1(m_top)));
  if (lane < 2 * kGMax && !(lane & 1)) {            // lane 2h of the first row: head h
    red_ml[wave][lane >> 1][0] = m_run;
    red_ml[wave][lane >> 1][1] = l_run;
    red_ml[wave][lane >> 1][2] = m_top;
  }
  __syncthreads();                                   // every wave is done with the tables
  float *red_acc = reinterpret_cast<float *>(tab);   // [wave][head][D]
  // accumulator rows 4g, 4g+1 (head 2g) and 4g+2, 4g+3 (head 2g+1);
  // coordinate kVDL n + dt in dv[dt]
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    if (2 * g + hp < G) {
      float *r = red_acc + (size_t)(wave * kGMax + 2 * g + hp) * D + kVDL * n;
#pragma unroll
      for (int q = 0; q < kVDL / 4; ++q)
        *reinterpret_cast<float4_t *>(r + 4 * q) =
            (float4_t){dv[4 * q][2 * hp] + dv[4 * q][2 * hp + 1], dv[4 * q + 1][2 * hp] + dv[4 * q + 1][2 * hp + 1],
                       dv[4 * q + 2][2 * hp] + dv[4 * q + 2][2 * hp + 1], dv[4 * q + 3][2 * hp] + dv[4 * q + 3][2 * hp + 1]};
    }
  }
  // Weight of each wave's rows in its group's merge, one lane of wave 0 per
  // (head h, wave w) (h = tid / 8, w = tid % 8): a group's waves are gw
  // consecutive lanes, reduced with DPP exchanges.  The weight
  // exp2(m_w - M) / (L * code scale) folds in the softmax denominator.
  if (tid < kWaves * kGMax) {
    const int h = tid >> 3, w = tid & (kWaves - 1);
    const float m = red_ml[w][h][0], l = red_ml[w][h][1], mt = red_ml[w][h][2];
    float M = m;
    if (gw > 1) M = fmaxf(M, xor_lane<1>(M, lane));
    if (gw > 2) M = fmaxf(M, xor_lane<2>(M, lane));
    if (gw > 4) M = fmaxf(M, xor_lane<4>(M, lane));
    const float f = (m == -INFINITY) ? 0.f : exp2f(m - M);
    float L = l * f;
    if (gw > 1) L += xor_lane<1>(L, lane);
    if (gw > 2) L += xor_lane<2>(L, lane);
    if (gw > 4) L += xor_lane<4>(L, lane);
    wfac[w][h] = (L > 0.f) ? f / (L * kCodeScale) : 0.f;
    // the split's state is reported against its largest score
    float Mt = mt;
    if (gw > 1) Mt = fmaxf(Mt, xor_lane<1>(Mt, lane));
    if (gw > 2) Mt = fmaxf(Mt, xor_lane<2>(Mt, lane));
    if (gw > 4) Mt = fmaxf(Mt, xor_lane<4>(Mt, lane));
    const int u = (blockIdx.x << lg) + (w >> (3 - lg));
    if ((w & (gw - 1)) == 0 && h < G && u < P.units) {
      const int upr = u / S, usp = u - upr * S;
      const size_t row = ((size_t)upr * G + h) * P.part_stride + usp;
      const bool any = L > 0.f;
      P.part_ml[row * 2 + 0] = any ? Mt * kLn2 : -INFINITY;
      P.part_ml[row * 2 + 1] = any ? L * exp2f(M - Mt) : 0.f;
    }
  }
  __syncthreads();

  // ---- merge each group's waves: one thread per (head, coordinate) ----
  for (int gi = 0; gi < (1 << lg); ++gi) {
    const int u = (blockIdx.x << lg) + gi;
    if (u >= P.units) break;
    const int upr = u / S, usp = u - upr * S;
    for (int i = tid; i < G * D; i += kBlock) {
      const int h = i / D, j = i & (D - 1);
      float o = 0.f;
      for (int w = gi * gw; w < (gi + 1) * gw; ++w) o += red_acc[(size_t)(w * kGMax + h) * D + j] * wfac[w][h];
      P.part_o[(((size_t)upr * G + h) * P.part_stride + usp) * D + j] = o;
    }
  }
}

// log2 of the units per work-group: as few as keep the grid within one
// work-group per compute unit, with at most 8 query rows per work-group.
int wide_group_log2(int64_t units, int G, int cus) {
  int lg = 0;
  while (lg < 3 && (G << (lg + 1)) <= kGMax && ((units + (1 << lg) - 1) >> lg) > (int64_t)cus) ++lg;
  return lg;
}

}  // namespace

bool wide_attend_supported(const AttendArgs &a) {
  const int G = a.q_heads / a.kv_heads;
  const int bits = a.k_format > a.v_format ? a.k_format : a.v_format;
  const bool fits = (int64_t)a.capacity * a.head_dim * bits / 8 < (1ll << 31) &&
                    (int64_t)a.capacity * kOutlierCount < (1ll << 31) &&
                    (int64_t)a.batch * a.kv_heads * a.num_splits < (1ll << 30);
  if (a.num_near_splits != 0 || G < 1 || G > kGMax || !fits) return false;
  // the outlier stream: 4-bit keys and values at d = 128
  if (a.outlier_idx) return a.head_dim == 128 && a.k_format == 4 && a.v_format == 4;
  // the QJL sketch (m = d): 3-bit keys beside 4-bit values at d = 128, the
  // page's 68-byte key
  if (a.qjl_proj) return a.head_dim == 128 && a.k_format == 3 && a.v_format == 4 && G >= 2;
  // 3-bit codes at G = 1 stay on the VALU kernel, which is faster there: the
  // tile's 16 matrix-core columns then carry one head, and 3-bit fields cost
  // two address operations per table read against one for 4-bit bytes
  if (a.head_dim == 128) return a.k_format == 3 && a.v_format == 4 && G >= 2;
  const bool width = a.k_format == 4 || a.k_format == 2 || (a.k_format == 3 && G >= 2);
  return a.head_dim == 256 && a.v_format == a.k_format && width;
}

hipError_t launch_attend_wide(const AttendArgs &a, hipStream_t stream, int part_base) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int G = a.q_heads / a.kv_heads;
  const int64_t units = (int64_t)a.batch * a.kv_heads * a.num_splits;
  const int lg = wide_group_log2(units, G, cus);
  const int chunk = ((a.seq_len + a.num_splits - 1) / a.num_splits + kChunkTok - 1) / kChunkTok * kChunkTok;
  const int D = a.head_dim;
  WParams P{a.q, a.q_f16, a.kv_heads, a.capacity, a.seq_len, a.num_splits, G, chunk, lg, (int)units,
            part_base + a.num_splits, a.k_codes, a.v_codes, a.k_norms, a.v_norms, a.signs, a.k_centroids,
            a.v_centroids, a.part_o + (size_t)part_base * D, a.part_ml + (size_t)part_base * 2,
            a.outlier_idx, a.outlier_codes, a.outlier_scales, a.qjl_proj, a.qjl_signs, a.qjl_norms};
  dim3 grid((unsigned)((units + (1 << lg) - 1) >> lg));
  if (a.outlier_idx) hipLaunchKernelGGL((attend_wide_kernel<128, 4, 4, kSideOut>), grid, dim3(kBlock), 0, stream, P);
  else if (a.qjl_proj) hipLaunchKernelGGL((attend_wide_kernel<128, 3, 4, kSideQjl>), grid, dim3(kBlock), 0, stream, P);
  else if (D == 128) hipLaunchKernelGGL((attend_wide_kernel<128, 3, 4, kSideNone>), grid, dim3(kBlock), 0, stream, P);
  else if (a.k_format == 4) hipLaunchKernelGGL((attend_wide_kernel<256, 4, 4, kSideNone>), grid, dim3(kBlock), 0, stream, P);
  else if (a.k_format == 3) hipLaunchKernelGGL((attend_wide_kernel<256, 3, 3, kSideNone>), grid, dim3(kBlock), 0, stream, P);
  else hipLaunchKernelGGL((attend_wide_kernel<256, 2, 2, kSideNone>), grid, dim3(kBlock), 0, stream, P);
  return hipGetLastError();
}

}  // namespace kvq
