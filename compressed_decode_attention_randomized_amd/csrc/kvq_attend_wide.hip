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
  // key outlier stream (OUT kernels): [b * Hkv + KV head][8] channels,
  // [..][capacity][8] int8 codes, [..][capacity] scales
  const int32_t *out_idx;
  const int8_t *out_codes;
  const float *out_scales;
};

// Outlier stream registers of one tile: the int8 codes (two 8-byte rows)
// and scales of the lane's two tokens 4g + 2 (n & 1) + {0, 1}.
struct OutTile {
  uint4_t oc;
  uint2_t os;
};

struct OutSources {
  const int8_t *oc;
  const float *os;
  uint32_t code_bytes, scale_bytes;
  uint32_t co, so;                     // per-lane offsets
};

__device__ inline void load_out(OutTile &t, const OutSources &src, int tb, bool skip) {
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(src.oc, skip ? 0u : src.code_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(src.os, skip ? 0u : src.scale_bytes);
  t.oc = __builtin_amdgcn_raw_buffer_load_b128(cr, src.co, tb * kOutlierCount, kStream);
  t.os = __builtin_amdgcn_raw_buffer_load_b64(sr, src.so, tb * 4, kStream);
}

// The partial last tile: descriptors from the tile to the slice's end.
__device__ inline void load_out_tail(OutTile &t, const OutSources &src, int tb) {
  OutSources s = src;
  s.oc += (size_t)tb * kOutlierCount;
  s.os += tb;
  s.code_bytes -= (uint32_t)tb * kOutlierCount;
  s.scale_bytes -= (uint32_t)tb * 4;
  load_out(t, s, 0, false);
}

// scale * sum_k qo_k code_k for the lane's two tokens (qo: q at the channels
// times log2(e) / sqrt(d), zero for unused columns).
__device__ inline void outlier_terms(const OutTile &t, const float (&qo)[kOutlierCount], float (&s)[2]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t w0 = u ? t.oc.z : t.oc.x, w1 = u ? t.oc.w : t.oc.y;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kOutlierCount; ++k) {
      const uint32_t w = (k < 4) ? w0 : w1;
      const float c = (float)(int8_t)(uint8_t)(w >> (8 * (k & 3)));
      acc = __builtin_fmaf(qo[k], c, acc);
    }
    s[u] = __builtin_fmaf(__builtin_bit_cast(float, u ? t.os.y : t.os.x), acc, s[u]);
  }
}

// process_tile with the outlier stream's term added before the softmax update.
template <int D, bool TAIL>
__device__ inline void process_tile_out(const Tile<D, 4, 4> &t, const OutTile &ot, const float (&qo)[kOutlierCount],
                                        const uint4_t (&bk)[D / 16], const uint8_t *tab, uint32_t kslot, uint32_t vslot,
                                        float sfac, float m1, int tb, int t1, int g, int n, float4_t (&dv)[D / 16],
                                        float &m_run, float &l_run, float &m_top) {
  float4_t dk = {0.f, 0.f, 0.f, 0.f};
  key_scores<D, 4>(t.kw, bk, tab, kslot, dk);
  const bool odd = n & 1;
  const uint32_t knp = odd ? t.kn.y : t.kn.x;
  const uint32_t vnp = odd ? t.vn.y : t.vn.x;
  float s[2];
  raw_scores<true>(dk, knp, sfac, n, s);
  outlier_terms(ot, qo, s);
  tile_update<D, TAIL>(s, tb, t1, g, n, dv, m_run, l_run, m_top);
  ValueBytes<D, 4> vb;
  value_bytes<D, 4>(t, vb, n);
  const half8_t aw = tile_weights<TAIL, true>(s, vnp, m1, n, m_run, l_run);
  value_update<D, 4>(vb, tab, vslot, aw, dv);
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

template <int D, int KB, int VB, bool OUT>
__global__ __launch_bounds__(kBlock, kMinWaves) void attend_wide_kernel(WParams P) {
  static_assert(D == 256 || (D == 128 && VB == 4 && KB >= 3), "head dimension 256, or 128 with 4-bit values");
  static_assert(!OUT || (KB == 4 && VB == 4), "the outlier stream beside 4-bit codes");
  using TileT = Tile<D, KB, VB>;
  constexpr int kKRow = TileT::kKRow, kVRow = TileT::kVRow;
  constexpr int kVDL = D / 16;                    // value coordinates per lane
  constexpr int kRowPad = D + 4;                  // query table row stride (words)
  constexpr int kLoads = kTileLoads<D, KB, VB> + (OUT ? 2 : 0);
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
  OutSources osrc;
  if constexpr (OUT) {
    osrc.oc = P.out_codes + (size_t)pr * cap * kOutlierCount;
    osrc.os = P.out_scales + (size_t)pr * cap;
    osrc.code_bytes = cap * kOutlierCount;
    osrc.scale_bytes = cap * 4;
    osrc.co = (uint32_t)(4 * g + 2 * (n & 1)) * kOutlierCount;
    osrc.so = (uint32_t)(4 * g + 2 * (n & 1)) * 4;
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
  OutTile oa, oc;
  if (wave < kSetupWaves) {
    fill_tables<KB, VB>(tab, P.k_centroids, P.v_centroids, wave, lane, tid, v_table);
    if (tid < D) qtab[kZeroRow][tid] = 0u;

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
      if constexpr (E == 4) {
        // both forms are read; the one of the other element size goes unused
        // (for fp16 rows its upper lanes lie past the row and read as zero)
        const uint2_t qh = __builtin_amdgcn_raw_buffer_load_b64(qsrc, lane * 8, 0, 0);
        const uint4_t qf = __builtin_amdgcn_raw_buffer_load_b128(qsrc, lane * 16, 0, 0);
        const uint32_t sg = __builtin_amdgcn_raw_buffer_load_b32(ssrc, lane * 4, 0, 0);   // signs of 4l..4l+3
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t hw = (e < 2) ? qh.x : qh.y;
          const float v = q_f16 ? half_value((hw >> (16 * (e & 1))) & 0xFFFFu) : __builtin_bit_cast(float, qf[e]);
          z[e] = ((sg >> (8 * e + 7)) & 1u) ? -v : v;
        }
        const float a0 = z[0] + z[1], a1 = z[0] - z[1], a2 = z[2] + z[3], a3 = z[2] - z[3];
        z[0] = a0 + a2;
        z[1] = a1 + a3;
        z[2] = a0 - a2;
        z[3] = a1 - a3;
      } else {
        const uint32_t qh = __builtin_amdgcn_raw_buffer_load_b32(qsrc, lane * 4, 0, 0);
        const uint2_t qf = __builtin_amdgcn_raw_buffer_load_b64(qsrc, lane * 8, 0, 0);
        const uint32_t sg = __builtin_amdgcn_raw_buffer_load_b16(ssrc, lane * 2, 0, 0);   // signs of 2l, 2l+1
        const float v0 = q_f16 ? half_value(qh & 0xFFFFu) : __builtin_bit_cast(float, qf.x);
        const float v1 = q_f16 ? half_value(qh >> 16) : __builtin_bit_cast(float, qf.y);
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
  if constexpr (OUT) load_out(oa, osrc, t0 + ia * kTile, ia >= ntiles);
  __builtin_amdgcn_sched_barrier(0);
  load_tile<D, KB, VB>(tc, src, t0 + ic * kTile, ic >= ntiles);
  if constexpr (OUT) load_out(oc, osrc, t0 + ic * kTile, ic >= ntiles);
  __builtin_amdgcn_sched_barrier(0);

  // Wait for the set-up counts (bounded: every set-up wave reaches its count
  // without waiting on anything but its own loads).
  for (int spin = 0; spin < kSpinLimit; ++spin) {
    const uint32_t r = __hip_atomic_load(&ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(r) >= (uint32_t)kSetupWaves) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  // B operand of key block kb for column n: the group's query row 2h + form
  // for n = 2h + form < 2G (the zero row otherwise), coordinates
  // 64g + 4kb .. +3
  const bool col = n < 2 * G;
  const int qrow = col ? grp * 2 * G + n : kZeroRow;
  uint4_t bk[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) bk[kb] = *reinterpret_cast<const uint4_t *>(&qtab[qrow][g * (D / 4) + 4 * kb]);
  const float sfac = col ? qfac[grp * G + (n >> 1)] : 0.f;
  float qo[kOutlierCount];
#pragma unroll
  for (int k = 0; k < kOutlierCount; ++k) qo[k] = 0.f;
  if constexpr (OUT) {
    if (col) {
#pragma unroll
      for (int k = 0; k < kOutlierCount; ++k) qo[k] = qout[grp * G + (n >> 1)][k];
    }
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
    if constexpr (OUT)
      process_tile_out<D, false>(ta, oa, qo, bk, tab, kslot, vslot, sfac, m1, t0 + ia * kTile, t1, g, n, dv, m_run, l_run,
                                 m_top);
    else
      process_tile<D, KB, VB, false>(ta, bk, tab, kslot, vslot, sfac, m1, t0 + ia * kTile, t1, g, n, dv, m_run, l_run, m_top);
    asm volatile("" : "+v"(nx));                     // keeps the read of the answer here
    const int na = __builtin_amdgcn_readfirstlane(nx);
    load_tile<D, KB, VB>(ta, src, t0 + na * kTile, na >= ntiles);
    if constexpr (OUT) load_out(oa, osrc, t0 + na * kTile, na >= ntiles);
    int nc = ntiles;
    if (ic < ntiles) {
      uint32_t ny = 0u;
      if (lane == 0) ny = atomicAdd(&next_tile[grp], 1u);
      __builtin_amdgcn_s_waitcnt(kWaitOlderTile);
      if constexpr (OUT)
        process_tile_out<D, false>(tc, oc, qo, bk, tab, kslot, vslot, sfac, m1, t0 + ic * kTile, t1, g, n, dv, m_run,
                                   l_run, m_top);
      else
        process_tile<D, KB, VB, false>(tc, bk, tab, kslot, vslot, sfac, m1, t0 + ic * kTile, t1, g, n, dv, m_run, l_run,
                                     m_top);
      asm volatile("" : "+v"(ny));
      nc = __builtin_amdgcn_readfirstlane(ny);
    }
    load_tile<D, KB, VB>(tc, src, t0 + nc * kTile, nc >= ntiles);
    if constexpr (OUT) load_out(oc, osrc, t0 + nc * kTile, nc >= ntiles);
    ia = na;
    ic = nc;
  }
  // the last split's partial tile [t1f, t1)
  if (gwave == 0 && t1f < t1) {
    load_tail_tile<D, KB, VB>(ta, src, t1f);
    if constexpr (OUT) {
      load_out_tail(oa, osrc, t1f);
      process_tile_out<D, true>(ta, oa, qo, bk, tab, kslot, vslot, sfac, m1, t1f, t1, g, n, dv, m_run, l_run, m_top);
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
  if (a.qjl_proj || a.num_near_splits != 0 || G < 1 || G > kGMax || !fits) return false;
  // the outlier stream: 4-bit keys and values at d = 128
  if (a.outlier_idx) return a.head_dim == 128 && a.k_format == 4 && a.v_format == 4;
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
            a.outlier_idx, a.outlier_codes, a.outlier_scales};
  dim3 grid((unsigned)((units + (1 << lg) - 1) >> lg));
  if (a.outlier_idx) hipLaunchKernelGGL((attend_wide_kernel<128, 4, 4, true>), grid, dim3(kBlock), 0, stream, P);
  else if (D == 128) hipLaunchKernelGGL((attend_wide_kernel<128, 3, 4, false>), grid, dim3(kBlock), 0, stream, P);
  else if (a.k_format == 4) hipLaunchKernelGGL((attend_wide_kernel<256, 4, 4, false>), grid, dim3(kBlock), 0, stream, P);
  else if (a.k_format == 3) hipLaunchKernelGGL((attend_wide_kernel<256, 3, 3, false>), grid, dim3(kBlock), 0, stream, P);
  else hipLaunchKernelGGL((attend_wide_kernel<256, 2, 2, false>), grid, dim3(kBlock), 0, stream, P);
  return hipGetLastError();
}

}  // namespace kvq
