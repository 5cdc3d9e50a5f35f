// Tile processing shared by the pair-table attention kernels (4-bit Lloyd-Max
// keys and values): matrix-core products fed from a byte-indexed pair table.
//
// Each packed byte holds two 4-bit codes.  The LDS table maps a byte to the
// operand registers of both codes at once: entry(byte) = (e(c[lo]), e(c[hi])),
// e(x) the fp16 (hi, lo) split of x = RN(x) + RN(x - RN(x)) in one 32-bit
// word.  So one 64-bit LDS read serves two codes and needs one address op.
// The table is replicated over 32 lane slots (address = byte*256 + slot*8,
// slot = lane % 32) so that the 32 lanes an LDS cycle serves use all 64 banks
// and never meet in one; a separate value table follows the key table at
// +64 KB.  The address is one v_perm: slot*8 (and the +64 KB) from a per-lane
// register, the code byte in byte 1.
//
// A tile is 16 tokens; lane l = 16g + n of a wave:
//   keys    token n of the tile in A row n; the byte pair (2kb, 2kb+1) of the
//           lane's D/8-byte slice (coordinates [D/4 g, D/4 (g+1))) gives
//           coordinates 4kb..4kb+3 of the slice as k-slot pairs (c_hi, c_lo);
//           B column 2h holds (z_hi, z_hi) of head h and column 2h+1 holds
//           (z_lo, 0), so columns 2h + 2h+1 give the score of head h up to
//           the fp32 accumulation.
//   values  tokens 4g..4g+3, coordinates [D/16 n, D/16 (n+1)); k-slot pairs
//           are the 4 tokens of the lane group; a value byte built from the
//           same coordinate of two tokens (low nibble token t, high nibble
//           token t+1) reads both tokens' (c_hi, c_lo) at once; A row 2h holds
//           (w_hi, w_hi) and row 2h+1 (w_lo, w_lo) of head h's weight
//           w = exp2(score - max) * norm, so the two halves of a head land in
//           the same lane of the accumulator.
// Sources: "The Engineering Behind AdapTQ", "Engineering the Hot Path"
// (rotate q once, score from codes through a table, no dequantize pass);
// "FoveatedKV", "Making it fast" (pre-scaled q, online softmax with one exp
// per score); "I Ported a Google Research Paper to Apple Silicon", "The
// Bit-Packing Problem" (4-bit codes, low nibble first).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_lane.h"

namespace kvq {
namespace pair {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));

constexpr int kTile = 16;
constexpr int kChunkTok = 32;                   // split chunks are multiples of this many tokens
constexpr int kGMax = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kCodeScale = 256.f;             // centroid scale: keeps the low fp16 half a normal number
// The softmax reference (log2 units) is moved only when a score passes it,
// and then to the column maximum plus this slack: weights stay <= 1, the
// largest at least 2^-kSlack, and most tiles skip the accumulator rescale.
constexpr float kSlack = 4.f;
constexpr int kRawBufferFlags = 0x00020000;     // 32-bit data format, untyped raw access
constexpr uint32_t kNib = 0x0F0F0F0Fu;
constexpr int kStream = 2;                      // cache policy nt: the cache is read once per step
constexpr int kSpinLimit = 1 << 20;             // bound of the set-up wait (s_sleep 1 each)

__device__ inline uint32_t pack2(_Float16 a, _Float16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ inline half8_t as_half8(uint2_t a, uint2_t b) {
  const uint4_t v = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(half8_t, v);
}

__device__ inline float half_value(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }

// (hi, lo) fp16 split of x in one word: hi = RN(x), lo = RN(x - hi).
__device__ inline uint32_t split_entry(float x) {
  const _Float16 hi = (_Float16)x;
  return pack2(hi, (_Float16)(x - (float)hi));
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBufferFlags);
}

// Table address of code byte B of `word` in one v_perm: byte 0 and byte 2
// come from the lane's slot register (slot * 8, plus 1 in byte 2 for the
// value table), byte 1 is the code byte, byte 3 is zero.
template <int B>
__device__ inline uint32_t pair_addr(uint32_t word, uint32_t slotreg) {
  return __builtin_amdgcn_perm(word, slotreg, 0x0C020000u | ((4u + B) << 8));
}

__device__ inline uint2_t table_read(const uint8_t *tab, uint32_t addr) {
  return *reinterpret_cast<const uint2_t *>(tab + addr);
}

// xor-1 exchange (DPP quad permutation [1, 0, 3, 2]).
__device__ inline float lane_swap1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}

__device__ inline uint32_t swap1_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}

// x + (x of lane l ^ 1); written as a DPP update with a zero old value so
// that the exchange folds into the add (one v_add_f32_dpp).
__device__ inline float add_swap1(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}

// o[i] = c[B + S*i] for the key and value centroid tables.
template <int B, int S, int N>
__device__ inline void pick(const float (&ck)[16], const float (&cv)[16], float (&ok)[N], float (&ov)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    ok[i] = ck[B + S * i];
    ov[i] = cv[B + S * i];
  }
}

// o[i] = c[B + i], i = 0..3, of one centroid table.
template <int B>
__device__ inline void pick1(const float (&c)[16], float (&o)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = c[B + i];
}

// f16(half H of a packed pair) * f: one v_fma_mix_f32 (the fma with a zero
// addend of a converted fp16 and an fp32 value, rounded once to fp32:
// equal to a conversion then a multiply).
template <int H>
__device__ inline float half_mul(uint32_t packed, float f) {
  return __builtin_fmaf(half_value(packed >> (16 * H)), f, 0.f);
}

// hp = (RN(w0), RN(w1)) and lp = (RN(w0 - hi0), RN(w1 - hi1)) as fp16
// pairs.  m1 holds -1 where the compiler cannot fold it, so the low parts
// stay fused multiply-adds of an fp16 and two fp32 operands (v_fma_mix).
__device__ inline void split_pair(float w0, float w1, float m1, uint32_t &hp, uint32_t &lp) {
  const half2_t h = {(_Float16)w0, (_Float16)w1};
  const half2_t l = {(_Float16)__builtin_fmaf((float)h.x, m1, w0), (_Float16)__builtin_fmaf((float)h.y, m1, w1)};
  hp = __builtin_bit_cast(uint32_t, h);
  lp = __builtin_bit_cast(uint32_t, l);
}

// Registers of one tile for head dimension D (128 or 256), KB-bit key codes
// and VB-bit value codes (4; 2 with quad entries, see quad_read; 3 with
// 6-bit pair fields, see field_addr; 3-bit values at D = 256 only).
template <int D, int KB = 4, int VB = KB>
struct Tile {
  static_assert(VB != 3 || D == 256, "3-bit value tiles are laid out for head dimension 256");
  static constexpr int kKRow = D * KB / 8;        // packed key bytes per vector
  static constexpr int kVRow = D * VB / 8;        // packed value bytes per vector
  static constexpr int kKeyWords = kKRow / 16;    // key slice: token n, bytes [kKRow/4 g, kKRow/4 (g+1))
  // value words per token: bytes [kVRow/16 n, kVRow/16 (n+1)); for 3-bit codes
  // (6 bytes at 6n) the 8 bytes from the word boundary at or below 6n
  static constexpr int kValWords = (VB == 3) ? 2 : kVRow / 64;
  // buffer loads of the key slice: 16-byte loads, or for 3-bit codes (a
  // slice starting on 4 or 8 bytes) 8-byte loads and a 4-byte one for an odd word
  static constexpr int kKeyLoads = (KB == 3) ? (kKeyWords + 1) / 2 : kKeyWords / 4;
  uint32_t kw[kKeyWords];
  uint32_t vw[4][kValWords];                      // tokens 4g+i
  uint2_t kn, vn;                                 // fp16 norms of tokens 4g..4g+3
};

// Per (b, KV head) cache slices; a tile's loads use a per-lane constant
// VGPR offset and the tile's token offset in an SGPR (no per-tile vector
// address arithmetic).
struct Sources {
  const uint8_t *kc, *vc;
  const uint16_t *kn, *vn;
  uint32_t kcode_bytes, vcode_bytes, norm_bytes;
  uint32_t ko, vo, no;                 // per-lane offsets: key slice, value word, norm pair
};

// Every code width gives lane (g, n) the key coordinates [D/4 g, D/4 (g+1))
// of token n and the value coordinates [D/16 n, D/16 (n+1)) of tokens
// 4g..4g+3.
template <int D, int KB = 4, int VB = KB>
__device__ inline void set_offsets(Sources &src, int g, int n) {
  constexpr int kKRow = Tile<D, KB, VB>::kKRow, kVRow = Tile<D, KB, VB>::kVRow;
  src.ko = n * kKRow + g * (kKRow / 4);
  src.vo = 4 * g * kVRow + ((VB == 3) ? (n * (kVRow / 16)) & ~3 : n * (kVRow / 16));
  src.no = 4 * g * 2;
}

// Loads of the tile at token tb.  A skipped tile reads through descriptors
// of size zero, where buffer loads return zeros without touching memory, so
// loads need no branch and a tile's wait sits at its first use.
template <int D, int KB = 4, int VB = KB>
__device__ inline void load_tile(Tile<D, KB, VB> &t, const Sources &src, int tb, bool skip) {
  using T = Tile<D, KB, VB>;
  const __amdgpu_buffer_rsrc_t kc = make_rsrc(src.kc, skip ? 0u : src.kcode_bytes);
  const __amdgpu_buffer_rsrc_t vc = make_rsrc(src.vc, skip ? 0u : src.vcode_bytes);
  const __amdgpu_buffer_rsrc_t kn = make_rsrc(src.kn, skip ? 0u : src.norm_bytes);
  const __amdgpu_buffer_rsrc_t vn = make_rsrc(src.vn, skip ? 0u : src.norm_bytes);
  const int ks = tb * T::kKRow, vs = tb * T::kVRow, ns = tb * 2;
  if constexpr (KB == 3) {
#pragma unroll
    for (int i = 0; i < T::kKeyWords / 2; ++i) {
      const uint2_t k = __builtin_amdgcn_raw_buffer_load_b64(kc, src.ko + 8 * i, ks, kStream);
      t.kw[2 * i] = k.x;
      t.kw[2 * i + 1] = k.y;
    }
    if constexpr (T::kKeyWords % 2)
      t.kw[T::kKeyWords - 1] = __builtin_amdgcn_raw_buffer_load_b32(kc, src.ko + 4 * (T::kKeyWords - 1), ks, kStream);
  } else {
#pragma unroll
    for (int i = 0; i < T::kKeyWords / 4; ++i) {
      const uint4_t k = __builtin_amdgcn_raw_buffer_load_b128(kc, src.ko + 16 * i, ks, kStream);
#pragma unroll
      for (int e = 0; e < 4; ++e) t.kw[4 * i + e] = k[e];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (T::kValWords == 1) {
      t.vw[i][0] = __builtin_amdgcn_raw_buffer_load_b32(vc, src.vo + i * T::kVRow, vs, kStream);
    } else {
      const uint2_t v = __builtin_amdgcn_raw_buffer_load_b64(vc, src.vo + i * T::kVRow, vs, kStream);
      t.vw[i][0] = v.x;
      t.vw[i][1] = v.y;
    }
  }
  t.kn = __builtin_amdgcn_raw_buffer_load_b64(kn, src.no, ns, kStream);
  t.vn = __builtin_amdgcn_raw_buffer_load_b64(vn, src.no, ns, kStream);
}

// Loads of the partial last tile at token tb through descriptors that start
// at the tile and end at the slice's end: its rows past the slice read as
// zero from the descriptor's range check on the lane offset alone (the
// full-tile loads above keep the tile offset in a scalar register; their
// rows always lie inside the slice).
template <int D, int KB = 4, int VB = KB>
__device__ inline void load_tail_tile(Tile<D, KB, VB> &t, const Sources &src, int tb) {
  using T = Tile<D, KB, VB>;
  Sources s = src;
  s.kc += (size_t)tb * T::kKRow;
  s.vc += (size_t)tb * T::kVRow;
  s.kn += tb;
  s.vn += tb;
  s.kcode_bytes -= (uint32_t)tb * T::kKRow;
  s.vcode_bytes -= (uint32_t)tb * T::kVRow;
  s.norm_bytes -= (uint32_t)tb * 2;
  load_tile<D, KB, VB>(t, s, 0, false);
}

// Buffer loads one tile issues (the s_waitcnt vmcnt that leaves one tile in flight).
template <int D, int KB = 4, int VB = KB>
constexpr int kTileLoads = Tile<D, KB, VB>::kKeyLoads + 4 + 2;

// 2-bit codes: a byte holds four codes, and the quad table maps it to
// (e(c[b & 3]), e(c[(b >> 2) & 3]), e(c[(b >> 4) & 3]), e(c[b >> 6])), 16
// bytes: one 128-bit LDS read gives a whole 8-half MFMA operand.  The table
// is replicated over 16 lane slots (address = byte*256 + slot*16, slot =
// lane % 16): an LDS cycle serves 16 lanes of a 128-bit read, which then use
// all 64 banks.
__device__ inline uint4_t quad_read(const uint8_t *tab, uint32_t addr) {
  return *reinterpret_cast<const uint4_t *>(tab + addr);
}

// 3-bit codes: two neighbouring codes form a 6-bit field (the first code in
// its low three bits), and the pair table maps a field f to (e(c[f & 7]),
// e(c[f >> 3])), 8 bytes, replicated over 32 lane slots like the 4-bit
// table (address = f*256 + slot*8).  The field at bit P of a lane's packed
// words, as that address: a bit-field extract and a shift-or, or for a field
// across a word boundary a funnel shift and an and-or.
template <int P, int N>
__device__ inline uint32_t field_addr(const uint32_t (&w)[N], uint32_t slot) {
  constexpr int W = P / 32, O = P % 32;
  if constexpr (O + 6 <= 32) {
    return (__builtin_amdgcn_ubfe(w[W], (uint32_t)O, 6u) << 8) | slot;
  } else {
    static_assert(W + 1 < N, "field past the lane's words");
    return (__builtin_amdgcn_alignbit(w[W + 1], w[W], (uint32_t)(O - 8)) & 0x3F00u) | slot;
  }
}

// Key block kb: coordinates 4kb..4kb+3 of the lane's slice = bytes 2kb, 2kb+1
// (4-bit), byte kb (2-bit) or the fields at bits 12kb and 12kb+6 (3-bit).
template <int D, int BITS, int KB = 0, int N>
__device__ inline void key_scores(const uint32_t (&kw)[N], const uint4_t (&bk)[D / 16], const uint8_t *tab,
                                  uint32_t slot, float4_t &dk) {   // slot: key slot register
  if constexpr (KB < D / 16) {
    half8_t a;
    if constexpr (BITS == 4) {
      const uint32_t w = kw[KB / 2];
      const uint2_t e0 = table_read(tab, pair_addr<2 * (KB % 2)>(w, slot));
      const uint2_t e1 = table_read(tab, pair_addr<2 * (KB % 2) + 1>(w, slot));
      a = as_half8(e0, e1);
    } else if constexpr (BITS == 3) {
      a = as_half8(table_read(tab, field_addr<12 * KB>(kw, slot)), table_read(tab, field_addr<12 * KB + 6>(kw, slot)));
    } else {
      a = __builtin_bit_cast(half8_t, quad_read(tab, pair_addr<KB % 4>(kw[KB / 4], slot)));
    }
    dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8_t, bk[KB]), dk, 0, 0, 0);
    key_scores<D, BITS, KB + 1, N>(kw, bk, tab, slot, dk);
  }
}

// Value bytes of one coordinate across the lane group's tokens, and the
// coordinate tiles they feed.
//   4-bit: byte m of word w of ev[w][p] (od[w][p]) holds coordinate
//          8w + 2m (8w + 2m + 1) of tokens 4g+2p (low nibble) and 4g+2p+1;
//          two pair-table reads give the operand of tile 8w + 2m (+1).
//   2-bit: byte j of x[r] holds coordinate 4j + r of tokens 4g..4g+3 (2 bits
//          each, token 4g lowest); one quad-table read gives the operand of
//          tile 4j + r.
//   3-bit: the 6-bit field j of ev[c][p] (od[c][p]) holds coordinate
//          8c + 2j (8c + 2j + 1) of tokens 4g+2p (low three bits) and
//          4g+2p+1; two pair-table reads give the operand of tile 8c + 2j
//          (+1).
template <int D, int BITS>
struct ValueBytes {
  static constexpr int kWords = (BITS == 4) ? D / 128 : (BITS == 3) ? 2 : 1;
  uint32_t ev[kWords][2], od[kWords][2];
  uint32_t x[4];
};

template <int D, int BITS, int KB>
__device__ inline void value_bytes(const Tile<D, KB, BITS> &t, ValueBytes<D, BITS> &vb, int n) {
  if constexpr (BITS == 3) {
    // lane n's 16 codes of a token start at bit 16 (n & 1) of its two words;
    // c0: codes 0..7 (coordinates 16n..16n+7), c1: codes 8..15, each in the
    // low 24 bits (bits above are ignored)
    const uint32_t sh = (uint32_t)(n & 1) * 16u;
    uint32_t c0[4], c1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c0[i] = __builtin_amdgcn_alignbit(t.vw[i][1], t.vw[i][0], sh);
      c1[i] = __builtin_amdgcn_alignbit(t.vw[i][1] >> sh, c0[i], 24u);
    }
    constexpr uint32_t kLow3 = 0x001C71C7u;         // bits 6j..6j+2, j = 0..3
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      vb.ev[0][p] = (c0[2 * p] & kLow3) | ((c0[2 * p + 1] << 3) & ~kLow3);
      vb.od[0][p] = ((c0[2 * p] >> 3) & kLow3) | (c0[2 * p + 1] & ~kLow3);
      vb.ev[1][p] = (c1[2 * p] & kLow3) | ((c1[2 * p + 1] << 3) & ~kLow3);
      vb.od[1][p] = ((c1[2 * p] >> 3) & kLow3) | (c1[2 * p + 1] & ~kLow3);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int w = 0; w < D / 128; ++w) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        vb.ev[w][p] = (t.vw[2 * p][w] & kNib) | ((t.vw[2 * p + 1][w] << 4) & ~kNib);
        vb.od[w][p] = ((t.vw[2 * p][w] >> 4) & kNib) | (t.vw[2 * p + 1][w] & ~kNib);
      }
    }
  } else {
    static_assert(Tile<D, KB, BITS>::kValWords == 1, "one value word per token");
    constexpr uint32_t kCrumb = 0x33333333u;
    // nibble k of a01: coordinate 2k of tokens 0 (bits 0-1) and 1 (bits
    // 2-3); of b01: coordinate 2k+1; likewise a23, b23 for tokens 2, 3
    const uint32_t w0 = t.vw[0][0], w1 = t.vw[1][0], w2 = t.vw[2][0], w3 = t.vw[3][0];
    const uint32_t a01 = (w0 & kCrumb) | ((w1 << 2) & ~kCrumb), b01 = ((w0 >> 2) & kCrumb) | (w1 & ~kCrumb);
    const uint32_t a23 = (w2 & kCrumb) | ((w3 << 2) & ~kCrumb), b23 = ((w2 >> 2) & kCrumb) | (w3 & ~kCrumb);
    // byte j: coordinates 4j (x[0]), 4j+1 (x[1]), 4j+2 (x[2]), 4j+3 (x[3])
    vb.x[0] = (a01 & kNib) | ((a23 << 4) & ~kNib);
    vb.x[2] = ((a01 >> 4) & kNib) | (a23 & ~kNib);
    vb.x[1] = (b01 & kNib) | ((b23 << 4) & ~kNib);
    vb.x[3] = ((b01 >> 4) & kNib) | (b23 & ~kNib);
  }
}

template <int D, int BITS, int M = 0>
__device__ inline void value_update(const ValueBytes<D, BITS> &vb, const uint8_t *tab, uint32_t slot,
                                    const half8_t &aw, float4_t (&dv)[D / 16]) {
  if constexpr (BITS == 4) {
    if constexpr (M < D / 32) {
      constexpr int W = M / 4, B = M % 4;
      const uint2_t a0 = table_read(tab, pair_addr<B>(vb.ev[W][0], slot));
      const uint2_t a1 = table_read(tab, pair_addr<B>(vb.ev[W][1], slot));
      dv[2 * M] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, as_half8(a0, a1), dv[2 * M], 0, 0, 0);
      const uint2_t b0 = table_read(tab, pair_addr<B>(vb.od[W][0], slot));
      const uint2_t b1 = table_read(tab, pair_addr<B>(vb.od[W][1], slot));
      dv[2 * M + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, as_half8(b0, b1), dv[2 * M + 1], 0, 0, 0);
      value_update<D, BITS, M + 1>(vb, tab, slot, aw, dv);
    }
  } else if constexpr (BITS == 3) {
    if constexpr (M < D / 16) {
      constexpr int C = M / 8, J = (M % 8) / 2;      // tile M = 8C + 2J (+1 for the odd words)
      const uint32_t(&w)[2] = (M & 1) ? vb.od[C] : vb.ev[C];
      const uint2_t a0 = table_read(tab, (__builtin_amdgcn_ubfe(w[0], 6u * J, 6u) << 8) | slot);
      const uint2_t a1 = table_read(tab, (__builtin_amdgcn_ubfe(w[1], 6u * J, 6u) << 8) | slot);
      dv[M] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, as_half8(a0, a1), dv[M], 0, 0, 0);
      value_update<D, BITS, M + 1>(vb, tab, slot, aw, dv);
    }
  } else {
    if constexpr (M < D / 16) {
      constexpr int J = M / 4, R = M % 4;          // tile M = 4J + R
      const uint4_t e = quad_read(tab, pair_addr<J>(vb.x[R], slot));
      dv[M] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, e), dv[M], 0, 0, 0);
      value_update<D, BITS, M + 1>(vb, tab, slot, aw, dv);
    }
  }
}

// The online-softmax step of one 16-token tile, shared by the code tiles
// and the fp16 near-tier tiles of the head-dimension-128 kernel.  TAIL masks
// tokens at or past t1.
//
// Columns 2h and 2h+1 of the score tile dk hold the two parts of head h's
// scores, so lanes 2h and 2h+1 of a lane row share the work of their four
// tokens: lane 2h finishes tokens 4g, 4g+1 and lane 2h+1 tokens 4g+2, 4g+3
// (one exponential per score), then they trade weight halves: A row 2h takes
// the high fp16 parts of all four weights, row 2h+1 the low parts.  Both
// lanes of a head keep the same softmax reference.
//
// tile_scores: the lane's two scores, scaled by sfac times the tokens' fp16
// key norms (knp, NORMS) or by sfac alone (raw_scores), then the state moved
// (and the accumulator rescaled) when a score passes the reference
// (tile_update, which masks tokens at or past t1 first).  A key side stream
// adds its term to the raw scores before the update.
template <bool NORMS>
__device__ inline void raw_scores(const float4_t &dk, uint32_t knp, float sfac, int n, float (&s)[2]) {
  const bool odd = n & 1;
  const float f0 = add_swap1(dk[0]), f1 = add_swap1(dk[1]), f2 = add_swap1(dk[2]), f3 = add_swap1(dk[3]);
  if constexpr (NORMS) {
    s[0] = (odd ? f2 : f0) * half_mul<0>(knp, sfac);
    s[1] = (odd ? f3 : f1) * half_mul<1>(knp, sfac);
  } else {
    s[0] = (odd ? f2 : f0) * sfac;
    s[1] = (odd ? f3 : f1) * sfac;
  }
}

template <int D, bool TAIL>
__device__ inline void tile_update(float (&s)[2], int tb, int t1, int g, int n, float4_t (&dv)[D / 16], float &m_run,
                                   float &l_run, float &m_top) {
  if constexpr (TAIL) {
    const int tok = tb + 4 * g + 2 * (n & 1);
    s[0] = (tok < t1) ? s[0] : -INFINITY;
    s[1] = (tok + 1 < t1) ? s[1] : -INFINITY;
  }
  float mt = fmaxf(s[0], s[1]);

  // The column maximum over the four lane rows is needed only when some
  // lane's scores pass the reference (then the rescale below runs).
  m_top = (mt > m_top) ? mt : m_top;
  if (__builtin_amdgcn_ballot_w64(mt > m_run) != 0) {
    mt = max_rows(mt);
    mt = fmaxf(mt, lane_swap1(mt));
    const float mn = (mt > m_run) ? mt + kSlack : m_run;
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
    l_run *= alpha;
    m_run = mn;
    // accumulator rows 4g, 4g+1 belong to head 2g, rows 4g+2, 4g+3 to head 2g+1
    const float a0 = __shfl(alpha, 4 * g), a1 = __shfl(alpha, 4 * g + 2);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      dv[dt][0] *= a0;
      dv[dt][1] *= a0;
      dv[dt][2] *= a1;
      dv[dt][3] *= a1;
    }
  }
}

template <int D, bool TAIL, bool NORMS>
__device__ inline void tile_scores(const float4_t &dk, uint32_t knp, float sfac, int tb, int t1, int g, int n,
                                   float4_t (&dv)[D / 16], float &m_run, float &l_run, float &m_top, float (&s)[2]) {
  raw_scores<NORMS>(dk, knp, sfac, n, s);
  tile_update<D, TAIL>(s, tb, t1, g, n, dv, m_run, l_run, m_top);
}

// tile_weights: w = exp2(s - m) times the tokens' fp16 value norms (vnp,
// NORMS) or alone, split as w = hi + lo (fp16 each, about 22 bits together)
// and traded between the lanes of a head into the A operand of the value
// products.
template <bool TAIL, bool NORMS>
__device__ inline half8_t tile_weights(const float (&s)[2], uint32_t vnp, float m1, int n, float m_run, float &l_run) {
  const bool odd = n & 1;
  float w[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float p = __builtin_amdgcn_exp2f(s[u] - m_run);
    if constexpr (TAIL) p = (s[u] == -INFINITY) ? 0.f : p;
    l_run += p;
    if constexpr (NORMS) w[u] = u ? half_mul<1>(vnp, p) : half_mul<0>(vnp, p);
    else w[u] = p;
  }
  uint32_t hp, lp;
  split_pair(w[0], w[1], m1, hp, lp);
  // lane 2h gets the partner's high parts, lane 2h+1 the partner's low parts
  const uint32_t got = swap1_u32(odd ? hp : lp);
  const uint32_t first = odd ? got : hp, second = odd ? lp : got;      // tokens 4g, 4g+1 | 4g+2, 4g+3
  const uint4_t a4 = {__builtin_amdgcn_perm(first, first, 0x01000100u), __builtin_amdgcn_perm(first, first, 0x03020302u),
                      __builtin_amdgcn_perm(second, second, 0x01000100u),
                      __builtin_amdgcn_perm(second, second, 0x03020302u)};
  return __builtin_bit_cast(half8_t, a4);
}

// One 16-token tile of packed codes (KB-bit keys, VB-bit values).
template <int D, int KB, int VB, bool TAIL>
__device__ inline void process_tile(const Tile<D, KB, VB> &t, const uint4_t (&bk)[D / 16], const uint8_t *tab,
                                    uint32_t kslot, uint32_t vslot, float sfac, float m1, int tb, int t1, int g, int n,
                                    float4_t (&dv)[D / 16], float &m_run, float &l_run, float &m_top) {
  float4_t dk = {0.f, 0.f, 0.f, 0.f};
  key_scores<D, KB>(t.kw, bk, tab, kslot, dk);

  const bool odd = n & 1;
  const uint32_t knp = odd ? t.kn.y : t.kn.x;        // fp16 norms of this lane's two tokens
  const uint32_t vnp = odd ? t.vn.y : t.vn.x;
  float s[2];
  tile_scores<D, TAIL, true>(dk, knp, sfac, tb, t1, g, n, dv, m_run, l_run, m_top, s);

  ValueBytes<D, VB> vb;
  value_bytes<D, VB>(t, vb, n);

  const half8_t aw = tile_weights<TAIL, true>(s, vnp, m1, n, m_run, l_run);
  value_update<D, VB>(vb, tab, vslot, aw, dv);
}

}  // namespace pair
}  // namespace kvq
