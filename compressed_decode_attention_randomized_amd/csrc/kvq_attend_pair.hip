// Split-K GQA decode attention on 4-bit Lloyd-Max keys and values, head
// dimension 128: matrix-core products fed from a byte-indexed pair table (the
// table, the tile layout and the per-tile softmax are described with the
// shared tile code), and in the same launch an fp16 near tier (a decode
// buffer of recent tokens kept unquantised).
//
// Work mapping: grid (split group, b * Hkv), one work-group of 16 waves per
// compute unit sharing one table; with more splits than compute units a
// work-group covers 2-8 consecutive splits of one (b, KV head), one wave
// group each.  Waves take 16-token tiles from an LDS counter (so all waves
// of a group finish within a tile of each other whatever their issue
// priority), two tiles in flight per wave.  All HBM reads are buffer loads
// with the cache arrays as SGPR resources.
//
// Near tier: work-group j < (near splits) of a (b, KV head) also serves
// near split j with its last near_waves waves (chosen on the host from the
// two tiers' bytes per split, so both wave sets finish together).  A near
// tile is 16 fp16 rows in the original domain: the key rows are the A
// operand as they are, against the unrotated query split into fp16 hi and
// lo rows (B columns 2h and 2h+1), and each value coordinate of four tokens
// is one B operand with zero low halves, so the softmax step and the value
// accumulator are those of the code tiles.  The near split's state is
// written as its own partial row, in the original domain.
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

constexpr int D = 128;
constexpr int kWaves = 16;
constexpr int kMinWaves = 4;                   // waves per SIMD the register budget is sized for
constexpr int kBlock = kWaves * 64;
constexpr int kRow = D / 2;                     // packed bytes per 4-bit vector
constexpr int kVDL = D / 16;                    // value coordinates per lane
constexpr int kRowPad = D + 4;                  // query table row stride (words)
// s_waitcnt vmcnt(7) expcnt(7) lgkmcnt(15): the seven loads of one tile
constexpr int kWaitOlderTile = 0x0F70 | kTileLoads<D>;
static_assert(kTileLoads<D> == 7, "tile loads");
constexpr int kSetupWaves = 8;                  // waves that build the tables and the rotated query

struct PParams {
  const void *q;
  int q_f16;
  int kv_heads, q_heads, capacity, seq_len, num_splits;
  int group_size;                  // query heads per KV head
  int chunk;                       // tokens per split (a multiple of 32)
  int group_log2;                  // log2 of the splits one work-group covers (its wave groups)
  int part_stride;                 // splits per (b, query head) row of the partial buffers
  int far_base;                    // partial row of far split 0 (the near splits come first)
  const uint8_t *k_codes, *v_codes;
  const uint16_t *k_norms, *v_norms;
  const int8_t *signs;
  const float *k_centroids, *v_centroids;
  float *part_o, *part_ml;         // partial rows from row 0
  // fp16 near tier [b * Hkv + KV head][near_len][D] (num_near_splits 0: none;
  // then group_log2 is 0 and num_near_splits <= num_splits)
  const uint16_t *near_k, *near_v;
  int near_len, num_near_splits;
  int near_chunk;                  // near tokens per near split (a multiple of 32)
  int near_waves;                  // waves (1-8) of a work-group that serve its near split
};

constexpr float kRsqrtD = 0.08838834764831845f;   // 1 / sqrt(128), the softmax scale of the near tier
constexpr int kNearRow = D / 2 + 4;               // near query table row stride (words)

// fp16 near-tier tile: key row of token n, coordinates [32g, 32g+32) (four
// 16-byte loads); value rows of tokens 4g..4g+3, coordinates [8n, 8n+8) (one
// 16-byte load each).
struct NearTile {
  uint4_t k[4];
  uint4_t v[4];
};

struct NearSources {
  const uint16_t *k, *v;           // this (b, KV head)'s rows
  int len;                         // near_len
  uint32_t ko, vo;                 // per-lane offsets
};

// Loads of the near tile at token tb < len (skip: none).  The descriptor
// starts at the tile and ends at the tier's end, so rows past it read as
// zero without touching memory; a skipped tile reads through descriptors
// of size zero.
__device__ inline void load_near_keys(NearTile &t, const NearSources &src, int tb, bool skip) {
  const __amdgpu_buffer_rsrc_t kr =
      make_rsrc(src.k + (size_t)(skip ? 0 : tb) * D, skip ? 0u : (uint32_t)(src.len - tb) * D * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, src.ko + 16 * i, 0, kStream);
}

__device__ inline void load_near_values(NearTile &t, const NearSources &src, int tb, bool skip) {
  const __amdgpu_buffer_rsrc_t vr =
      make_rsrc(src.v + (size_t)(skip ? 0 : tb) * D, skip ? 0u : (uint32_t)(src.len - tb) * D * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, src.vo + i * D * 2, 0, kStream);
}

// One near tile: keys block kb = coordinates 32g + 8kb .. +7 of token n
// (A row n, k slots 8g..8g+7) against the query's hi and lo rows; value
// tile M = coordinate 8n + M, B k slots (v, 0) per token 4g..4g+3 against
// the weight rows (w_hi, w_hi) and (w_lo, w_lo) of the shared softmax step.
__device__ inline void process_near(NearTile &t, const NearSources &src, int tn, bool skip_next,
                                    const uint4_t (&bq)[4], float sfac, float m1, int tb, int t1, int g, int n,
                                    float4_t (&dv)[D / 16], float &m_run, float &l_run, float &m_top) {
  float4_t dk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, t.k[kb]), __builtin_bit_cast(half8_t, bq[kb]),
                                                 dk, 0, 0, 0);
  load_near_keys(t, src, tn, skip_next);             // the key registers are free again
  float s[2];
  tile_scores<D, true, false>(dk, 0u, sfac, tb, t1, g, n, dv, m_run, l_run, m_top, s);
  const half8_t aw = tile_weights<true, false>(s, 0u, m1, n, m_run, l_run);
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    uint4_t b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (m & 1) ? t.v[i][m >> 1] >> 16 : t.v[i][m >> 1] & 0xFFFFu;
    dv[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, b), dv[m], 0, 0, 0);
  }
  load_near_values(t, src, tn, skip_next);
}

// Bounded wait for the set-up waves' counts: every set-up wave reaches its
// count without waiting on anything but its own loads, so the limit (tens
// of milliseconds) only guards against a hang.
__device__ inline void wait_setup(const uint32_t *ready, uint32_t count) {
  for (int spin = 0; spin < kSpinLimit; ++spin) {
    const uint32_t r = __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(r) >= count) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Maximum and sum over the 16 lanes of a lane row.
__device__ inline float row16_max(float x, int lane) {
  x = fmaxf(x, xor_lane<1>(x, lane));
  x = fmaxf(x, xor_lane<2>(x, lane));
  x = fmaxf(x, xor_lane<4>(x, lane));
  return fmaxf(x, xor_lane<8>(x, lane));
}

__device__ inline float row16_sum(float x, int lane) {
  x += xor_lane<1>(x, lane);
  x += xor_lane<2>(x, lane);
  x += xor_lane<4>(x, lane);
  return x + xor_lane<8>(x, lane);
}

// Weighted sum over waves [w0, w1) of value row (head h, coordinate j).
__device__ inline float merge_range(const float *red_acc, const float (*wfac)[kGMax], int w0, int w1, int h, int j) {
  const int in_wave = (((h >> 1) * 4 + 2 * (h & 1) + ((j >> 2) & 1)) * 16 + (j >> 3)) * 4 + (j & 3);
  float o = 0.f;
  for (int w = w0; w < w1; ++w) o += red_acc[w * (4 * 4 * 16 * 4) + in_wave] * wfac[w][h];
  return o;
}

// Weighted sum over the GW waves w0.. of a group of value row (head h,
// coordinate j); the rows sit in LDS as [wave][g][part][n][4] with head
// h = 2g + hp and coordinate j = 8n + c in part 2hp + c / 4, float c % 4.
template <int GW>
__device__ inline float merge_rows(const float *red_acc, const float (*wfac)[kGMax], int w0, int h, int j) {
  const int in_wave = (((h >> 1) * 4 + 2 * (h & 1) + ((j >> 2) & 1)) * 16 + (j >> 3)) * 4 + (j & 3);
  float o = 0.f;
#pragma unroll
  for (int w = 0; w < GW; ++w) o += red_acc[(w0 + w) * (4 * 4 * 16 * 4) + in_wave] * wfac[w0 + w][h];
  return o;
}

__global__ __launch_bounds__(kBlock, kMinWaves) void attend_pair_kernel(PParams P) {
  // pair tables during the loop, the waves' value rows afterwards
  __shared__ __attribute__((aligned(16))) uint8_t tab[2 * 65536];
  __shared__ __attribute__((aligned(16))) uint32_t qtab[2 * kGMax][kRowPad];
  __shared__ __attribute__((aligned(16))) uint32_t qnear[2 * kGMax][kNearRow];   // unrotated query (hi row, lo row) per head
  __shared__ float qfacn[kGMax];
  __shared__ uint32_t next_near;                     // near tile counter
  __shared__ float red_ml[kWaves][kGMax][3];      // (reference, sum, largest score) per wave and head
  __shared__ float qfac[kGMax];
  __shared__ float wfac[kWaves][kGMax];
  __shared__ uint32_t next_tile[kWaves];
  __shared__ uint32_t ready;                         // set-up waves done
  __shared__ uint32_t v_table[1];                    // offset of the value table: 0 when shared with the keys

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  // Index arithmetic is kept free of divisions: at kernel start every wave
  // of a SIMD runs it on the one scalar issue slot the SIMD gets per cycle
  // group, ahead of its first loads.
  const int G = P.group_size;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const int bh = b * P.kv_heads + hkv;
  // the work-group covers 2^group_log2 consecutive splits of one (b, KV head),
  // each with its own group of gw waves (all share the query and the tables);
  // with a near split (group_log2 0) the last nwn waves serve it instead
  const int lg = P.group_log2;
  const int nwn = ((int)blockIdx.x < P.num_near_splits) ? P.near_waves : 0;
  const int nf = kWaves - nwn;                       // waves on the far split(s)
  const bool near_wave = wave >= nf;
  const int gw = (lg == 0) ? nf : kWaves >> lg;
  const int grp = wave >> (4 - lg), gwave = (lg == 0) ? wave : wave & (gw - 1);
  const int split = (blockIdx.x << lg) + grp;

  // chunks of ceil(T/S) tokens rounded up to a multiple of 32 (from the
  // host); full tiles [t0, t1f) go through the main loop, a partial last
  // tile (only the last split can have one) after it; splits past S (a
  // partly used last group) get no tokens and write nothing
  const int chunk = P.chunk;
  const int t0 = min(P.seq_len, split * chunk), t1 = min(P.seq_len, t0 + chunk);
  const int ntiles = (t1 - t0) / kTile;
  const int t1f = t0 + ntiles * kTile;
  const uint32_t cap = (uint32_t)P.capacity;
  Sources src;
  src.kc = P.k_codes + (size_t)bh * cap * kRow;
  src.vc = P.v_codes + (size_t)bh * cap * kRow;
  src.kn = P.k_norms + (size_t)bh * cap;
  src.vn = P.v_norms + (size_t)bh * cap;
  src.kcode_bytes = src.vcode_bytes = cap * kRow;
  src.norm_bytes = cap * 2;
  set_offsets<D>(src, g, n);

  // ---- set-up ----
  // Waves 0-7 build the pair tables and the rotated query; waves 8-15 first
  // request their first two tiles.  The set-up waves request theirs after
  // the set-up: at kernel start every compute unit floods the memory system,
  // a wave's tile requests can sit in the issue queue for microseconds, and
  // a wave issues in order, so a set-up wave stuck behind its own tile
  // requests would hold up the tables everybody needs.  Readiness is an LDS
  // count the set-up waves bump, not a barrier, so no wave waits for another
  // wave's requests to go out.
  static_assert(kBlock == 1024 && kSetupWaves * 64 * 16 == 2 * 65536 / 16, "pair-table fill layout");
  if (tid < kWaves) next_tile[tid] = 2 * gw;
  if (tid == 0) ready = 0u;
  if (tid == 0) next_near = (uint32_t)nwn;
  __syncthreads();                                   // cheap here: no wave has memory requests yet

  int ia = gwave, ic = gwave + gw;                   // first tiles of this wave; later ones from its group's counter
  Tile<D> ta, tc;
  if (wave < kSetupWaves) {
    // Centroids through uniform addresses (scalar loads the scalar cache
    // serves to every wave of the chip); query rows and signs for the waves
    // that rotate them (zero-size descriptors elsewhere).
    float ck[16], cv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ck[i] = P.k_centroids[i];
      cv[i] = P.v_centroids[i];
    }
    const bool has_q = wave < G;
    const int q_f16 = P.q_f16;
    const uint32_t q_es = q_f16 ? 2u : 4u;
    const size_t q_row0 = ((size_t)b * P.q_heads + (size_t)hkv * G) * D;
    const __amdgpu_buffer_rsrc_t qsrc = make_rsrc(static_cast<const uint8_t *>(P.q) + q_row0 * q_es,
                                                  has_q ? (uint32_t)(G * D) * q_es : 0u);
    const __amdgpu_buffer_rsrc_t ssrc = make_rsrc(P.signs, has_q ? (uint32_t)D : 0u);
    const uint32_t q_off = (uint32_t)(wave * D + lane * 2) * q_es;
    // coordinates 2l, 2l+1: both halves of q0 (fp16) or q0 and q1 (fp32);
    // for fp16 queries q1 is unused (past the last row it reads as zero)
    const uint32_t q0 = __builtin_amdgcn_raw_buffer_load_b32(qsrc, q_off, 0, 0);
    const uint32_t q1 = __builtin_amdgcn_raw_buffer_load_b32(qsrc, q_off + 4u, 0, 0);
    const uint32_t sg = __builtin_amdgcn_raw_buffer_load_b16(ssrc, lane * 2, 0, 0);   // signs of coordinates 2l, 2l+1
    const bool near_tier = P.num_near_splits > 0;

    // Keys and values with one codebook (the usual case: one format for
    // both) share the key table.
    bool same = true;
#pragma unroll
    for (int i = 0; i < 16; ++i) same = same && (ck[i] == cv[i]);

    // ---- pair tables: key table in the first 64 KB, value table in the next ----
    // Row (code byte) r of a table holds 32 slots of the 8-byte entry
    // (e(c[r % 16]), e(c[r / 16])).  Chunks of 16 bytes (two slots) are
    // written by consecutive lanes: thread t < 512 writes chunks t + 512k,
    // k = 0..15, i.e. table k / 8, row t/16 + 32 (k % 8): low nibble
    // (t/16) % 16 = 4 (wave % 4) + lane / 16 for every k, high nibble
    // wave / 4 + 2 (k % 8).
    {
      // uniform parts chosen by a scalar switch (constant indices keep the
      // centroids in scalar registers), then one of four values by lane row
      const int r4 = lane >> 4;
      float lk[4], lv[4], hk[8], hv[8];
      switch (wave & 3) {
        case 0: pick<0, 1>(ck, cv, lk, lv); break;
        case 1: pick<4, 1>(ck, cv, lk, lv); break;
        case 2: pick<8, 1>(ck, cv, lk, lv); break;
        default: pick<12, 1>(ck, cv, lk, lv); break;
      }
      if (wave >> 2) pick<1, 2>(ck, cv, hk, hv);
      else pick<0, 2>(ck, cv, hk, hv);
      float lo_k = lk[0], lo_v = lv[0];
#pragma unroll
      for (int u = 1; u < 4; ++u) {
        lo_k = (r4 == u) ? lk[u] : lo_k;
        lo_v = (r4 == u) ? lv[u] : lo_v;
      }
      const uint32_t lok = split_entry(lo_k * kCodeScale), lov = split_entry(lo_v * kCodeScale);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t hi = split_entry(hk[k] * kCodeScale);
        const uint4_t e = {lok, hi, lok, hi};
        *reinterpret_cast<uint4_t *>(tab + (tid + 512 * k) * 16) = e;
      }
      if (!same) {
#pragma unroll
        for (int k = 8; k < 16; ++k) {
          const uint32_t hi = split_entry(hv[k & 7] * kCodeScale);
          const uint4_t e = {lov, hi, lov, hi};
          *reinterpret_cast<uint4_t *>(tab + (tid + 512 * k) * 16) = e;
        }
      }
      if (tid == 0) v_table[0] = same ? 0u : 0x10000u;
    }

    // ---- rotated query of head `wave` (waves G..7 write zero rows) ----
    // Lane l holds coordinates 2l, 2l+1: sign flip, the stride-1 butterfly in
    // the lane, strides 2..64 across lanes (xor 1..32).  The rotated vector
    // is scaled so that its largest |z| lies in (64, 128] and stored in the
    // two B-operand forms (z_hi, z_hi) (row 2h) and (z_lo, 0) (row 2h+1).
    static_assert(kSetupWaves == kGMax, "one set-up wave per query row pair");
    uint2_t f0 = {0u, 0u}, f1 = {0u, 0u};
    float fac = 0.f;
    uint32_t n0 = 0u, n1 = 0u;
    float facn = 0.f;
    if (has_q) {
      float z0 = q_f16 ? half_value(q0 & 0xFFFFu) : __builtin_bit_cast(float, q0);
      float z1 = q_f16 ? half_value(q0 >> 16) : __builtin_bit_cast(float, q1);
      if (near_tier) {
        // the unrotated query for the near tier, scaled like the rotated one
        const float nmax = wave_max(fmaxf(fabsf(z0), fabsf(z1)), lane);
        const float ns = (nmax > 0.f) ? exp2f(7.f - ceilf(log2f(nmax))) : 1.f;
        const float a = z0 * ns, c = z1 * ns;
        const _Float16 ha = (_Float16)a, hc = (_Float16)c;
        n0 = pack2(ha, hc);
        n1 = pack2((_Float16)(a - (float)ha), (_Float16)(c - (float)hc));
        facn = kLog2e * kRsqrtD / ns;
      }
      z0 = (sg & 0x80u) ? -z0 : z0;
      z1 = (sg & 0x8000u) ? -z1 : z1;
      float a = z0 + z1, c = z0 - z1;
      a = fwht_lanes(a, lane);
      c = fwht_lanes(c, lane);
      const float zmax = wave_max(fmaxf(fabsf(a), fabsf(c)), lane);
      const float qscale = (zmax > 0.f) ? exp2f(7.f - ceilf(log2f(zmax))) : 1.f;
      const float za = a * qscale, zc = c * qscale;
      const _Float16 ha = (_Float16)za, hc = (_Float16)zc;
      const _Float16 la = (_Float16)(za - (float)ha), lc = (_Float16)(zc - (float)hc);
      f0 = (uint2_t){pack2(ha, ha), pack2(hc, hc)};
      f1 = (uint2_t){pack2(la, (_Float16)0.f), pack2(lc, (_Float16)0.f)};
      fac = kLog2e / ((float)D * kCodeScale * qscale);
    }
    *reinterpret_cast<uint2_t *>(&qtab[2 * wave][lane * 2]) = f0;
    *reinterpret_cast<uint2_t *>(&qtab[2 * wave + 1][lane * 2]) = f1;
    if (lane == 0) qfac[wave] = fac;
    if (near_tier) {
      qnear[2 * wave][lane] = n0;
      qnear[2 * wave + 1][lane] = n1;
      if (lane == 0) qfacn[wave] = facn;
    }
    // this wave's table, query and factor writes complete before its count
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(&ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  float m1 = -1.f;
  asm volatile("" : "+s"(m1));                       // no instruction: keeps -1 from being folded
  float4_t dv[kVDL];
#pragma unroll
  for (int dt = 0; dt < kVDL; ++dt) dv[dt] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;             // softmax reference and sum for this lane's column
  float m_top = -INFINITY;                           // largest score of this lane's rows

  if (near_wave) {
    // ---- near split blockIdx.x: tiles [n0, n1) of the fp16 rows, one tile
    // per wave in flight, its key and value halves refilled as each is used ----
    const int nsp = blockIdx.x;
    const int n0 = min(P.near_len, nsp * P.near_chunk), n1 = min(P.near_len, n0 + P.near_chunk);
    const int nnt = (n1 - n0 + kTile - 1) / kTile;
    NearSources nsrc;
    nsrc.k = P.near_k + (size_t)bh * P.near_len * D;
    nsrc.v = P.near_v + (size_t)bh * P.near_len * D;
    nsrc.len = P.near_len;
    nsrc.ko = n * D * 2 + g * 64;
    nsrc.vo = 4 * g * D * 2 + n * 16;
    int it = wave - nf;
    NearTile nt;
    load_near_keys(nt, nsrc, n0 + it * kTile, it >= nnt);
    load_near_values(nt, nsrc, n0 + it * kTile, it >= nnt);
    wait_setup(&ready, kSetupWaves);
    // B operand of key block kb for column n: near query row n (head n / 2,
    // hi or lo form), coordinates 32g + 8kb .. +7
    uint4_t bq[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) bq[kb] = *reinterpret_cast<const uint4_t *>(&qnear[n][g * 16 + 4 * kb]);
    const float sfac = qfacn[n >> 1];
    while (it < nnt) {
      uint32_t nx = 0u;
      if (lane == 0) nx = atomicAdd(&next_near, 1u);
      __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this tile's loads
      asm volatile("" : "+v"(nx));
      const int na = __builtin_amdgcn_readfirstlane(nx);
      process_near(nt, nsrc, n0 + na * kTile, na >= nnt, bq, sfac, m1, n0 + it * kTile, n1, g, n, dv, m_run, l_run,
                   m_top);
      it = na;
    }
  } else {
  __builtin_amdgcn_sched_barrier(0);
  load_tile(ta, src, t0 + ia * kTile, ia >= ntiles);
  __builtin_amdgcn_sched_barrier(0);
  load_tile(tc, src, t0 + ic * kTile, ic >= ntiles);
  __builtin_amdgcn_sched_barrier(0);

  // Wait for the eight set-up counts.
  wait_setup(&ready, kSetupWaves);

  // B operand of key block kb for column n: query table row n (head n / 2,
  // form n % 2), coordinates 32g + 4kb .. +3
  uint4_t bk[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) bk[kb] = *reinterpret_cast<const uint4_t *>(&qtab[n][g * 32 + 4 * kb]);
  const float sfac = qfac[n >> 1];
  const uint32_t kslot = (uint32_t)(lane & 31) * 8, vslot = kslot | v_table[0];

  // Tiles alternate between the two tile buffers; each buffer is refilled
  // with a newly claimed tile right after use (ia < ic always holds, so once
  // ic runs past the end the next ia does too).  Every iteration issues both
  // buffers' loads, so the explicit vmcnt(7) (the older tile's seven loads)
  // is the only wait for a tile's data; loads past the end return zeros.
  // The counter's answer is first read after the tile, so the atomic's
  // latency hides behind the tile's own LDS traffic.
  while (ia < ntiles) {
    uint32_t nx = 0u;
    if (lane == 0) nx = atomicAdd(&next_tile[grp], 1u);
    __builtin_amdgcn_s_waitcnt(kWaitOlderTile);
    process_tile<D, 4, 4, false>(ta, bk, tab, kslot, vslot, sfac, m1, t0 + ia * kTile, t1, g, n, dv, m_run, l_run, m_top);
    asm volatile("" : "+v"(nx));                     // keeps the read of the answer here
    const int na = __builtin_amdgcn_readfirstlane(nx);
    load_tile(ta, src, t0 + na * kTile, na >= ntiles);
    int nc = ntiles;
    if (ic < ntiles) {
      uint32_t ny = 0u;
      if (lane == 0) ny = atomicAdd(&next_tile[grp], 1u);
      __builtin_amdgcn_s_waitcnt(kWaitOlderTile);
      process_tile<D, 4, 4, false>(tc, bk, tab, kslot, vslot, sfac, m1, t0 + ic * kTile, t1, g, n, dv, m_run, l_run, m_top);
      asm volatile("" : "+v"(ny));
      nc = __builtin_amdgcn_readfirstlane(ny);
    }
    load_tile(tc, src, t0 + nc * kTile, nc >= ntiles);
    ia = na;
    ic = nc;
  }
  // the last split's partial tile [t1f, t1)
  if (gwave == 0 && t1f < t1) {
    load_tail_tile(ta, src, t1f);
    process_tile<D, 4, 4, true>(ta, bk, tab, kslot, vslot, sfac, m1, t1f, t1, g, n, dv, m_run, l_run, m_top);
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
  float *red_acc = reinterpret_cast<float *>(tab);   // per wave: 8 heads x D floats
  {
    // layout [wave][g][part][n][4]: part = 2 * (head - 2g) + half, so each
    // 16-lane row of a write covers 256 contiguous bytes
    float *r = red_acc + ((size_t)(wave * 4 + g) * 4 * 16 + n) * 4;
    if (2 * g < G) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        *reinterpret_cast<float4_t *>(r + 64 * q) =
            (float4_t){dv[4 * q][0] + dv[4 * q][1], dv[4 * q + 1][0] + dv[4 * q + 1][1],
                       dv[4 * q + 2][0] + dv[4 * q + 2][1], dv[4 * q + 3][0] + dv[4 * q + 3][1]};
    }
    if (2 * g + 1 < G) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        *reinterpret_cast<float4_t *>(r + 128 + 64 * q) =
            (float4_t){dv[4 * q][2] + dv[4 * q][3], dv[4 * q + 1][2] + dv[4 * q + 1][3],
                       dv[4 * q + 2][2] + dv[4 * q + 2][3], dv[4 * q + 3][2] + dv[4 * q + 3][3]};
    }
  }
  // Weight of each wave's rows in its group's merge, one lane per (head h,
  // wave w) in waves 0-1 (h = tid / 16, w = tid % 16): a group's waves are
  // gw consecutive lanes of a 16-lane row, reduced with DPP exchanges.  The
  // weight exp2(m_w - M) / (L * code scale) folds in the softmax
  // denominator, so the per-coordinate pass below is a plain weighted sum.
  if (tid < kWaves * kGMax) {
    const int h = tid >> 4, w = tid & (kWaves - 1);
    const float m = red_ml[w][h][0], l = red_ml[w][h][1], mt = red_ml[w][h][2];
    float M, L, Mt, f;
    if (nwn == 0) {
      M = fmaxf(m, xor_lane<1>(m, lane));           // gw >= 2
      if (gw > 2) M = fmaxf(M, xor_lane<2>(M, lane));
      if (gw > 4) M = fmaxf(M, xor_lane<4>(M, lane));
      if (gw > 8) M = fmaxf(M, xor_lane<8>(M, lane));
      f = (m == -INFINITY) ? 0.f : exp2f(m - M);
      L = l * f;
      L += xor_lane<1>(L, lane);
      if (gw > 2) L += xor_lane<2>(L, lane);
      if (gw > 4) L += xor_lane<4>(L, lane);
      if (gw > 8) L += xor_lane<8>(L, lane);
      // the split's state is reported against its largest score
      Mt = fmaxf(mt, xor_lane<1>(mt, lane));
      if (gw > 2) Mt = fmaxf(Mt, xor_lane<2>(Mt, lane));
      if (gw > 4) Mt = fmaxf(Mt, xor_lane<4>(Mt, lane));
      if (gw > 8) Mt = fmaxf(Mt, xor_lane<8>(Mt, lane));
    } else {
      // two groups in the head's 16 lanes: far waves [0, nf), near waves
      // [nf, 16); each reduced over all 16 lanes with the other group's
      // lanes neutral
      const bool mine = w >= nf;
      M = row16_max(mine ? -INFINITY : m, lane);
      const float Mn = row16_max(mine ? m : -INFINITY, lane);
      M = mine ? Mn : M;
      Mt = row16_max(mine ? -INFINITY : mt, lane);
      const float Mtn = row16_max(mine ? mt : -INFINITY, lane);
      Mt = mine ? Mtn : Mt;
      f = (m == -INFINITY) ? 0.f : exp2f(m - M);
      L = row16_sum(mine ? 0.f : l * f, lane);
      const float Ln = row16_sum(mine ? l * f : 0.f, lane);
      L = mine ? Ln : L;
    }
    // near rows carry fp16 values, code rows centroids scaled by kCodeScale
    const bool near_row = nwn > 0 && w >= nf;
    wfac[w][h] = (L > 0.f) ? f / (near_row ? L : L * kCodeScale) : 0.f;
    const bool any = L > 0.f;
    const size_t hrow = ((size_t)b * P.q_heads + hkv * G + h) * P.part_stride;
    if (near_row) {
      if (w == nf && h < G) {
        const size_t row = hrow + blockIdx.x;
        P.part_ml[row * 2 + 0] = any ? Mt * kLn2 : -INFINITY;
        P.part_ml[row * 2 + 1] = any ? L * exp2f(M - Mt) : 0.f;
      }
    } else {
      const int sp = (blockIdx.x << lg) + (w >> (4 - lg));
      const int lead = (lg == 0) ? 0 : w & ~(gw - 1);
      if (w == lead && h < G && sp < P.num_splits) {
        const size_t row = hrow + P.far_base + sp;
        P.part_ml[row * 2 + 0] = any ? Mt * kLn2 : -INFINITY;
        P.part_ml[row * 2 + 1] = any ? L * exp2f(M - Mt) : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- merge each group's waves: one thread per (group, head, coordinate);
  // a wave's lanes share (group, head), so the weight reads are broadcasts
  // and the value reads are consecutive ----
  static_assert(kGMax * D <= kBlock, "one thread per (head, coordinate)");
  if (nwn > 0) {
    if (tid < G * D) {
      const int h = tid >> 7, j = tid & (D - 1);
      const size_t hrow = ((size_t)b * P.q_heads + hkv * G + h) * P.part_stride;
      if ((int)blockIdx.x < P.num_splits) P.part_o[(hrow + P.far_base + blockIdx.x) * D + j] = merge_range(red_acc, wfac, 0, nf, h, j);
      P.part_o[(hrow + blockIdx.x) * D + j] = merge_range(red_acc, wfac, nf, kWaves, h, j);
    }
    return;
  }
  for (int gi = 0; gi < (1 << lg) && tid < G * D; ++gi) {
    const int h = tid >> 7, j = tid & (D - 1);
    const int sp = (blockIdx.x << lg) + gi;
    if (sp >= P.num_splits) break;
    float o;
    switch (lg) {
      case 0: o = merge_rows<16>(red_acc, wfac, 0, h, j); break;
      case 1: o = merge_rows<8>(red_acc, wfac, gi * 8, h, j); break;
      case 2: o = merge_rows<4>(red_acc, wfac, gi * 4, h, j); break;
      default: o = merge_rows<2>(red_acc, wfac, gi * 2, h, j); break;
    }
    const size_t row = ((size_t)b * P.q_heads + hkv * G + h) * P.part_stride + P.far_base + sp;
    P.part_o[row * D + j] = o;
  }
}

}  // namespace

namespace {

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  return cus;
}

// One work-group fills a compute unit.  When the splits outnumber the
// compute units, a work-group takes 2, 4 or 8 consecutive splits of one
// (b, KV head) with a wave group each instead of running in several rounds.
int pair_group_log2(const AttendArgs &a, int cus) {
  const int64_t pairs = (int64_t)a.batch * a.kv_heads;
  int lg = 0;
  while (lg < 3 && pairs * ((a.num_splits + (1 << lg) - 1) >> lg) > (int64_t)cus) ++lg;
  return lg;
}

bool pair_codes_supported(const AttendArgs &a) {
  const int G = a.q_heads / a.kv_heads;
  const bool fits = (int64_t)a.capacity * a.head_dim / 2 < (1ll << 31);
  return a.head_dim == D && a.k_format == 4 && a.v_format == 4 && G >= 1 && G <= kGMax && fits;
}

}  // namespace

bool pair_attend_supported(const AttendArgs &a) { return pair_codes_supported(a) && a.num_near_splits == 0; }

bool pair_near_supported(const AttendArgs &a) {
  return pair_codes_supported(a) && a.num_near_splits > 0 && a.num_near_splits <= a.num_splits && a.near_k &&
         a.near_v && (int64_t)a.near_len * D * 2 < (1ll << 31) && pair_group_log2(a, device_cus()) == 0;
}

hipError_t launch_attend_pair(const AttendArgs &a, hipStream_t stream, int part_base) {
  const int lg = pair_group_log2(a, device_cus());
  const int chunk = ((a.seq_len + a.num_splits - 1) / a.num_splits + kChunkTok - 1) / kChunkTok * kChunkTok;
  const int SN = a.num_near_splits;
  int near_chunk = 0, near_waves = 0;
  if (SN > 0) {
    // near waves in proportion to the two tiers' bytes per split (fp16 key
    // and value rows against 132-byte code rows), 1 to 8 of the 16
    near_chunk = ((a.near_len + SN - 1) / SN + kChunkTok - 1) / kChunkTok * kChunkTok;
    const double nb = (double)near_chunk * D * 4, fb = (double)chunk * (D + 4);
    near_waves = (int)(kWaves * nb / (nb + fb) + 0.5);
    near_waves = near_waves < 1 ? 1 : (near_waves > kSetupWaves ? kSetupWaves : near_waves);
    part_base = SN;
  }
  PParams P{a.q, a.q_f16, a.kv_heads, a.q_heads, a.capacity, a.seq_len, a.num_splits, a.q_heads / a.kv_heads, chunk, lg,
            part_base + a.num_splits, part_base, a.k_codes, a.v_codes, a.k_norms, a.v_norms, a.signs, a.k_centroids,
            a.v_centroids, a.part_o, a.part_ml, SN > 0 ? a.near_k : nullptr, SN > 0 ? a.near_v : nullptr,
            SN > 0 ? a.near_len : 0, SN, near_chunk, near_waves};
  dim3 grid((a.num_splits + (1 << lg) - 1) >> lg, a.kv_heads, a.batch);
  hipLaunchKernelGGL(attend_pair_kernel, grid, dim3(kBlock), 0, stream, P);
  return hipGetLastError();
}

}  // namespace kvq
