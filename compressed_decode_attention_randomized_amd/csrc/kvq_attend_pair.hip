// Split-K GQA decode attention on 4-bit Lloyd-Max keys and values, head
// dimension 128: matrix-core products fed from a byte-indexed pair table (the
// table, the tile layout and the per-tile softmax are described with the
// shared tile code).
//
// Work mapping: grid (split group, b * Hkv), one work-group of 16 waves per
// compute unit sharing one table; with more splits than compute units a
// work-group covers 2-8 consecutive splits of one (b, KV head), one wave
// group each.  Waves take 16-token tiles from an LDS counter (so all waves
// of a group finish within a tile of each other whatever their issue
// priority), two tiles in flight per wave.  All HBM reads are buffer loads
// with the cache arrays as SGPR resources.
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
  const uint8_t *k_codes, *v_codes;
  const uint16_t *k_norms, *v_norms;
  const int8_t *signs;
  const float *k_centroids, *v_centroids;
  float *part_o, *part_ml;
};

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
  // each with its own group of gw waves (all share the query and the tables)
  const int lg = P.group_log2;
  const int gw = kWaves >> lg;
  const int grp = wave >> (4 - lg), gwave = wave & (gw - 1);
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
  src.code_bytes = cap * kRow;
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
    if (has_q) {
      float z0 = q_f16 ? half_value(q0 & 0xFFFFu) : __builtin_bit_cast(float, q0);
      float z1 = q_f16 ? half_value(q0 >> 16) : __builtin_bit_cast(float, q1);
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
    // this wave's table, query and factor writes complete before its count
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(&ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_tile(ta, src, t0 + ia * kTile, ia >= ntiles);
  __builtin_amdgcn_sched_barrier(0);
  load_tile(tc, src, t0 + ic * kTile, ic >= ntiles);
  __builtin_amdgcn_sched_barrier(0);

  // Wait for the eight set-up counts.  The spin is bounded: every set-up
  // wave reaches its count without waiting on anything but its own loads,
  // so the limit (tens of milliseconds) only guards against a hang.
  for (int spin = 0; spin < kSpinLimit; ++spin) {
    const uint32_t r = __hip_atomic_load(&ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(r) >= (uint32_t)kSetupWaves) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  // B operand of key block kb for column n: query table row n (head n / 2,
  // form n % 2), coordinates 32g + 4kb .. +3
  uint4_t bk[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) bk[kb] = *reinterpret_cast<const uint4_t *>(&qtab[n][g * 32 + 4 * kb]);
  const float sfac = qfac[n >> 1];
  const uint32_t kslot = (uint32_t)(lane & 31) * 8, vslot = kslot | v_table[0];
  float m1 = -1.f;
  asm volatile("" : "+s"(m1));                       // no instruction: keeps -1 from being folded

  float4_t dv[kVDL];
#pragma unroll
  for (int dt = 0; dt < kVDL; ++dt) dv[dt] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;             // softmax reference and sum for this lane's column
  float m_top = -INFINITY;                           // largest score of this lane's rows

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
    process_tile<D, 4, false>(ta, bk, tab, kslot, vslot, sfac, m1, t0 + ia * kTile, t1, g, n, dv, m_run, l_run, m_top);
    asm volatile("" : "+v"(nx));                     // keeps the read of the answer here
    const int na = __builtin_amdgcn_readfirstlane(nx);
    load_tile(ta, src, t0 + na * kTile, na >= ntiles);
    int nc = ntiles;
    if (ic < ntiles) {
      uint32_t ny = 0u;
      if (lane == 0) ny = atomicAdd(&next_tile[grp], 1u);
      __builtin_amdgcn_s_waitcnt(kWaitOlderTile);
      process_tile<D, 4, false>(tc, bk, tab, kslot, vslot, sfac, m1, t0 + ic * kTile, t1, g, n, dv, m_run, l_run, m_top);
      asm volatile("" : "+v"(ny));
      nc = __builtin_amdgcn_readfirstlane(ny);
    }
    load_tile(tc, src, t0 + nc * kTile, nc >= ntiles);
    ia = na;
    ic = nc;
  }
  // the last split's partial tile [t1f, t1)
  if (gwave == 0 && t1f < t1) {
    load_tile(ta, src, t1f, false);
    process_tile<D, 4, true>(ta, bk, tab, kslot, vslot, sfac, m1, t1f, t1, g, n, dv, m_run, l_run, m_top);
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
    float M = fmaxf(m, xor_lane<1>(m, lane));       // gw >= 2
    if (gw > 2) M = fmaxf(M, xor_lane<2>(M, lane));
    if (gw > 4) M = fmaxf(M, xor_lane<4>(M, lane));
    if (gw > 8) M = fmaxf(M, xor_lane<8>(M, lane));
    const float f = (m == -INFINITY) ? 0.f : exp2f(m - M);
    float L = l * f;
    L += xor_lane<1>(L, lane);
    if (gw > 2) L += xor_lane<2>(L, lane);
    if (gw > 4) L += xor_lane<4>(L, lane);
    if (gw > 8) L += xor_lane<8>(L, lane);
    wfac[w][h] = (L > 0.f) ? f / (L * kCodeScale) : 0.f;
    // the split's state is reported against its largest score
    float Mt = fmaxf(mt, xor_lane<1>(mt, lane));
    if (gw > 2) Mt = fmaxf(Mt, xor_lane<2>(Mt, lane));
    if (gw > 4) Mt = fmaxf(Mt, xor_lane<4>(Mt, lane));
    if (gw > 8) Mt = fmaxf(Mt, xor_lane<8>(Mt, lane));
    const int sp = (blockIdx.x << lg) + (w >> (4 - lg));
    if ((w & (gw - 1)) == 0 && h < G && sp < P.num_splits) {
      const size_t row = ((size_t)b * P.q_heads + hkv * G + h) * P.part_stride + sp;
      const bool any = L > 0.f;
      P.part_ml[row * 2 + 0] = any ? Mt * kLn2 : -INFINITY;
      P.part_ml[row * 2 + 1] = any ? L * exp2f(M - Mt) : 0.f;
    }
  }
  __syncthreads();

  // ---- merge each group's waves: one thread per (group, head, coordinate);
  // a wave's lanes share (group, head), so the weight reads are broadcasts
  // and the value reads are consecutive ----
  static_assert(kGMax * D <= kBlock, "one thread per (head, coordinate)");
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
    const size_t row = ((size_t)b * P.q_heads + hkv * G + h) * P.part_stride + sp;
    P.part_o[row * D + j] = o;
  }
}

}  // namespace

bool pair_attend_supported(const AttendArgs &a) {
  const int G = a.q_heads / a.kv_heads;
  const bool fits = (int64_t)a.capacity * a.head_dim / 2 < (1ll << 31);
  return a.head_dim == D && a.k_format == 4 && a.v_format == 4 && a.num_near_splits == 0 && G >= 1 &&
         G <= kGMax && fits;
}

hipError_t launch_attend_pair(const AttendArgs &a, hipStream_t stream, int part_base) {
  // One work-group fills a compute unit.  When the splits outnumber the
  // compute units, a work-group takes 2, 4 or 8 consecutive splits of one
  // (b, KV head) with a wave group each instead of running in several rounds.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int64_t pairs = (int64_t)a.batch * a.kv_heads;
  int lg = 0;
  while (lg < 3 && pairs * ((a.num_splits + (1 << lg) - 1) >> lg) > (int64_t)cus) ++lg;
  const int chunk = ((a.seq_len + a.num_splits - 1) / a.num_splits + kChunkTok - 1) / kChunkTok * kChunkTok;
  PParams P{a.q, a.q_f16, a.kv_heads, a.q_heads, a.capacity, a.seq_len, a.num_splits, a.q_heads / a.kv_heads, chunk, lg,
            part_base + a.num_splits, a.k_codes, a.v_codes, a.k_norms, a.v_norms, a.signs, a.k_centroids, a.v_centroids,
            a.part_o + (size_t)part_base * D, a.part_ml + (size_t)part_base * 2};
  dim3 grid((a.num_splits + (1 << lg) - 1) >> lg, a.kv_heads, a.batch);
  hipLaunchKernelGGL(attend_pair_kernel, grid, dim3(kBlock), 0, stream, P);
  return hipGetLastError();
}

}  // namespace kvq
