// Split merge of one (b, query head) row and the single inverse rotation,
// one wave (the merge kernel's body).
//
// Lane l owns output coordinates [l*E, (l+1)*E), E = D / 64.  The lanes read
// the split states (m_s, l_s) and form, with wave reductions,
//   M = max m_s, w_s = l_s exp(m_s - M), W = sum w_s,
// then accumulate the near-tier splits (original domain) and the far-tier
// splits (rotated domain) separately.  With at most eight splits every load
// of the row is issued before the first wait; with more, 64 / E rows are in
// flight at a time.  The far sum is mapped back once with R^T y = s * (H y) / sqrt(D):
// the Walsh-Hadamard stages inside a lane's E coordinates run in registers,
// the six across lanes with DPP and row swaps.
// Source: "FoveatedKV", "Making it fast" (split-K partial states merged after
// the fused pass; near and far tiers share one softmax).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_lane.h"

namespace kvq {

template <int E>
__device__ inline void merge_load_row(const float *p, float (&v)[E]) {
  if constexpr (E == 1) {
    v[0] = p[0];
  } else if constexpr (E == 2) {
    const float2 t = *reinterpret_cast<const float2 *>(p);
    v[0] = t.x;
    v[1] = t.y;
  } else {
    static_assert(E == 4, "coordinates per lane");
    const float4 t = *reinterpret_cast<const float4 *>(p);
    v[0] = t.x;
    v[1] = t.y;
    v[2] = t.z;
    v[3] = t.w;
  }
}

// Output of a merged row: the far sum's inverse rotation (stages of stride
// < E inside the lane, then the six cross-lane stages), the near sum added,
// both divided by W; the log-sum-exp M + ln W.
template <int D>
__device__ inline void merge_finish(float (&near_acc)[D / 64], float (&far_acc)[D / 64], float W, float M,
                                    const int8_t (&sg)[D / 64], float *__restrict__ out_row, float *__restrict__ lse,
                                    int lane) {
  constexpr int E = D / 64;
#pragma unroll
  for (int st = 1; st < E; st <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!(e & st)) {
        const float a = far_acc[e], c = far_acc[e + st];
        far_acc[e] = a + c;
        far_acc[e + st] = a - c;
      }
    }
  }
  const float inv_w = (W > 0.f) ? 1.f / W : 0.f;
  const float rs = rsqrtf((float)D);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float y = fwht_lanes(far_acc[e], lane) * rs;
    const float far = (sg[e] < 0) ? -y : y;
    out_row[lane * E + e] = (near_acc[e] + far) * inv_w;
  }
  if (lse && lane == 0) *lse = (W > 0.f) ? M + logf(W) : -INFINITY;
}

// po: the row's S = near_splits + splits partial outputs [S][D]; ml: its
// states [S][2]; out_row: [D]; lse: one float or NULL.
template <int D>
__device__ inline void merge_row(const float *__restrict__ po, const float *__restrict__ ml, int splits,
                                 int near_splits, const int8_t *__restrict__ signs, float *__restrict__ out_row,
                                 float *__restrict__ lse, int lane) {
  constexpr int E = D / 64;
  constexpr int kUnroll = 8;                       // the few-split case
  const int S = splits + near_splits;
  po += lane * E;
  int8_t sg[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sg[e] = signs[lane * E + e];

  if (S <= kUnroll) {
    // Few splits: the states, every partial row and the signs are requested
    // together, so the row waits for memory once.
    float m = -INFINITY, l = 0.f;
    if (lane < S) {
      m = ml[2 * lane];
      l = ml[2 * lane + 1];
    }
    float v[kUnroll][E];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u < S) {
        merge_load_row<E>(po + (size_t)u * D, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[u][e] = 0.f;
      }
    }
    const float M = wave_max(m, lane);
    const float w = (m == -INFINITY || l == 0.f) ? 0.f : l * expf(m - M);
    const float W = wave_sum(w, lane);
    float near_acc[E], far_acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) near_acc[e] = far_acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float wk = (u < S) ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u)) : 0.f;
      const bool near = u < near_splits;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (near) near_acc[e] = fmaf(wk, v[u][e], near_acc[e]);
        else far_acc[e] = fmaf(wk, v[u][e], far_acc[e]);
      }
    }
    merge_finish<D>(near_acc, far_acc, W, M, sg, out_row, lse, lane);
    return;
  }

  // More splits: groups of 64 / E rows (64 registers of partial rows).
  constexpr int kG = 64 / E;
  float near_acc[E], far_acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) near_acc[e] = far_acc[e] = 0.f;
  if (S <= 64) {
    // Up to 64 splits: lane s holds split s's state, requested with the
    // first group's rows, so up to kG splits take one round trip.
    float m = -INFINITY, l = 0.f;
    if (lane < S) {
      m = ml[2 * lane];
      l = ml[2 * lane + 1];
    }
    float v[kG][E];
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      if (u < S) {
        merge_load_row<E>(po + (size_t)u * D, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[u][e] = 0.f;
      }
    }
    const float M = wave_max(m, lane);
    const float w = (m == -INFINITY || l == 0.f) ? 0.f : l * expf(m - M);
    const float W = wave_sum(w, lane);
    for (int g0 = 0; g0 < S; g0 += kG) {
      if (g0 > 0) {
#pragma unroll
        for (int u = 0; u < kG; ++u) {
          if (g0 + u < S) {
            merge_load_row<E>(po + (size_t)(g0 + u) * D, v[u]);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = 0.f;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int sp = g0 + u;
        const float wk = (sp < S) ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), sp & 63)) : 0.f;
        const bool near = sp < near_splits;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (near) near_acc[e] = fmaf(wk, v[u][e], near_acc[e]);
          else far_acc[e] = fmaf(wk, v[u][e], far_acc[e]);
        }
      }
    }
    merge_finish<D>(near_acc, far_acc, W, M, sg, out_row, lse, lane);
    return;
  }

  // More than 64 splits: the maximum first, then each group's rows and
  // states requested together.
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, ml[2 * s]);
  M = wave_max(M, lane);

  float W = 0.f;
  for (int g0 = 0; g0 < S; g0 += kG) {
    float v[kG][E];
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      if (g0 + u < S) {
        merge_load_row<E>(po + (size_t)(g0 + u) * D, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[u][e] = 0.f;
      }
    }
    float w = 0.f;                                   // lane u < kG: weight of split g0 + u
    if (lane < kG && g0 + lane < S) {
      const float m = ml[2 * (g0 + lane)], l = ml[2 * (g0 + lane) + 1];
      w = (m == -INFINITY || l == 0.f) ? 0.f : l * expf(m - M);
    }
    W += w;
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
      const bool near = g0 + u < near_splits;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (near) near_acc[e] = fmaf(wk, v[u][e], near_acc[e]);
        else far_acc[e] = fmaf(wk, v[u][e], far_acc[e]);
      }
    }
  }
  W = wave_sum(W, lane);
  merge_finish<D>(near_acc, far_acc, W, M, sg, out_row, lse, lane);
}

}  // namespace kvq
