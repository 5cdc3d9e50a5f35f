// Split merge and the single inverse rotation, gfx950.
//
// One work-group of D threads per (b, query head); thread j owns output
// coordinate j.  All threads read the split states (m_s, l_s), form
//   M = max m_s, w_s = l_s exp(m_s - M), W = sum w_s,
// and accumulate near-tier splits (original domain) and far-tier splits
// (rotated domain) separately.  The far sum is mapped back once with
// R^T y = s * (H y) / sqrt(D), the Walsh-Hadamard transform running in LDS.
// Source: "FoveatedKV", "Making it fast" (split-K partial states merged after
// the fused pass; near and far tiers share one softmax).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const float *__restrict__ part_o, const float *__restrict__ part_ml,
                                                 int splits, int near_splits, const int8_t *__restrict__ signs,
                                                 float *__restrict__ out, float *__restrict__ lse) {
  __shared__ float y[D];
  const int j = threadIdx.x;
  const size_t row = blockIdx.x;
  const int S = splits + near_splits;
  const float *ml = part_ml + row * S * 2;
  const float *po = part_o + row * S * D;

  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float W = 0.f, near_acc = 0.f, far_acc = 0.f;
  for (int s = 0; s < S; ++s) {
    const float m = ml[2 * s], l = ml[2 * s + 1];
    const float w = (m == -INFINITY || l == 0.f) ? 0.f : l * expf(m - M);
    W += w;
    const float o = po[(size_t)s * D + j];
    if (s < near_splits) near_acc = fmaf(w, o, near_acc); else far_acc = fmaf(w, o, far_acc);
  }
  y[j] = far_acc;
  __syncthreads();
  for (int len = 1; len < D; len <<= 1) {
    const bool active = j < D / 2;
    const int lo = active ? (j / len) * 2 * len + (j % len) : 0;
    const float a = active ? y[lo] : 0.f, c = active ? y[lo + len] : 0.f;
    __syncthreads();
    if (active) {
      y[lo] = a + c;
      y[lo + len] = a - c;
    }
    __syncthreads();
  }
  const float far = (signs[j] < 0 ? -y[j] : y[j]) * rsqrtf((float)D);
  out[row * D + j] = (W > 0.f) ? (near_acc + far) / W : 0.f;
  if (lse && j == 0) lse[row] = (W > 0.f) ? M + logf(W) : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream, bool *supported) {
  *supported = true;
  const dim3 grid(a.batch * a.q_heads);
  switch (a.head_dim) {
    case 64:
      hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, stream, a.part_o, a.part_ml, a.num_splits,
                         a.num_near_splits, a.signs, a.out, a.lse);
      break;
    case 128:
      hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(128), 0, stream, a.part_o, a.part_ml, a.num_splits,
                         a.num_near_splits, a.signs, a.out, a.lse);
      break;
    case 256:
      hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(256), 0, stream, a.part_o, a.part_ml, a.num_splits,
                         a.num_near_splits, a.signs, a.out, a.lse);
      break;
    default:
      *supported = false;
      return hipSuccess;
  }
  return hipGetLastError();
}

}  // namespace kvq
