// Split-merge kernel: one wave per (b, query head) row; the merge itself is
// merge_row.
// Source: "FoveatedKV", "Making it fast" (split-K partial states merged after
// the fused pass; near and far tiers share one softmax).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"
#include "kvq_merge.h"

namespace kvq {
namespace {

template <int D>
__global__ __launch_bounds__(64) void merge_kernel(const float *__restrict__ part_o, const float *__restrict__ part_ml,
                                                  int splits, int near_splits, const int8_t *__restrict__ signs,
                                                  float *__restrict__ out, float *__restrict__ lse) {
  const size_t row = blockIdx.x;
  const int S = splits + near_splits;
  merge_row<D>(part_o + row * S * D, part_ml + row * S * 2, splits, near_splits, signs, out + row * D,
               lse ? lse + row : nullptr, threadIdx.x);
}

template <int D>
hipError_t go(const MergeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel<D>, dim3(a.batch * a.q_heads), dim3(64), 0, stream, a.part_o, a.part_ml,
                     a.num_splits, a.num_near_splits, a.signs, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream, bool *supported) {
  *supported = true;
  switch (a.head_dim) {
    case 64: return go<64>(a, stream);
    case 128: return go<128>(a, stream);
    case 256: return go<256>(a, stream);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace kvq
