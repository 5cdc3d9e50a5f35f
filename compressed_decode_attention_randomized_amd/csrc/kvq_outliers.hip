// Outlier-channel calibration of the key outlier stream ("I Ported a Google
// Research Paper to Apple Silicon", "Outlier Two-Stream Cache": a calibration
// pass over the first tokens, then detection of the largest-variance
// channels).
//
// One work-group of D threads per (b, KV head).  Thread c takes channel c's
// population variance over the n calibration tokens in float64 (the mean
// first, then the mean squared deviation); kOutlierCount rounds of a
// work-group argmax (ties to the lower channel) pick the channels, which are
// written ascending.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

template <typename T>
__device__ inline double as_double(T v);
template <>
__device__ inline double as_double<_Float16>(_Float16 v) { return (double)(float)v; }
template <>
__device__ inline double as_double<float>(float v) { return (double)v; }

template <int D, typename T>
__global__ __launch_bounds__(D) void calibrate_kernel(const T *__restrict__ keys, int n, int32_t *__restrict__ idx) {
  __shared__ double rv[D];
  __shared__ int ri[D];
  __shared__ int chosen[kOutlierCount];
  const int c = threadIdx.x;
  const size_t bh = blockIdx.x;
  const T *x = keys + bh * (size_t)n * D + c;
  double sum = 0.0;
  for (int t = 0; t < n; ++t) sum += as_double<T>(x[(size_t)t * D]);
  const double mean = sum / n;
  double ss = 0.0;
  for (int t = 0; t < n; ++t) {
    const double dv = as_double<T>(x[(size_t)t * D]) - mean;
    ss = fma(dv, dv, ss);
  }
  double var = ss / n;
  for (int r = 0; r < kOutlierCount; ++r) {
    rv[c] = var;
    ri[c] = c;
    __syncthreads();
    for (int s = D / 2; s > 0; s >>= 1) {
      if (c < s) {
        const double a = rv[c], b = rv[c + s];
        if (b > a || (b == a && ri[c + s] < ri[c])) {
          rv[c] = b;
          ri[c] = ri[c + s];
        }
      }
      __syncthreads();
    }
    if (c == 0) chosen[r] = ri[0];
    __syncthreads();
    if (c == chosen[r]) var = -1.0;                  // taken: below every variance
    __syncthreads();
  }
  if (c == 0) {
    int v[kOutlierCount];
#pragma unroll
    for (int i = 0; i < kOutlierCount; ++i) v[i] = chosen[i];
    for (int i = 1; i < kOutlierCount; ++i)
      for (int j = i; j > 0 && v[j - 1] > v[j]; --j) {
        const int t = v[j];
        v[j] = v[j - 1];
        v[j - 1] = t;
      }
#pragma unroll
    for (int i = 0; i < kOutlierCount; ++i) idx[bh * kOutlierCount + i] = v[i];
  }
}

template <int D>
hipError_t go(const void *keys, int in_f16, int pairs, int n, int32_t *idx, hipStream_t stream) {
  if (in_f16)
    hipLaunchKernelGGL((calibrate_kernel<D, _Float16>), dim3(pairs), dim3(D), 0, stream,
                       static_cast<const _Float16 *>(keys), n, idx);
  else
    hipLaunchKernelGGL((calibrate_kernel<D, float>), dim3(pairs), dim3(D), 0, stream, static_cast<const float *>(keys),
                       n, idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_calibrate(const void *keys, int in_f16, int batch, int kv_heads, int head_dim, int n,
                            int32_t *idx, hipStream_t stream) {
  const int pairs = batch * kv_heads;
  switch (head_dim) {
    case 64: return go<64>(keys, in_f16, pairs, n, idx, stream);
    case 128: return go<128>(keys, in_f16, pairs, n, idx, stream);
    default: return go<256>(keys, in_f16, pairs, n, idx, stream);
  }
}

}  // namespace kvq
