// Quantize-on-append for Lloyd-Max keys and values, gfx950: the bulk path.
//
// Same encoding as the reference kernel in kvq_append.hip (sign flip, exact
// unnormalised Walsh-Hadamard transform in float64, exact fp16 norm, code =
// number of decision midpoints at or below the coordinate, LSB-first
// packing), organised for throughput:
//   * 16 coordinates per lane, D/16 lanes per vector (4, 8 or 16);
//   * the butterflies of strides 1..8 run inside the lane; one transpose
//     through LDS brings the coordinates that the strides 16..D/2 pair
//     into the same lane, so every butterfly is a register op (no cross-lane
//     exchange of doubles);
//   * the code comes from a 1024-bin table over t = z / ||x|| (the
//     coordinate on the N(0,1) scale): a bin holds the code at its left end
//     and the one decision midpoint inside it (or +inf), so a code is one
//     table read and one compare, in fp32: the rounding of t and of the
//     midpoint stays below 4e-7 on that scale, inside the 1e-6 band around a
//     midpoint that the pages' parity contract leaves open;
//   * codes go back through LDS in coordinate order and each lane packs and
//     stores its 16 codes with one store.
// fp8 keys keep the reference kernel.
// Sources: "The Engineering Behind AdapTQ", "The Math Fix" (sign flip + FWHT,
// add/sub only); VeloxQuant-MLX "Stage 2" (normalise, fp16 norm, nearest
// centroid) and "The Bit-Packing Problem" (LSB-first layout).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kCpl = 16;                  // coordinates per lane
constexpr int kBins = 1024;               // code table bins over t in [-kRange, kRange)
constexpr float kRange = 8.f;
constexpr float kBinScale = kBins / (2.f * kRange);
constexpr float kBinEdgeSlack = 1e-3f;    // each bin's rule also holds this far past its edges
constexpr int kVpt = 8;                   // vectors per lane group, one after another (amortises the table)

__device__ inline double half_value_d(uint32_t bits) {
  if (bits >= 0x7C00u) return 65536.0;    // one step past the largest finite fp16
  return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// RNE_fp16(sqrt(S)) with an exact final decision against the squared fp16
// midpoints (the same rule as the reference kernel).
__device__ inline uint16_t norm_fp16(double S) {
  if (!(S > 0.0)) return 0;
  if (S >= 65520.0 * 65520.0) return 0x7C00;
  const float rf = (float)sqrt(S);
  uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)rf);
  if (h > 0x7BFFu) h = 0x7BFFu;
  if (h == 0u) h = 1u;
  const double v = half_value_d(h);
  const double lo = 0.5 * (half_value_d(h - 1) + v);
  const double hi = 0.5 * (v + half_value_d(h + 1));
  if (S < lo * lo || (S == lo * lo && (h & 1u))) h -= 1;
  else if (S > hi * hi || (S == hi * hi && (h & 1u))) h += 1;
  return (uint16_t)h;
}

template <typename T>
__device__ inline void load16(const T *p, double (&x)[kCpl]);

template <>
__device__ inline void load16<_Float16>(const _Float16 *p, double (&x)[kCpl]) {
  const uint4 a = reinterpret_cast<const uint4 *>(p)[0];
  const uint4 b = reinterpret_cast<const uint4 *>(p)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
    x[2 * i + 1] = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
}

template <>
__device__ inline void load16<float>(const float *p, double (&x)[kCpl]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 a = reinterpret_cast<const float4 *>(p)[i];
    x[4 * i] = a.x;
    x[4 * i + 1] = a.y;
    x[4 * i + 2] = a.z;
    x[4 * i + 3] = a.w;
  }
}

// In-register butterflies over the strides S, 2S, ... < N*S of groups of N
// elements spaced S apart inside v (sum in the lower slot, difference in the
// upper one).
template <int N, int S, int LEN>
__device__ inline void butterflies(double (&v)[LEN]) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < LEN; ++i) {
      const int k = (i / S) % N;
      if (!(k & h)) {
        const double a = v[i], b = v[i + h * S];
        v[i] = a + b;
        v[i + h * S] = a - b;
      }
    }
  }
}

struct Stream {
  const void *in;
  uint8_t *codes;
  uint16_t *norms;
  const float *centroids;
};

struct TableEntry {
  float boundary;      // the decision midpoint inside the bin (t scale), or +inf
  uint32_t code_lo;    // number of midpoints left of the bin
};

// fp16 or fp32 input as float (exact).
template <typename T>
__device__ inline void load16f(const T *p, float (&x)[kCpl]);

template <>
__device__ inline void load16f<_Float16>(const _Float16 *p, float (&x)[kCpl]) {
  const uint4 a = reinterpret_cast<const uint4 *>(p)[0];
  const uint4 b = reinterpret_cast<const uint4 *>(p)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
    x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
}

template <>
__device__ inline void load16f<float>(const float *p, float (&x)[kCpl]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 a = reinterpret_cast<const float4 *>(p)[i];
    x[4 * i] = a.x;
    x[4 * i + 1] = a.y;
    x[4 * i + 2] = a.z;
    x[4 * i + 3] = a.w;
  }
}

template <int N, int S, int LEN>
__device__ inline void butterflies_f(float (&v)[LEN]) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < LEN; ++i) {
      const int k = (i / S) % N;
      if (!(k & h)) {
        const float a = v[i], b = v[i + h * S];
        v[i] = a + b;
        v[i + h * S] = a - b;
      }
    }
  }
}

// Code of t through the table: the count of midpoints left of t's bin plus
// the bin's own midpoint if t is at or past it; *near is set when t lies
// within `margin` of that midpoint.
__device__ inline uint32_t table_code(const TableEntry *table, float t, float margin, bool *near) {
  const float f = fmaf(t, kBinScale, kRange * kBinScale);
  const int bn = min(max((int)f, 0), kBins - 1);
  const TableEntry te = table[bn];
  *near = *near || (fabsf(t - te.boundary) <= margin);
  return te.code_lo + (t >= te.boundary ? 1u : 0u);
}

// One vector in float64, as the reference kernel computes it (the
// butterflies are exact for fp16 input; each code counts the float64
// midpoints at or below u = z / sqrt(D ||x||^2)): its codes go to cb in
// coordinate order; returns the fp16 norm bits.
template <int D, int BITS, typename T>
__device__ uint16_t encode_exact(const T *src, const uint32_t (&smask)[kCpl], double *vb, const float *centroids,
                                 int lv) {
  constexpr int LPV = D / kCpl;
  constexpr int GROUPS = kCpl / LPV;
  constexpr int L = 1 << BITS;
  double x[kCpl];
  load16<T>(src, x);
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < kCpl; ++e) ss = fma(x[e], x[e], ss);
#pragma unroll
  for (int e = 0; e < kCpl; ++e) x[e] = smask[e] ? -x[e] : x[e];
  butterflies<kCpl, 1, kCpl>(x);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int e = 0; e < kCpl; ++e) vb[lv * kCpl + e] = x[e];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  double z[kCpl];
#pragma unroll
  for (int g = 0; g < GROUPS; ++g) {
#pragma unroll
    for (int k = 0; k < LPV; ++k) z[g * LPV + k] = vb[GROUPS * lv + g + kCpl * k];
  }
  butterflies<LPV, 1, kCpl>(z);
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) ss += __shfl_xor(ss, m);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint8_t *cb = reinterpret_cast<uint8_t *>(vb);
  if (ss > 0.0) {
    double mid[L - 1];
#pragma unroll
    for (int i = 0; i < L - 1; ++i) mid[i] = 0.5 * ((double)centroids[i] + (double)centroids[i + 1]);
    const double r = 1.0 / sqrt((double)D * ss);
#pragma unroll
    for (int i = 0; i < kCpl; ++i) {
      const double u = z[i] * r;
      uint32_t code = 0;
#pragma unroll
      for (int m = 0; m < L - 1; ++m) code += (u >= mid[m]) ? 1u : 0u;
      const int g = i / LPV, k = i % LPV;
      cb[GROUPS * lv + g + kCpl * k] = (uint8_t)code;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kCpl; ++i) {
      const int g = i / LPV, k = i % LPV;
      cb[GROUPS * lv + g + kCpl * k] = (uint8_t)(L / 2);
    }
  }
  return norm_fp16(ss);
}

template <int D, int BITS, typename T>
__device__ void encode_fast(const Stream &st, const int8_t *__restrict__ signs, int n_new, int capacity,
                            int start_pos, double *buf, TableEntry *table) {
  constexpr int LPV = D / kCpl;              // lanes per vector
  constexpr int VPB = kThreads / LPV;        // vectors per block
  constexpr int L = 1 << BITS;
  constexpr int GROUPS = kCpl / (D / kCpl);  // low indices held per lane after the transpose
  constexpr int BSTRIDE = D + 1;             // doubles per vector in buf (odd: staggers the banks)
  constexpr int STAGES = __builtin_ctz(D);   // butterfly stages
  static_assert(D / kCpl * GROUPS == kCpl, "transpose shape");

  // ---- the code table for this stream (t = z / ||x||, N(0,1) scale) ----
  {
    const double root_d = sqrt((double)D);
    double mid[L - 1];
#pragma unroll
    for (int i = 0; i < L - 1; ++i)
      mid[i] = 0.5 * ((double)st.centroids[i] + (double)st.centroids[i + 1]) * root_d;
    for (int bn = threadIdx.x; bn < kBins; bn += kThreads) {
      const double lo = (double)bn / kBinScale - kRange - kBinEdgeSlack;
      const double hi = (double)(bn + 1) / kBinScale - kRange + kBinEdgeSlack;
      uint32_t below = 0;
      float bnd = INFINITY;
#pragma unroll
      for (int i = 0; i < L - 1; ++i) {
        below += (mid[i] < lo) ? 1u : 0u;
        bnd = (mid[i] >= lo && mid[i] < hi) ? (float)mid[i] : bnd;
      }
      table[bn] = TableEntry{bnd, below};
    }
  }
  __syncthreads();

  const int lv = threadIdx.x % LPV;
  const int vloc = threadIdx.x / LPV;
  const int bh = blockIdx.z;
  double *vb = buf + vloc * BSTRIDE;
  float *fb = reinterpret_cast<float *>(vb);
  uint8_t *cb = reinterpret_cast<uint8_t *>(vb);

  // sign masks of coordinates 16 lv .. 16 lv + 15 (bit 31 set where s = -1)
  uint32_t smask[kCpl];
  {
    const uint4 sr = *reinterpret_cast<const uint4 *>(signs + lv * kCpl);
    const uint32_t sw[4] = {sr.x, sr.y, sr.z, sr.w};
#pragma unroll
    for (int e = 0; e < kCpl; ++e) smask[e] = ((sw[e >> 2] >> (8 * (e & 3) + 7)) & 1u) << 31;
  }

  for (int it = 0; it < kVpt; ++it) {
    const int tok = (blockIdx.x * kVpt + it) * VPB + vloc;
    if (tok >= n_new) break;
    const T *src = static_cast<const T *>(st.in) + ((size_t)bh * n_new + tok) * D + lv * kCpl;

    // ---- float path: sign flip, butterflies, norm, codes; flags what it
    // cannot decide within its error bound ----
    float x[kCpl];
    load16f<T>(src, x);
    float ss = 0.f, sa = 0.f;
#pragma unroll
    for (int e = 0; e < kCpl; ++e) {
      ss = fmaf(x[e], x[e], ss);
      sa += fabsf(x[e]);
      x[e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x[e]) ^ smask[e]);
    }
    butterflies_f<kCpl, 1, kCpl>(x);
#pragma unroll
    for (int e = 0; e < kCpl; ++e) fb[lv * kCpl + e] = x[e];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float z[kCpl];                           // z[g * LPV + k] = coordinate GROUPS lv + g + 16 k
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
#pragma unroll
      for (int k = 0; k < LPV; ++k) z[g * LPV + k] = fb[GROUPS * lv + g + kCpl * k];
    }
    butterflies_f<LPV, 1, kCpl>(z);
#pragma unroll
    for (int m = 1; m < LPV; m <<= 1) {
      ss += __shfl_xor(ss, m);
      sa += __shfl_xor(sa, m);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // Error bounds: each butterfly stage rounds once (<= 2^-24 of a partial
    // sum, itself <= sum |x|); ss carries < 1e-6 relative error, so t =
    // z / ||x|| (fp32 reciprocal square root) is within
    // STAGES 2^-24 sa / ||x|| + 2e-6 |t| of the exact value.  Codes within
    // that bound plus the 1e-6 band of a midpoint, and fp16 norms near a
    // rounding midpoint, go to the float64 path.
    bool near = !(ss > 1e-30f && ss < 1e30f);       // (also zero vectors: exact path)
    uint16_t norm16 = 0;
    if (!near) {
      const double S = (double)ss;
      norm16 = norm_fp16(S);
      const double v = half_value_d(norm16);
      const double mlo = 0.5 * (half_value_d(norm16 - 1) + v), mhi = 0.5 * (v + half_value_d(norm16 + 1));
      near = fabs(S - mlo * mlo) <= 4e-6 * S || fabs(S - mhi * mhi) <= 4e-6 * S;
      const float r = __builtin_amdgcn_rsqf(ss);
      const float base = (float)STAGES * 5.97e-8f * sa * r + 1.5e-6f;
#pragma unroll
      for (int i = 0; i < kCpl; ++i) {
        const float t = z[i] * r;
        const int g = i / LPV, k = i % LPV;
        cb[GROUPS * lv + g + kCpl * k] = (uint8_t)table_code(table, t, fmaf(2e-6f, fabsf(t), base), &near);
      }
    }
    // the vector's lanes agree on the path
    uint32_t nv = near ? 1u : 0u;
#pragma unroll
    for (int m = 1; m < LPV; m <<= 1) nv |= __shfl_xor(nv, m);
    if (nv) norm16 = encode_exact<D, BITS, T>(src, smask, vb, st.centroids, lv);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // ---- pack this lane's 16 codes (coordinates 16 lv .. 16 lv + 15), LSB
    // first (the vector's LDS slice is 8-byte aligned) ----
    const size_t slot = (size_t)bh * capacity + start_pos + tok;
    constexpr int ROW = D * BITS / 8;
    uint8_t *row = st.codes + slot * ROW;
    if (lv == 0) st.norms[slot] = norm16;
    const uint2 c01 = reinterpret_cast<const uint2 *>(cb + lv * kCpl)[0];
    const uint2 c23 = reinterpret_cast<const uint2 *>(cb + lv * kCpl)[1];
    const uint32_t cws[4] = {c01.x, c01.y, c23.x, c23.y};
    uint64_t packed = 0;
#pragma unroll
    for (int i = 0; i < kCpl; ++i) packed |= (uint64_t)((cws[i >> 2] >> (8 * (i & 3))) & 0xFFu) << (BITS * i);
    uint8_t *dst = row + lv * (kCpl * BITS / 8);
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint2 *>(dst) = make_uint2((uint32_t)packed, (uint32_t)(packed >> 32));
    } else if constexpr (BITS == 2) {
      *reinterpret_cast<uint32_t *>(dst) = (uint32_t)packed;
    } else {  // 3 bits: 48 stream bits at byte offset 6 lv (2-byte aligned)
#pragma unroll
      for (int i = 0; i < 3; ++i) reinterpret_cast<uint16_t *>(dst)[i] = (uint16_t)(packed >> (16 * i));
    }
    // the next vector reuses this LDS slice
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

template <int D, int KB, int VB, typename T>
__global__ __launch_bounds__(kThreads) void append_fast_kernel(Stream ks, Stream vs, const int8_t *__restrict__ signs,
                                                               int n_new, int capacity, int start_pos) {
  __shared__ __attribute__((aligned(16))) double buf[(kThreads / (D / kCpl)) * (D + 1) + 2];
  __shared__ TableEntry table[kBins];
  if (blockIdx.y == 0) encode_fast<D, KB, T>(ks, signs, n_new, capacity, start_pos, buf, table);
  else encode_fast<D, VB, T>(vs, signs, n_new, capacity, start_pos, buf, table);
}

template <int D, int KB, int VB>
hipError_t go(const AppendArgs &a, hipStream_t stream) {
  constexpr int VPB = kThreads / (D / kCpl);
  dim3 grid((a.n_new + VPB * kVpt - 1) / (VPB * kVpt), 2, a.batch * a.kv_heads);
  Stream ks{a.k, a.k_codes, a.k_norms, a.k_centroids};
  Stream vs{a.v, a.v_codes, a.v_norms, a.v_centroids};
  if (a.in_f16)
    hipLaunchKernelGGL((append_fast_kernel<D, KB, VB, _Float16>), grid, dim3(kThreads), 0, stream, ks, vs, a.signs,
                       a.n_new, a.capacity, a.start_pos);
  else
    hipLaunchKernelGGL((append_fast_kernel<D, KB, VB, float>), grid, dim3(kThreads), 0, stream, ks, vs, a.signs,
                       a.n_new, a.capacity, a.start_pos);
  return hipGetLastError();
}

template <int D, int KB>
hipError_t go_v(const AppendArgs &a, hipStream_t stream, bool *ok) {
  switch (a.v_format) {
    case 2: return go<D, KB, 2>(a, stream);
    case 3: return go<D, KB, 3>(a, stream);
    case 4: return go<D, KB, 4>(a, stream);
  }
  *ok = false;
  return hipSuccess;
}

template <int D>
hipError_t go_k(const AppendArgs &a, hipStream_t stream, bool *ok) {
  switch (a.k_format) {
    case 2: return go_v<D, 2>(a, stream, ok);
    case 3: return go_v<D, 3>(a, stream, ok);
    case 4: return go_v<D, 4>(a, stream, ok);
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

bool fast_append_supported(const AppendArgs &a) {
  // bulk appends only: a few tokens per (b, KV head) would not repay the
  // per-block code table
  const bool lm = a.k_format >= 2 && a.k_format <= 4 && a.v_format >= 2 && a.v_format <= 4;
  return lm && (a.head_dim == 64 || a.head_dim == 128 || a.head_dim == 256) && a.batch * a.kv_heads <= 65535 &&
         a.n_new >= 64 && a.outlier_idx == nullptr && a.qjl_proj == nullptr;
}

hipError_t launch_append_fast(const AppendArgs &a, hipStream_t stream) {
  bool ok = true;
  hipError_t e = hipSuccess;
  switch (a.head_dim) {
    case 64: e = go_k<64>(a, stream, &ok); break;
    case 128: e = go_k<128>(a, stream, &ok); break;
    case 256: e = go_k<256>(a, stream, &ok); break;
    default: ok = false;
  }
  return ok ? e : hipErrorInvalidValue;
}

}  // namespace kvq
