// Quantize-on-append kernel for gfx950.
//
// One key or value vector is encoded by D/8 consecutive lanes of a wave, each
// lane holding 8 consecutive coordinates (one 16-byte fp16 load).  Per vector:
//   1. sign flip, then the unnormalised Sylvester Walsh-Hadamard transform
//      (three butterfly stages inside the lane, log2(D/8) stages across lanes
//      by xor-shuffles), in float64: for fp16 input every partial sum is a
//      multiple of 2^-24 below 2^49, so the transform is exact;
//   2. squared norm in float64 from the original coordinates, reduced across
//      the lanes; the fp16 norm is rounded to nearest-even and then confirmed
//      against the exact squared fp16 midpoints;
//   3. each code is the count of decision midpoints m_i <= z_j / (sqrt(D)||x||),
//      found by a branch-free binary search over the midpoint table held in LDS
//      in float64 (midpoints of float32 centroids are exact in float64);
//   4. codes packed LSB-first: 8 codes per lane are 32 (4-bit), 24 (3-bit) or
//      16 (2-bit) stream bits at byte offset lane*bits.
// fp8 keys skip the norm: y = z / sqrt(D) is rounded to E4M3FN directly from
// float64 (nearest-even, saturating at 448).
// With a QJL sketch, each key's rotated-domain residual r = z / sqrt(D) -
// n16 * c[code] is kept in LDS in float64 (the lane computes its 8
// coordinates; the fp16 norm of r is decided exactly like the key norm); the
// work-group then forms the D x D product of the projection with the
// residuals of its vectors (one thread per sketch row and 8 vectors, the
// projection column read coalesced, residuals as LDS broadcasts), and each
// sign bit is S_i . r >= 0, gathered 64 rows at a time by a wave ballot.
// Sources: "The Engineering Behind AdapTQ", "The Math Fix" (sign flip + FWHT,
// add/sub only); VeloxQuant-MLX "Stage 2" (normalise, fp16 norm, nearest
// centroid) and "The Bit-Packing Problem" (LSB-first layout), "Stage 3: QJL Residual
// Correction" (sign sketch of the residual, its fp16 norm); "FoveatedKV",
// "The VR headset thing" (fp8 E4M3 far-tier keys).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kBlock = 256;

__device__ inline double half_bits_value(uint32_t bits) {
  if (bits >= 0x7C00u) return 65536.0;   // one step past the largest finite fp16
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits);
  return (double)(float)h;
}

// RNE_fp16(sqrt(S)) with an exact final decision against squared midpoints.
__device__ inline uint16_t fp16_norm(double S) {
  if (!(S > 0.0)) return 0;
  if (S >= 65520.0 * 65520.0) return 0x7C00;     // rounds past 65504 -> +inf
  float rf = (float)sqrt(S);
  uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)rf);
  if (h > 0x7BFFu) h = 0x7BFFu;
  if (h == 0u) h = 1u;
  const double v = half_bits_value(h);
  const double lo = 0.5 * (half_bits_value(h - 1) + v);
  const double hi = 0.5 * (v + half_bits_value(h + 1));
  if (S < lo * lo || (S == lo * lo && (h & 1u))) {
    h -= 1;
  } else if (S > hi * hi || (S == hi * hi && (h & 1u))) {
    h += 1;
  }
  return (uint16_t)h;
}

// E4M3FN code of a float64 value: nearest-even, saturating at +-448; a value
// that rounds to zero keeps its sign.
__device__ inline uint32_t e4m3_from_double(double y) {
  const uint32_t sign = (y < 0.0) ? 0x80u : 0u;
  const double a = fabs(y);
  uint32_t code;
  if (a < 0.015625) {                              // below 2^-6: subnormal grid 2^-9
    code = (uint32_t)rint(a * 512.0);              // 0..8; 8 is the smallest normal
  } else if (a >= 464.0) {
    code = 0x7Eu;
  } else {
    const uint64_t bits = __builtin_bit_cast(uint64_t, a);
    const int e = (int)((bits >> 52) & 0x7FF) - 1023;      // -6 .. 8
    const uint64_t man = bits & ((1ull << 52) - 1);
    const uint64_t half = 1ull << 48, lsb = (man >> 49) & 1ull;
    uint64_t m3 = (man + half - 1 + lsb) >> 49;             // round to 3 bits, ties even
    uint32_t ee = (uint32_t)(e + 7);
    if (m3 == 8) { m3 = 0; ee += 1; }
    code = (ee << 3) | (uint32_t)m3;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// v from lane ^ m (m < 32, within a vector's lanes): row-local DPP moves for
// m = 1, 2 and ds_swizzle in xor mode above (no LDS access, no address
// registers, shorter latency than a ds_bpermute shuffle).
__device__ inline uint32_t swap_xor_u32(uint32_t v, int m) {
  const int x = (int)v;
  if (m == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);     // quad_perm [1,0,3,2]
  if (m == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);     // quad_perm [2,3,0,1]
  if (m == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x101F);
  if (m == 8) return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x201F);
  return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x401F);
}

__device__ inline float swap_xor(float v, int m) {
  return __builtin_bit_cast(float, swap_xor_u32(__builtin_bit_cast(uint32_t, v), m));
}

__device__ inline double swap_xor(double v, int m) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = swap_xor_u32((uint32_t)b, m), hi = swap_xor_u32((uint32_t)(b >> 32), m);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <typename T>
__device__ inline void load8(const T *p, double (&x)[8]);

template <>
__device__ inline void load8<_Float16>(const _Float16 *p, double (&x)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
    x[2 * i + 1] = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
}

template <>
__device__ inline void load8<float>(const float *p, double (&x)[8]) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

struct Stream {
  const void *in;
  uint8_t *codes;
  uint16_t *norms;
  const float *centroids;
  // key outlier stream ("Outlier Two-Stream Cache"; NULL idx: off): the
  // vector's kOutlierCount channels idx are zeroed before the codec and
  // stored as int8 codes with an fp32 per-token scale
  const int32_t *out_idx;
  int8_t *out_codes;
  float *out_scales;
  // QJL residual sketch (keys; NULL proj: off): S^T [D][D] float32, sign
  // bytes [..][capacity][D/8], fp16 residual norms [..][capacity]
  const float *qjl_proj;
  uint8_t *qjl_signs;
  uint16_t *qjl_norms;
};

// Residuals of a work-group's vectors, [D][VPB] float64 (VPB * D = 2048).
constexpr int kResidual = 2048;

// Encode the vectors of one stream (keys or values).  BITS in {2,3,4} for
// Lloyd-Max codes, 8 for fp8.
template <int D, int BITS, typename T, bool QJL = false>
__device__ void encode(const Stream &st, const int8_t *__restrict__ signs, int nvec, int n_new,
                       int capacity, int start_pos, double *mids, double *cents = nullptr,
                       double *resid = nullptr) {
  constexpr int LPV = D / 8;            // lanes per vector
  constexpr int VPB = kBlock / LPV;     // vectors per block
  constexpr int L = 1 << (BITS == 8 ? 1 : BITS);
  constexpr int ROW = D * BITS / 8;

  // the vector and sign loads go out before the midpoint table's barrier,
  // so a one-token append waits for memory once
  const int lv = threadIdx.x % LPV;
  const int vec = blockIdx.x * VPB + threadIdx.x / LPV;
  const bool live = vec < nvec;
  double x[8];
  uint2 sraw = make_uint2(0u, 0u);
  if (live) {
    load8<T>(static_cast<const T *>(st.in) + (size_t)vec * D + lv * 8, x);
    sraw = *reinterpret_cast<const uint2 *>(signs + lv * 8);
  }
  if (BITS != 8) {
    if (threadIdx.x < L - 1) {
      mids[threadIdx.x] = 0.5 * ((double)st.centroids[threadIdx.x] + (double)st.centroids[threadIdx.x + 1]);
    }
    if (QJL && threadIdx.x < L) cents[threadIdx.x] = (double)st.centroids[threadIdx.x];
    __syncthreads();
  }
  if (!live) return;

  const int bvec = vec / n_new;                    // (b * Hkv + h)
  const int t = start_pos + (vec - bvec * n_new);
  const size_t slot = (size_t)bvec * capacity + t;

  if (st.out_idx) {
    // outlier channels of this vector: slot k of the stream holds channel
    // idx[k]; the lane's coordinates lv*8 .. lv*8+7 are checked against all
    const int4 i0 = reinterpret_cast<const int4 *>(st.out_idx + (size_t)bvec * kOutlierCount)[0];
    const int4 i1 = reinterpret_cast<const int4 *>(st.out_idx + (size_t)bvec * kOutlierCount)[1];
    const int idx[kOutlierCount] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
    int which[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      which[e] = -1;
#pragma unroll
      for (int k = 0; k < kOutlierCount; ++k) which[e] = (idx[k] == lv * 8 + e) ? k : which[e];
      if (which[e] >= 0) amax = fmaxf(amax, fabsf((float)x[e]));
    }
#pragma unroll
    for (int m = 1; m < LPV; m <<= 1) amax = fmaxf(amax, swap_xor(amax, m));
    const float scale = amax / 127.f;               // one float32 rounding
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (which[e] >= 0) {
        const double u = (scale > 0.f) ? x[e] / (double)scale : 0.0;
        const double c = fmin(fmax(rint(u), -127.0), 127.0);
        st.out_codes[slot * kOutlierCount + which[e]] = (int8_t)(int)c;
        x[e] = 0.0;
      }
    }
    if (lv == 0) st.out_scales[slot] = scale;
  }

  // squared norm from the original coordinates
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fma(x[e], x[e], ss);

  // sign flip
  const uint32_t sw[2] = {sraw.x, sraw.y};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int8_t s = (int8_t)((sw[e >> 2] >> (8 * (e & 3))) & 0xFF);
    x[e] = (s < 0) ? -x[e] : x[e];
  }

  // Walsh-Hadamard: strides 1, 2, 4 inside the lane ...
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!(i & h)) {
        const double a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  // ... strides 8, 16, ... across lanes
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) {
    const bool upper = (lv & m) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double o = swap_xor(x[e], m);
      x[e] = upper ? (o - x[e]) : (x[e] + o);
    }
  }
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) ss += swap_xor(ss, m);

  uint8_t *row = st.codes + slot * ROW;

  if (BITS == 8) {
    const double inv_root_d = 1.0 / sqrt((double)D);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t c = e4m3_from_double(x[e] * inv_root_d);
      if (e < 4) lo |= c << (8 * e); else hi |= c << (8 * (e - 4));
    }
    *reinterpret_cast<uint2 *>(row + lv * 8) = make_uint2(lo, hi);
    return;
  }

  const uint16_t n16 = fp16_norm(ss);
  if (lv == 0) st.norms[slot] = n16;

  uint32_t packed = 0;
  if (ss > 0.0) {
    const double inv = 1.0 / sqrt((double)D * ss);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double u = x[e] * inv;
      int idx = 0;
#pragma unroll
      for (int step = L / 2; step >= 1; step >>= 1) {
        if (u >= mids[idx + step - 1]) idx += step;
      }
      packed |= (uint32_t)idx << (BITS * e);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) packed |= (uint32_t)(L / 2) << (BITS * e);
  }
  if (BITS == 4) {
    *reinterpret_cast<uint32_t *>(row + lv * 4) = packed;
  } else if (BITS == 2) {
    *reinterpret_cast<uint16_t *>(row + lv * 2) = (uint16_t)packed;
  } else {  // 3 bits: 24 stream bits at byte offset 3*lv
    row[lv * 3 + 0] = (uint8_t)(packed & 0xFF);
    row[lv * 3 + 1] = (uint8_t)((packed >> 8) & 0xFF);
    row[lv * 3 + 2] = (uint8_t)((packed >> 16) & 0xFF);
  }

  if constexpr (QJL && BITS != 8) {
    // residual in the rotated domain: y_j - n16 * c[code_j], y = z / sqrt(D)
    // (n16 * c is exact in float64, so r takes two roundings: y's and the
    // difference's)
    const double n = (n16 == 0) ? 0.0 : half_bits_value(n16);
    const int vloc = threadIdx.x / LPV;
    double rss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = (int)((packed >> (BITS * e)) & (uint32_t)(L - 1));
      const double r = x[e] / sqrt((double)D) - n * cents[c];
      rss = fma(r, r, rss);
      resid[(lv * 8 + e) * VPB + vloc] = r;
    }
#pragma unroll
    for (int m = 1; m < LPV; m <<= 1) rss += swap_xor(rss, m);
    if (lv == 0) st.qjl_norms[slot] = fp16_norm(rss);
  }
}

// Sign sketch of the residuals in `resid` (the work-group's VPB vectors):
// thread (i, g) forms S_i . r for sketch row i = tid % D and vectors
// 8g .. 8g+7; a wave holds 64 consecutive rows of 8 vectors, and one ballot
// per vector gives 64 sign bits, stored as one 8-byte word by lane k for
// vector k.
template <int D>
__device__ void sketch(const Stream &st, const double *resid, int nvec, int n_new, int capacity, int start_pos) {
  constexpr int LPV = D / 8, VPB = kBlock / LPV, kPer = 8;
  static_assert(VPB * D == kResidual && kPer * kBlock == kResidual && D >= 64, "sketch mapping");
  const int i = threadIdx.x % D, g = threadIdx.x / D;
  const int lane = threadIdx.x & 63;
  double acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.0;
  const float *col = st.qjl_proj + i;
#pragma unroll 16
  for (int j = 0; j < D; ++j) {
    const double s = (double)col[(size_t)j * D];
    const double *rv = resid + j * VPB + g * kPer;
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] = fma(s, rv[k], acc[k]);
  }
  const int i0 = i - lane;                       // the wave's first sketch row
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint64_t bits = __builtin_amdgcn_ballot_w64(acc[k] >= 0.0);
    const int vec = blockIdx.x * VPB + g * kPer + k;
    if (lane == k && vec < nvec) {
      const int bvec = vec / n_new;
      const size_t slot = (size_t)bvec * capacity + start_pos + (vec - bvec * n_new);
      *reinterpret_cast<uint64_t *>(st.qjl_signs + slot * (D / 8) + i0 / 8) = bits;
    }
  }
}

template <int D, int KB, int VB, typename T, bool QJL = false>
__global__ __launch_bounds__(kBlock) void append_kernel(Stream ks, Stream vs, const int8_t *__restrict__ signs,
                                                        int nvec, int n_new, int capacity, int start_pos) {
  __shared__ double mids[15];
  if (blockIdx.y == 0) {
    if constexpr (QJL) {
      __shared__ double cents[16];
      __shared__ double resid[kResidual];
      encode<D, KB, T, true>(ks, signs, nvec, n_new, capacity, start_pos, mids, cents, resid);
      __syncthreads();
      sketch<D>(ks, resid, nvec, n_new, capacity, start_pos);
    } else {
      encode<D, KB, T>(ks, signs, nvec, n_new, capacity, start_pos, mids);
    }
  } else {
    encode<D, VB, T>(vs, signs, nvec, n_new, capacity, start_pos, mids);
  }
}

template <int D, int KB, int VB>
hipError_t launch3(const AppendArgs &a, hipStream_t stream) {
  const int nvec = a.batch * a.kv_heads * a.n_new;
  constexpr int VPB = kBlock / (D / 8);
  dim3 grid((nvec + VPB - 1) / VPB, 2);
  Stream ks{a.k, a.k_codes, a.k_norms, a.k_centroids, a.outlier_idx, a.outlier_codes, a.outlier_scales,
            a.qjl_proj, a.qjl_signs, a.qjl_norms};
  Stream vs{a.v, a.v_codes, a.v_norms, a.v_centroids, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if constexpr (KB != 8) {
    if (a.qjl_proj) {
      if (a.in_f16) {
        hipLaunchKernelGGL((append_kernel<D, KB, VB, _Float16, true>), grid, dim3(kBlock), 0, stream, ks, vs, a.signs,
                           nvec, a.n_new, a.capacity, a.start_pos);
      } else {
        hipLaunchKernelGGL((append_kernel<D, KB, VB, float, true>), grid, dim3(kBlock), 0, stream, ks, vs, a.signs,
                           nvec, a.n_new, a.capacity, a.start_pos);
      }
      return hipGetLastError();
    }
  }
  if (a.in_f16) {
    hipLaunchKernelGGL((append_kernel<D, KB, VB, _Float16>), grid, dim3(kBlock), 0, stream, ks, vs, a.signs, nvec,
                       a.n_new, a.capacity, a.start_pos);
  } else {
    hipLaunchKernelGGL((append_kernel<D, KB, VB, float>), grid, dim3(kBlock), 0, stream, ks, vs, a.signs, nvec,
                       a.n_new, a.capacity, a.start_pos);
  }
  return hipGetLastError();
}

template <int D, int KB>
hipError_t launch2(const AppendArgs &a, hipStream_t stream, bool *ok) {
  switch (a.v_format) {
    case 2: return launch3<D, KB, 2>(a, stream);
    case 3: return launch3<D, KB, 3>(a, stream);
    case 4: return launch3<D, KB, 4>(a, stream);
  }
  *ok = false;
  return hipSuccess;
}

template <int D>
hipError_t launch1(const AppendArgs &a, hipStream_t stream, bool *ok) {
  switch (a.k_format) {
    case 2: return launch2<D, 2>(a, stream, ok);
    case 3: return launch2<D, 3>(a, stream, ok);
    case 4: return launch2<D, 4>(a, stream, ok);
    case 8: return launch2<D, 8>(a, stream, ok);
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t stream, bool *supported) {
  *supported = true;
  if (bulk_append_supported(a)) return launch_append_bulk(a, stream);
  if (fast_append_supported(a)) return launch_append_fast(a, stream);
  switch (a.head_dim) {
    case 64: return launch1<64>(a, stream, supported);
    case 128: return launch1<128>(a, stream, supported);
    case 256: return launch1<256>(a, stream, supported);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace kvq
