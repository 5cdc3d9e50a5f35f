// Cross-lane exchanges of a 64-lane wave on gfx950 without LDS: DPP inside a
// 16-lane row, v_permlane16_swap / v_permlane32_swap across rows.  Used by the
// Walsh-Hadamard butterflies and the wave reductions of the attention and
// merge kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

// After v_permlane16_swap on two copies of a value, lanes of even rows find
// the value of their xor-16 partner in the second copy and lanes of odd rows
// in the first; v_permlane32_swap does the same for the two wave halves.
// Compiler builtins, so that the compiler sees the instructions and pads
// their hazards (with matrix-core operands too).
__device__ inline void swap16(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b), false, false);
  const unsigned r0 = r[0], r1 = r[1];   // (copied out first: a bit cast of r[1] itself reads element 0)
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ inline void swap32(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b), false, false);
  const unsigned r0 = r[0], r1 = r[1];   // (copied out first: a bit cast of r[1] itself reads element 0)
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}

// Max / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48).
__device__ inline float max_rows(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = fmaxf(a, b);
  a = x;
  b = x;
  swap32(a, b);
  return fmaxf(a, b);
}
__device__ inline float sum_rows(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = a + b;
  a = x;
  b = x;
  swap32(a, b);
  return a + b;
}

// Value of lane l ^ M (M = 1, 2, 4, 8, 16, 32).  row_ror:n hands lane i the
// value of lane i - n (mod 16).
template <int M>
__device__ inline float xor_lane(float x, int lane) {
  const int xi = __builtin_bit_cast(int, x);
  if constexpr (M == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false));
  if constexpr (M == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false));
  if constexpr (M == 4) {
    const int up = __builtin_amdgcn_mov_dpp(xi, 0x12C, 0xF, 0xF, false);    // row_ror:12: lane i + 4
    const int dn = __builtin_amdgcn_mov_dpp(xi, 0x124, 0xF, 0xF, false);    // row_ror:4: lane i - 4
    return __builtin_bit_cast(float, (lane & 4) ? dn : up);
  }
  if constexpr (M == 8) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(xi, 0x128, 0xF, 0xF, false));
  if constexpr (M == 16) {
    float a = x, b = x;
    swap16(a, b);
    return (lane & 16) ? a : b;
  }
  if constexpr (M == 32) {
    float a = x, b = x;
    swap32(a, b);
    return (lane & 32) ? a : b;
  }
}

// Walsh-Hadamard butterfly across lanes at lane stride M: the lower lane of
// each pair keeps x + partner, the upper one partner - x.
template <int M>
__device__ inline float butterfly(float x, int lane) {
  const float o = xor_lane<M>(x, lane);
  return (lane & M) ? (o - x) : (x + o);
}

// The six cross-lane stages (lane strides 1..32) of a length-64*E transform
// whose element i*E + e sits in lane i, slot e.
__device__ inline float fwht_lanes(float x, int lane) {
  x = butterfly<1>(x, lane);
  x = butterfly<2>(x, lane);
  x = butterfly<4>(x, lane);
  x = butterfly<8>(x, lane);
  x = butterfly<16>(x, lane);
  return butterfly<32>(x, lane);
}

__device__ inline float wave_max(float x, int lane) {
  x = fmaxf(x, xor_lane<1>(x, lane));
  x = fmaxf(x, xor_lane<2>(x, lane));
  x = fmaxf(x, xor_lane<4>(x, lane));
  x = fmaxf(x, xor_lane<8>(x, lane));
  return max_rows(x);
}

__device__ inline float wave_sum(float x, int lane) {
  x += xor_lane<1>(x, lane);
  x += xor_lane<2>(x, lane);
  x += xor_lane<4>(x, lane);
  x += xor_lane<8>(x, lane);
  return sum_rows(x);
}

}  // namespace kvq
