// Cross-lane helpers for one 64-lane wave on gfx950, with no LDS round trip:
// DPP moves within rows of 16 lanes and the v_permlane16/32_swap instructions
// between rows. Each full reduction leaves the same value in every lane (the
// pairs of each step hold equal values or are added in either order, and
// a + b == b + a), and its order is fixed, so results are reproducible.
#pragma once

#include <hip/hip_runtime.h>

namespace vq {

// DPP controls: 0xB1 quad_perm [1,0,3,2] (lane ^ 1), 0x4E quad_perm [2,3,0,1]
// (lane ^ 2), 0x141 row_half_mirror (lane i <-> 7 - i within each 8 lanes),
// 0x140 row_mirror (lane i <-> 15 - i within each 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The values of lanes i and i ^ 16 (a) and of lanes i and i ^ 32 (b): the swap
// exchanges the odd rows (16) or the upper half (32) of its first operand with
// the even rows or lower half of the second, so with both operands v each lane
// ends up holding v[i] and its partner's value.
struct LanePair {
  float a, b;
};
__device__ __forceinline__ LanePair xor16_pair(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair xor32_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Sum over each aligned group of 8 lanes, the same value in all 8 (the pairs
// of each step are those of an xor-1, xor-2, xor-4 butterfly).
__device__ __forceinline__ float sum8_lanes(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  return v + dpp_f32<0x141>(v);
}

// Sum over the whole wave: groups of 8, then 16, then rows 16 and 32 apart.
__device__ __forceinline__ float sum64_lanes(float v) {
  v = sum8_lanes(v);
  v += dpp_f32<0x140>(v);
  const LanePair p = xor16_pair(v);
  v = p.a + p.b;
  const LanePair q = xor32_pair(v);
  return q.a + q.b;
}

// Maximum over the whole wave, in the same steps.
__device__ __forceinline__ float max64_lanes(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  const LanePair p = xor16_pair(v);
  v = fmaxf(p.a, p.b);
  const LanePair q = xor32_pair(v);
  return fmaxf(q.a, q.b);
}

// Bitwise OR and AND of a 32-bit value over the whole wave, in the same steps.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t or64_lanes(uint32_t v) {
  v |= dpp_u32<0xB1>(v);
  v |= dpp_u32<0x4E>(v);
  v |= dpp_u32<0x141>(v);
  v |= dpp_u32<0x140>(v);
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = p[0] | p[1];
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return q[0] | q[1];
}
__device__ __forceinline__ uint32_t and64_lanes(uint32_t v) {
  v &= dpp_u32<0xB1>(v);
  v &= dpp_u32<0x4E>(v);
  v &= dpp_u32<0x141>(v);
  v &= dpp_u32<0x140>(v);
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = p[0] & p[1];
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return q[0] & q[1];
}

}  // namespace vq
