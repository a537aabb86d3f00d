// wave.hpp -- wavefront-level helpers for 64-lane CDNA4 waves.
//
// Group reductions over 2, 4, 8 or 16 neighbouring lanes use DPP (quad
// permutes, then the half-row and row mirrors), which never leave the VALU;
// the last two steps of a whole-wave sum go through ds_swizzle/bpermute.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// DPP control words (gfx9 encoding)
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within each 8
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within each 16

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Ctrl, 0xF, 0xF, false);
}
template <int Ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}

// max over aligned groups of N lanes (N = 1, 2, 4, 8, 16); every lane of a
// group receives the group's maximum
template <int N>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) v = max(v, dpp_u32<kDppQuadXor1>(v));
  if constexpr (N >= 4) v = max(v, dpp_u32<kDppQuadXor2>(v));
  if constexpr (N >= 8) v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  if constexpr (N >= 16) v = max(v, dpp_u32<kDppRowMirror>(v));
  return v;
}

// sum over the whole wave; every lane receives the total
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// a value the compiler may keep in a scalar register (the caller guarantees
// it is the same on every active lane)
__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace kvc
