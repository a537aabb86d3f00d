// wave.hpp -- wavefront-level helpers for 64-lane CDNA4 waves.
//
// Group reductions over 2, 4, 8 or 16 neighbouring lanes use DPP (quad
// permutes, then the half-row and row mirrors), which never leave the VALU;
// a whole-wave sum finishes with the gfx9 row broadcasts and a readlane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// DPP control words (gfx9 encoding)
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within each 8
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within each 16
constexpr int kDppRowBcast15 = 0x142;     // lane 15 of each row into the next row
constexpr int kDppRowBcast31 = 0x143;     // lane 31 into rows 2 and 3

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

// sum over the whole wave, returned as a wave-uniform value: each 16-lane row
// is reduced with DPP, row_bcast:15 / row_bcast:31 fold the rows into lane
// 63, and v_readlane broadcasts it (no LDS traffic)
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast15, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast31, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Inclusive prefix sum over the 64 lanes: within each 16-lane row by DPP
// row shifts of 1, 2, 4 and 8 (lanes past a row's start read 0), then the
// row totals carried across rows by the row_bcast:15 / row_bcast:31
// broadcasts -- six VALU steps, no LDS round trip.
template <int Ctrl>
__device__ __forceinline__ int32_t dpp_shr_or_zero(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, Ctrl, 0xF, 0xF, true);
}
__device__ __forceinline__ int32_t wave_incl_scan_i32(int32_t v) {
  v += dpp_shr_or_zero<0x111>(v);               // row_shr:1
  v += dpp_shr_or_zero<0x112>(v);               // row_shr:2
  v += dpp_shr_or_zero<0x114>(v);               // row_shr:4
  v += dpp_shr_or_zero<0x118>(v);               // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);   // rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);   // rows 2, 3
  return v;
}

// Pack one byte from each of four lanes spaced D apart into a dword on the
// last of them: lane l receives byte(v[l-3D]) | byte(v[l-2D]) << 8 |
// byte(v[l-D]) << 16 | byte(v[l]) << 24.  The lanes read must lie in l's
// 16-lane row (DPP row_shr), which the callers' lane choice guarantees.
template <int D>
__device__ __forceinline__ uint32_t pack4_bytes_shr(uint32_t v) {
  const uint32_t b0 = dpp_u32<0x110 + 3 * D>(v) & 0xFFu;   // row_shr:3D
  const uint32_t b1 = dpp_u32<0x110 + 2 * D>(v) & 0xFFu;   // row_shr:2D
  const uint32_t b2 = dpp_u32<0x110 + D>(v) & 0xFFu;       // row_shr:D
  return b0 | (b1 << 8) | (b2 << 16) | ((v & 0xFFu) << 24);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// set `bit` in the optional device status word (lane 0 of the wave)
__device__ __forceinline__ void raise_status(int32_t* status, int32_t bit) {
  if (status != nullptr && lane_id() == 0) atomicOr(status, bit);
}

// Load from memory that no thread writes while the kernel runs (the caller's
// read-only inputs: offsets, positions, page tables, ids).  Going through the
// constant address space lets the compiler use a scalar load when the address
// is wave-uniform; its completion is then tracked by lgkmcnt, so waiting for
// it never waits for outstanding vector stores.
template <typename T>
__device__ __forceinline__ T ld_ro(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// n / d for the DivMagic of d (launch.hpp)
__device__ __forceinline__ uint32_t udiv_magic(uint32_t n, uint32_t m, int32_t sh1, int32_t sh2) {
  const uint32_t t = __umulhi(m, n);
  return (t + ((n - t) >> sh1)) >> sh2;
}

// a value the compiler may keep in a scalar register (the caller guarantees
// it is the same on every active lane)
__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace kvc
