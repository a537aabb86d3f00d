// codec.hpp -- bit-exact number-format conversions for the KV row codecs.
//
// Formats: bfloat16; OCP fp8 e4m3fn (bias 7, max 448, 0x7F/0xFF NaN);
// OCP fp4 e2m1 (values 0, .5, 1, 1.5, 2, 3, 4, 6); ue8m0 (a bare biased
// exponent).  Encoders round to nearest, ties to even, and work on integer
// bit fields so the result does not depend on any hardware rounding mode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// |x| ordering of finite bf16 values equals the integer ordering of their
// low 15 bits, so a group's amax is an integer max.  The four words each hold
// two bf16; the maxima are taken per 16-bit half (v_pk_max_u16).
__device__ __forceinline__ uint32_t absmax_bf16x8(uint4 x) {
  const uint32_t m = 0x7FFF7FFFu;
  const u16x2 a = __builtin_bit_cast(u16x2, x.x & m), b = __builtin_bit_cast(u16x2, x.y & m);
  const u16x2 c = __builtin_bit_cast(u16x2, x.z & m), d = __builtin_bit_cast(u16x2, x.w & m);
  const u16x2 e = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                            __builtin_elementwise_max(c, d));
  return max((uint32_t)e.x, (uint32_t)e.y);
}

// ue8m0 scale exponent of a group from the fp32 bits of its amax: the
// closed form of 127 + ceil(log2(max(amax / 448, 1e-4))) given in sglang PR
// #39652, Review.  amax / 448 = 2^(e - 135) (1 + f) / 1.75, whose log2 rounds
// up past e - 135 exactly when the mantissa exceeds 0.75 (0x600000); the
// floor of 114 is the 1e-4 clamp (ceil(log2 1e-4) = -13).
__device__ __forceinline__ int ue8m0_from_amax_bits(uint32_t b) {
  const int e = (int)(b >> 23) - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e > 114 ? e : 114;
}

// fp8 e4m3fn code of the bf16 value h scaled by 2^(127 - E).  The caller
// guarantees |h| * 2^(127-E) <= 448 and E >= 114 (the ue8m0 exponent of h's
// group), so there is no overflow and bf16 subnormals round to zero.
__device__ __forceinline__ uint32_t fp8_from_bf16(uint32_t h, int E) {
  const uint32_t sign = (h >> 8) & 0x80u;
  const int bexp = (int)((h >> 7) & 0xFFu);
  const uint32_t mant = h & 0x7Fu;
  const int fe = bexp - E + 7;             // e4m3 biased exponent when normal
  // normal: keep 3 of the 7 mantissa bits, nearest even; a carry bumps fe
  const uint32_t rn = (mant + 7u + ((mant >> 4) & 1u)) >> 4;
  const uint32_t normal = ((uint32_t)fe << 3) + rn;
  // subnormal (fe <= 0): (128 + mant) * 2^(fe - 5) units of 2^-9, nearest
  // even; shifts past 9 leave less than half a unit, as 9 does
  int sh = 5 - fe;
  sh = sh > 9 ? 9 : (sh < 1 ? 1 : sh);
  const uint32_t v = 128u + mant;
  const uint32_t q = v >> sh;
  const uint32_t rem = v & ((1u << sh) - 1u);
  const uint32_t half = 1u << (sh - 1);
  const uint32_t sub = q + ((rem > half) || (rem == half && (q & 1u)) ? 1u : 0u);
  uint32_t code = fe >= 1 ? normal : sub;
  code = bexp == 0 ? 0u : code;
  return code | sign;
}

// e4m3fn code of a non-negative finite fp32, nearest even, clamped at 448
// (0x7E).  Used for the FP4 group scale.
__device__ __forceinline__ uint32_t e4m3_satfinite(float f) {
  const uint32_t u = __float_as_uint(f);
  const int fe = (int)(u >> 23) - 120;
  const uint32_t m = u & 0x7FFFFFu;
  const uint32_t rn = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;
  uint32_t normal = ((uint32_t)fe << 3) + rn;
  normal = fe >= 16 ? 0x7Eu : (normal > 0x7Eu ? 0x7Eu : normal);
  const uint32_t sub = (uint32_t)__builtin_rintf(f * 512.0f);   // below 2^-6: k * 2^-9
  return fe >= 1 ? normal : sub;
}

// exact fp32 value of an e4m3fn code (NaN codes excluded by the caller)
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float sub = (float)m * 0x1p-9f;
  const float mag = e == 0 ? sub : nrm;
  return (c & 0x80u) ? -mag : mag;
}

// The value whose round-to-nearest-even e2m1 code (gfx950's
// v_cvt_scalef32_pk_fp4_f32 with a unit scale) is the code of the exact
// quotient x / s, given rs = rcp(s) (within an ulp of 1 / s).
//   The e2m1 ties (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) and grid values have
// at most 3 significant bits.  x has at most 8 and s at most 4, so an exact
// quotient that is not such a value lies at least ~2^-15 (relative) from
// every one of them, and the product x * rs -- within a few ulps of x / s --
// rounds to the same code.  An exact quotient that is such a value is
// recovered exactly by rounding x * rs to 3 significant bits when it lies
// within 4 ulps of one.  (Checked on the device against a threshold encoder
// for every finite bf16 x under every positive finite e4m3 s.)
__device__ __forceinline__ float fp4_quotient(float x, float rs) {
  const uint32_t u = __float_as_uint(x * rs);
  const uint32_t snap = (u + 0x00100000u) & 0xFFE00000u;   // nearest 3-significant-bit value
  return __uint_as_float(snap - u + 4u <= 8u ? snap : u);
}

}  // namespace kvc
