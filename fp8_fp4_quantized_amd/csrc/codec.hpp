// codec.hpp -- number-format conversions for the KV row codecs.
//
// Formats: bfloat16; OCP fp8 e4m3fn (bias 7, max 448, 0x7F/0xFF NaN);
// OCP fp4 e2m1 (values 0, .5, 1, 1.5, 2, 3, 4, 6); ue8m0 (a bare biased
// exponent).  Every encoder rounds to nearest, ties to even.  The ue8m0
// exponent and the bf16 amax are integer work on bit fields; the fp8 and
// e2m1 codes and the bf16 packing come from gfx950's conversion instructions
// (v_cvt_scalef32_pk_fp8_f32, v_cvt_scalef32_pk_fp4_f32, v_cvt_pk_bf16_f32),
// which round to nearest even whatever the shader's float mode.  Each
// hardware path was checked on the device against the format's definition
// over every input the quantizers can meet: fp8 codes for every finite bf16
// under every ue8m0 exponent in range, e2m1 codes for every finite bf16
// under every positive e4m3 scale, and the dequant conversions for every
// code under every scale byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950 (converting the halves one by one costs two
// conversions, a shift and an or)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_pk __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_pk));
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

// fp8 e4m3fn codes of four fp32 values scaled by 2^(127 - E), nearest even,
// packed into a dword (the first value in the low byte).  gfx950's
// v_cvt_scalef32_pk_fp8_f32 divides by the power of two whose biased exponent
// is the scale operand's exponent field -- E itself here.  For every finite
// bf16 x and every E in 114..254 with |x| * 2^(127 - E) <= 448 (the range the
// ue8m0 exponent of x's group guarantees) its code equals the
// nearest-even encoding, negative zero and subnormals included (checked
// exhaustively on the device against the definition).  With a unit scale it
// also gives the FP4 group scale's e4m3 code of any fp32 in [0, 448].
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fp8x4_scaled(float a, float b, float c, float d, int E) {
  const float sc = __uint_as_float((uint32_t)E << 23);
  s16x2 w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, sc, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, sc, true);
  return __builtin_bit_cast(uint32_t, w);
}

// Correctly rounded fp32 quotient x / s from rs, an fp32 within an ulp of
// 1 / s (the nearest fp32, or v_rcp_f32): q0 = x * rs, the residual
// x - q0 * s (exact in one fma) and one correction step.  Used for the FP4
// group scale amax / 6 (equal to the fp32 division for every finite bf16
// amax >= 0) and for the element quotients x / s of the
// e2m1 codes (equal for every finite bf16 x with |x| <= 8 s under every
// positive finite e4m3 s; the quantizer's quotients are at most about 6.4).
// Both were checked exhaustively on the device against the division.  The
// sign is copied from x so that -0 stays -0.
__device__ __forceinline__ float div_by_rcp(float x, float s, float rs) {
  const float q0 = x * rs;
  const float r = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, rs, q0), x);
}

}  // namespace kvc
