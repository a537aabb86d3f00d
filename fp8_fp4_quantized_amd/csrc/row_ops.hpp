// row_ops.hpp -- one row of 512 dims on one wavefront: quantize-and-store
// (the single row quantizer of sglang PR #39652, Summary) and the per-lane
// dequantizer of the gather.
//
// Lane l owns dims [8l, 8l + 8) as a uint4 of four packed bf16 pairs (the even
// dim in the low half).  Group maxima are DPP reductions over the 4 (V41),
// 2 (V41_FP4) or 8 (V4) lanes of a scale group.
#pragma once

#include "codec.hpp"
#include "layout.hpp"
#include "wave.hpp"

namespace kvc {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_u4(const void* p) {
  const u32x4 v = *(const u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_u4_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_u4(void* p, uint4 v) {
  *(u32x4*)p = u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void st_u4_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4*)p);
}

// A 16-byte streaming store at device scope: non-temporal with the sc1
// cache-policy bit, a policy only the buffer instructions take from the
// compiler.  For rows written once and not read back by the kernel; on the
// gather's 268 MB of output it measured 3-4% faster than non-temporal
// alone.  `base` must be the same on every lane (it becomes the buffer
// descriptor: raw, stride 0, 2^31 - 1 bytes, 32-bit data format), and
// byte_off below 2^31.
constexpr int kCpolNtSc1 = 2 | 16;          // nt | sc1
constexpr int kCpolSc1 = 16;                // sc1: device scope
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF,
                                           0x00020000);
}
__device__ __forceinline__ void st_u4_stream(void* base, uint32_t byte_off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, raw_rsrc(base),
                                         (int)byte_off, 0, kCpolNtSc1);
}

// Loads through a buffer descriptor made from a base that is the same on
// every lane, at a 32-bit byte offset below 2^31, at device scope (sc1):
// cached (CPOL = kCpolSc1), or non-temporal (kCpolNtSc1) for bytes read once
// and not wanted in the L2.
template <int CPOL>
__device__ __forceinline__ uint4 ld_u4_buf(const void* base, uint32_t byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(raw_rsrc(base), (int)byte_off, 0, CPOL);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int CPOL>
__device__ __forceinline__ uint2 ld_u2_buf(const void* base, uint32_t byte_off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(raw_rsrc(base), (int)byte_off, 0, CPOL);
  return make_uint2(v.x, v.y);
}
template <int CPOL>
__device__ __forceinline__ uint32_t ld_u32_buf(const void* base, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(raw_rsrc(base), (int)byte_off, 0, CPOL);
}
__device__ __forceinline__ uint32_t ld_u8_dev(const void* base, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b8(raw_rsrc(base), (int)byte_off, 0, kCpolSc1);
}

// Gather the scale byte held by lane `stride * g` (g = 0 .. 4*W-1) into W
// dwords, byte g of the result in byte g % 4 of dword g / 4.  Uses
// v_readlane, so the result is wave-uniform.
template <int W, int Stride>
__device__ __forceinline__ void collect_scale_bytes(uint32_t v, uint32_t (&out)[W]) {
#pragma unroll
  for (int d = 0; d < W; ++d) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, (4 * d + k) * Stride);
      w |= (b & 0xFFu) << (8 * k);
    }
    out[d] = w;
  }
}

// ------------------------------------------------------------------ store_row
// Quantize the row held by the wave (x = this lane's 8 dims): quantize_row
// computes this lane's code words and the packed scale bytes, with no memory
// access and no branch, so several rows' quantization can be scheduled
// together; store_quantized writes them to `data` / `scale` (the row's parts
// in its page).  Every lane of the wave must call both (the group
// reductions read neighbouring lanes); `write` is wave-uniform.
template <int L> struct RowQ;
template <> struct RowQ<kV41> { uint32_t w0, w1, sw; };
template <> struct RowQ<kV41Fp4> { uint32_t w, sw; };
template <> struct RowQ<kV4> { uint32_t w0, w1, sc0, sc1; };

template <int L>
__device__ __forceinline__ RowQ<L> quantize_row(uint4 x);

template <>
__device__ __forceinline__ RowQ<kV41> quantize_row<kV41>(uint4 x) {
  const uint32_t amax = group_max_u32<4>(absmax_bf16x8(x));     // 32 dims = 4 lanes
  const int E = ue8m0_from_amax_bits(amax << 16);
  RowQ<kV41> q;
  q.w0 = fp8x4_scaled(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y), E);
  q.w1 = fp8x4_scaled(bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w), E);
  // scale bytes: group g's E sits on lanes 4g..4g+3; lane 16k+12 packs the
  // bytes of groups 4k..4k+3
  q.sw = pack4_bytes_shr<4>((uint32_t)E);
  return q;
}

template <>
__device__ __forceinline__ RowQ<kV4> quantize_row<kV4>(uint4 x) {
  const uint32_t amax = group_max_u32<8>(absmax_bf16x8(x));     // 64 dims = 8 lanes
  const int E = ue8m0_from_amax_bits(amax << 16);
  RowQ<kV4> q;
  q.w0 = fp8x4_scaled(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y), E);
  q.w1 = fp8x4_scaled(bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w), E);
  uint32_t sc[2];
  collect_scale_bytes<2, 8>((uint32_t)E, sc);     // lanes 0, 8, .., 56; the 8th is rope
  q.sc0 = sc[0];
  q.sc1 = sc[1] & 0x00FFFFFFu;                    // pad byte = 0
  return q;
}

template <>
__device__ __forceinline__ RowQ<kV41Fp4> quantize_row<kV41Fp4>(uint4 x) {
  const uint32_t amax = group_max_u32<2>(absmax_bf16x8(x));     // 16 dims = 2 lanes
  // scale = e4m3(amax / 6): the fp32 quotient, correctly rounded, clamped at
  // 448 and rounded to e4m3 by the unit-scale fp8 conversion, then its exact
  // value back through the fp8 -> fp32 conversion
  const float qs = div_by_rcp(__uint_as_float(amax << 16), 6.0f, 0x1.555556p-3f);
  const float qc = fminf(qs, 448.0f);
  const s16x2 cw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, qc, qc, 1.0f, false);
  const uint32_t sc = (uint32_t)cw.x & 0xFFu;
  const float s = __builtin_amdgcn_cvt_scalef32_f32_fp8(sc, 1.0f, 0);
  const float rs = __builtin_amdgcn_rcpf(s);
  const float xf[8] = {bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y),
                       bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
  float qf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) qf[k] = div_by_rcp(xf[k], s, rs);
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, qf[0], qf[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, qf[2], qf[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, qf[4], qf[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, qf[6], qf[7], 1.0f, 3);
  RowQ<kV41Fp4> q;
  q.w = sc == 0 ? 0u : w;                          // zero scale: all codes 0
  // scale bytes: group g's code sits on lanes 2g, 2g+1; lane 8k+6 packs the
  // bytes of groups 4k..4k+3
  q.sw = pack4_bytes_shr<2>(sc);
  return q;
}

template <int L>
__device__ __forceinline__ void store_quantized(const RowQ<L>& q, uint4 x, uint8_t* data,
                                                uint8_t* scale, bool write);

template <>
__device__ __forceinline__ void store_quantized<kV41>(const RowQ<kV41>& q, uint4, uint8_t* data,
                                                      uint8_t* scale, bool write) {
  if (!write) return;
  const int lane = lane_id();
  *(u32x2*)(data + 8 * lane) = u32x2{q.w0, q.w1};
  if ((lane & 15) == 12) *(uint32_t*)(scale + 4 * (lane >> 4)) = q.sw;   // 4 lanes x 4 B
}

template <>
__device__ __forceinline__ void store_quantized<kV4>(const RowQ<kV4>& q, uint4 x, uint8_t* data,
                                                     uint8_t* scale, bool write) {
  if (!write) return;
  const int lane = lane_id();
  if (lane < kRopeLane0) {
    *(u32x2*)(data + 8 * lane) = u32x2{q.w0, q.w1};
  } else {                                         // rope dims kept as bf16
    st_u4(data + kNope + 16 * (lane - kRopeLane0), x);
  }
  if (lane == 0) *(u32x2*)scale = u32x2{q.sc0, q.sc1};
}

template <>
__device__ __forceinline__ void store_quantized<kV41Fp4>(const RowQ<kV41Fp4>& q, uint4,
                                                         uint8_t* data, uint8_t* scale,
                                                         bool write) {
  if (!write) return;
  const int lane = lane_id();
  *(uint32_t*)(data + 4 * lane) = q.w;
  if ((lane & 7) == 6) *(uint32_t*)(scale + 4 * (lane >> 3)) = q.sw;     // 8 lanes x 4 B
}

template <int L>
__device__ __forceinline__ void store_row_wave(uint4 x, uint8_t* data, uint8_t* scale, bool write) {
  store_quantized<L>(quantize_row<L>(x), x, data, scale, write);
}

// ------------------------------------------------------------------ exact RoPE
// fp64 -> bf16, nearest even, with bf16 subnormals and overflow to infinity;
// NaN gives 0x7FC0.  Two roundings that together make one: d to fp32 by
// round-to-odd (the hardware's nearest-even conversion, stepped back one
// pattern when it rounded away from zero, then the last bit set when
// inexact), then that fp32 to bf16 by nearest even on its bit pattern.  With
// 16 more significand bits than bf16, also in the subnormal range (quantum
// 2^-149 against 2^-133), the odd intermediate never creates a false tie, so
// the result is d rounded once (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", 2008).
// Needs fp32 denormals kept by the conversions (the kernels' float mode).
// Branch-free: every lane of a wave takes the same instructions.
__device__ __forceinline__ uint32_t bf16_from_f64(double d) {
  const float t = (float)d;                      // nearest even, may overflow to inf
  const double back = (double)t;
  uint32_t u = __float_as_uint(t);
  const bool inexact = back != d;
  u = inexact && __builtin_fabs(back) > __builtin_fabs(d) ? u - 1u : u;
  u = inexact ? (u | 1u) : u;
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return d != d ? 0x7FC0u : r;
}

// Rotate the row's 64 rope dims, (448 + 2j, 449 + 2j) by (cos, sin) =
// (fr[2j], fr[2j + 1]), spreading them one dim per lane: lane l pulls the
// bf16 pair of dim 448 + l from the rope lane that holds it, forms its
// rotated value in fp64 (the products of a bf16 and an fp32 value are exact
// there, so one rounding remains) and rounds it to bf16; the rope lanes then
// pull the rotated pairs back.  Every lane of the wave must call this; the
// nope lanes get x back.  f: lane k's table entry k of the row's position.
__device__ __forceinline__ uint4 rope_row_exact(uint4 x, float f) {
  const int lane = lane_id();
  const int pair = lane >> 1;
  const int src = kRopeLane0 + (pair >> 2);
  const uint32_t w0 = (uint32_t)__shfl((int)x.x, src), w1 = (uint32_t)__shfl((int)x.y, src);
  const uint32_t w2 = (uint32_t)__shfl((int)x.z, src), w3 = (uint32_t)__shfl((int)x.w, src);
  const bool k1 = (pair & 1) != 0, k2 = (pair & 2) != 0;   // word pair & 3 of the rope lane
  const uint32_t w = k2 ? (k1 ? w3 : w2) : (k1 ? w1 : w0);
  const float g = dpp_f32<kDppQuadXor1>(f);     // the other entry of the pair
  const bool odd = (lane & 1) != 0;
  const double a = (double)bf16_lo(w), b = (double)bf16_hi(w);
  const double c = (double)(odd ? g : f), s = (double)(odd ? f : g);
  const double o = odd ? a * s + b * c : a * c - b * s;
  const uint32_t h = bf16_from_f64(o);
  const uint32_t word = h | (dpp_u32<kDppQuadXor1>(h) << 16);   // even lanes: dims l, l + 1
  const int base = 8 * (lane - kRopeLane0);
  const uint32_t r0 = (uint32_t)__shfl((int)word, base), r1 = (uint32_t)__shfl((int)word, base + 2);
  const uint32_t r2 = (uint32_t)__shfl((int)word, base + 4), r3 = (uint32_t)__shfl((int)word, base + 6);
  return lane >= kRopeLane0 ? make_uint4(r0, r1, r2, r3) : x;
}

// ------------------------------------------------------------------ dequant
// 8 fp8 codes + their ue8m0 exponent E -> 8 bf16.  gfx950's scaled
// conversion v_cvt_scalef32_pk_bf16_fp8 multiplies two e4m3fn codes by the
// power of two whose biased exponent is the fp32 scale's exponent field -- E
// itself here -- so it computes fp8 * 2^(E - 127) rounded to bf16, with NaN
// for NaN codes and for E = 255.  The products are exact in bf16 for E >= 3;
// the device tests compare it with the oracle for every code under every E.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 dq_fp8x8(uint2 codes, uint32_t E) {
  const float sc = __uint_as_float(E << 23);
  const bf16x2_hw a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, sc, false);
  const bf16x2_hw b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, sc, true);
  const bf16x2_hw c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, sc, false);
  const bf16x2_hw d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, sc, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// 8 e2m1 codes (nibbles, dim order from the low nibble) + their e4m3 scale
// code -> 8 bf16.  The hardware converts the scale code and a byte's two
// codes to fp32 (the codes at unit scale); the product is exact in fp32 (at
// most 7 significant bits, far from the fp32 and bf16 limits), so its top
// half is the bf16.  A NaN scale code makes every product a quiet NaN, whose
// top half is a bf16 NaN.
__device__ __forceinline__ uint4 dq_fp4x8(uint32_t w, uint32_t sc) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
  auto pair = [&](f32x2 f) -> uint32_t {
    // bytes 2, 3 of the first product, then bytes 2, 3 of the second
    return __builtin_amdgcn_perm(__float_as_uint(f[1] * s), __float_as_uint(f[0] * s),
                                 0x07060302u);
  };
  return make_uint4(pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)),
                    pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)),
                    pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)),
                    pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3)));
}

}  // namespace kvc
