// layout.hpp -- paged main-KV layouts and their address arithmetic (gfx950).
//
// The three KVLayout formats of sglang PR #39652 "dsv4.1: compression, KV
// I/O, and metadata kernels" (Summary), per 512-dim row:
//   V4       576 B data (448 fp8 nope codes + 64 bf16 rope dims) + 8 B scale
//            (7 ue8m0 bytes, one per 64 nope dims, + 1 zero pad)   = 584 B
//   V41      512 B data (fp8 codes) + 16 B scale (ue8m0 per 32)    = 528 B
//   V41_FP4  256 B data (e2m1, dim 2k in the low nibble of byte k)
//            + 32 B scale (e4m3 per 16)                            = 288 B
// Within a page the data parts of all rows come first, then the scale parts,
// so every data part starts on a 16-byte boundary (V4's 584-byte rows would
// not if rows were packed whole).  One address function serves every kernel,
// as PagedKV<layout, page_bits>::row does on that page.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int kDim = 512;               // latent dims per row
constexpr int kRope = 64;               // rotary dims (the last 64)
constexpr int kNope = kDim - kRope;     // 448
constexpr int kLanes = 64;              // wavefront width on CDNA4
constexpr int kDimsPerLane = kDim / kLanes;   // 8: lane l owns dims [8l, 8l+8)
constexpr int kRopeLane0 = kNope / kDimsPerLane;  // 56: lanes 56..63 hold the rope dims

enum Layout : int { kV4 = 0, kV41 = 1, kV41Fp4 = 2 };

template <int L> struct LayoutTraits;
template <> struct LayoutTraits<kV4> {
  static constexpr int kData = kNope + 2 * kRope;      // 576
  static constexpr int kScale = kNope / 64 + 1;        // 8
  static constexpr int kGroup = 64;
  static constexpr int kQuantDims = kNope;
};
template <> struct LayoutTraits<kV41> {
  static constexpr int kData = kDim;                   // 512
  static constexpr int kScale = kDim / 32;             // 16
  static constexpr int kGroup = 32;
  static constexpr int kQuantDims = kDim;
};
template <> struct LayoutTraits<kV41Fp4> {
  static constexpr int kData = kDim / 2;               // 256
  static constexpr int kScale = kDim / 16;             // 32
  static constexpr int kGroup = 16;
  static constexpr int kQuantDims = kDim;
};

static_assert(LayoutTraits<kV4>::kData + LayoutTraits<kV4>::kScale == 584, "V4 row");
static_assert(LayoutTraits<kV41>::kData + LayoutTraits<kV41>::kScale == 528, "V41 row");
static_assert(LayoutTraits<kV41Fp4>::kData + LayoutTraits<kV41Fp4>::kScale == 288, "FP4 row");

// Device view of one paged cache.  page_size = 1 << page_bits.
template <int L>
struct PagedKV {
  uint8_t* base;
  int64_t page_stride;
  int64_t num_pages;
  int32_t page_bits;

  __device__ __forceinline__ bool valid(int64_t slot) const {
    return slot >= 0 && (slot >> page_bits) < num_pages;
  }
  __device__ __forceinline__ uint8_t* data(int64_t slot) const {
    const int64_t page = slot >> page_bits, r = slot & ((int64_t(1) << page_bits) - 1);
    return base + page * page_stride + r * LayoutTraits<L>::kData;
  }
  __device__ __forceinline__ uint8_t* scale(int64_t slot) const {
    const int64_t page = slot >> page_bits, r = slot & ((int64_t(1) << page_bits) - 1);
    return base + page * page_stride + (LayoutTraits<L>::kData << page_bits) +
           r * LayoutTraits<L>::kScale;
  }
};

// Status bits a kernel may OR into the caller's status word.
enum : int32_t {
  kStIdRange = 1,
  kStPageRange = 2,
  kStPtRange = 4,
  kStLatentRange = 8,
  kStPosRange = 16,
  kStReqRange = 32,
  kStTokenRange = 64,
};

}  // namespace kvc
