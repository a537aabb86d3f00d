// ceiling.hip -- streaming kernels that move a headline kernel's bytes with
// no work attached, the yardstick the benchmark sets each kernel against
// (libkvc_ceiling.so, include/kvc_ceiling.h).  They are measurement aids, not
// part of the compressed-KV path.
//
//  - compress shape: per item, 8 KB read contiguously (two row pairs of a
//    fused |kv|score| buffer), then 2 KB (two latent rows), 512 B (two FP4
//    data parts) and 64 B (their scale parts) written contiguously -- the
//    bytes the ratio-2 compressor moves for two rows into a V41_FP4 cache;
//  - gather shape: per row, 528 B read (a V41 row's data and scale parts,
//    rows contiguous) and 1024 B written (its bf16 row).
// Loads are non-temporal and the large stores are non-temporal, the policies
// of the kernels they stand beside.  Each wave issues every load of its item
// (or of 8 rows) before it stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvc_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void compress_shape_kernel(const u32x4* __restrict__ src,
                                                                u32x4* __restrict__ lat,
                                                                uint32_t* __restrict__ data,
                                                                uint32_t* __restrict__ scale,
                                                                int64_t items) {
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (kBlock / 64);
  for (int64_t it = w0; it < items; it += nw) {
    u32x4 v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = __builtin_nontemporal_load(src + it * 512 + r * 64 + lane);
    u32x4 a = v[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) a ^= v[r];
    __builtin_nontemporal_store(a, lat + it * 128 + lane);
    __builtin_nontemporal_store(a + 1u, lat + it * 128 + 64 + lane);
    data[it * 128 + lane] = a.x;
    data[it * 128 + 64 + lane] = a.y;
    if (lane < 16) scale[it * 16 + lane] = a.z;
  }
}

constexpr int kRowsPerTrip = 8;

__global__ __launch_bounds__(kBlock) void gather_shape_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ out,
                                                              int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (kBlock / 64);
  // a 528-byte row is 33 16-byte units: lane l < 33 reads unit l
  const int u = lane < 33 ? lane : 32;
  for (int64_t r0 = w0 * kRowsPerTrip; r0 < rows; r0 += nw * kRowsPerTrip) {
    u32x4 v[kRowsPerTrip];
#pragma unroll
    for (int k = 0; k < kRowsPerTrip; ++k) {
      const int64_t r = r0 + k < rows ? r0 + k : rows - 1;
      v[k] = __builtin_nontemporal_load(src + r * 33 + u);
    }
#pragma unroll
    for (int k = 0; k < kRowsPerTrip; ++k) {
      if (r0 + k < rows) __builtin_nontemporal_store(v[k] ^ (uint32_t)lane, out + (r0 + k) * 64 + lane);
    }
  }
}

int grid(int64_t units, int64_t per_block, int cap) {
  int64_t b = (units + per_block - 1) / per_block;
  return (int)(b < 1 ? 1 : (b > cap ? cap : b));
}

}  // namespace

extern "C" {

int kvc_ceiling_compress_shape(const void* src, void* latent, void* data, void* scale,
                               int64_t items, void* stream) {
  if (items < 0 || (items > 0 && (!src || !latent || !data || !scale))) return -1;
  if (items == 0) return 0;
  // the compressor's grid: 1024 workgroups of 4 waves, two items per wave
  hipLaunchKernelGGL(compress_shape_kernel, dim3(grid(items, 4, 1024)), dim3(kBlock), 0,
                     (hipStream_t)stream, (const u32x4*)src, (u32x4*)latent, (uint32_t*)data,
                     (uint32_t*)scale, items);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int kvc_ceiling_gather_shape(const void* src, void* out, int64_t rows, void* stream) {
  if (rows < 0 || (rows > 0 && (!src || !out))) return -1;
  if (rows == 0) return 0;
  hipLaunchKernelGGL(gather_shape_kernel, dim3(grid(rows, 4 * kRowsPerTrip, 8192)), dim3(kBlock), 0,
                     (hipStream_t)stream, (const u32x4*)src, (u32x4*)out, rows);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
