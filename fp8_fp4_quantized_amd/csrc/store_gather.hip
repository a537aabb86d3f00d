// store_gather.hip -- plain quantize-store of bf16 rows and the paged
// dequant-gather (gfx950).
//
// Both kernels put one 512-dim row on one 64-lane wave (8 dims per lane), so
// every global access of a row is one contiguous, fully used span: the bf16
// row (1024 B), the data part (512 / 256 / 576 B) and the scale part.  A wave
// runs several rows per loop trip so that their loads are in flight
// together; the grid strides over the rows.
#include "launch.hpp"
#include "row_ops.hpp"

namespace kvc {

namespace {

constexpr int kBlock = 256;                 // 4 waves
constexpr int kWavesPerBlock = kBlock / kLanes;

template <int L>
__device__ __forceinline__ PagedKV<L> paged(const CacheView& c) {
  return PagedKV<L>{c.base, c.page_stride, c.num_pages, c.page_bits};
}

__device__ __forceinline__ void raise_status(int32_t* status, int32_t bit) {
  if (status != nullptr && lane_id() == 0) atomicOr(status, bit);
}

// ------------------------------------------------------------------ store
// ROPE: rotate the rope dims at positions[i] first (exact, one rounding).
template <int L, bool ROPE>
__global__ __launch_bounds__(kBlock) void store_rows_kernel(StoreParams p) {
  const PagedKV<L> kv = paged<L>(p.cache);
  const int lane = lane_id();
  const int64_t wave0 = uniform64((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t i = wave0; i < p.n; i += nwaves) {
    uint4 x = ld_u4_nt(p.rows + i * p.row_stride + kDimsPerLane * lane);
    const int64_t loc = uniform(p.out_loc[i]);
    bool write = loc != 0;
    if constexpr (ROPE) {
      if (write) {
        const int64_t pos = ld_ro(p.positions + i);
        if (pos < 0 || pos >= p.max_pos) {
          raise_status(p.status, kStPosRange);
          write = false;
        } else {
          x = rope_row_exact(x, p.freqs + pos * kRope);
        }
      }
    }
    if (write && !kv.valid(loc)) {
      raise_status(p.status, kStPageRange);
      write = false;
    }
    const int64_t slot = write ? loc : 0;
    store_row_wave<L>(x, kv.data(slot), kv.scale(slot), write);
  }
}

// ------------------------------------------------------------------ DCP ids
// One wave per row of ids, 64 ids per step: each lane tests its id for
// ownership and maps it to a slot, a ballot and a lane count give every kept
// id its place after the ones before it, and the row is finished with -1.
__global__ __launch_bounds__(kBlock) void dcp_filter_kernel(DcpFilterParams p) {
  const int lane = lane_id();
  const int64_t wave0 = uniform64((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int kl = p.interleave_log2;
  const uint32_t kmask = (1u << kl) - 1, pmask = (1u << p.page_bits) - 1;
  const uint32_t world = (uint32_t)p.world, rank = (uint32_t)p.rank;
  for (int64_t t = wave0; t < p.T; t += nwaves) {
    int32_t cnt = 0;
    bool keep = p.valid == nullptr || ld_ro(p.valid + t) != 0;
    const int32_t req = ld_ro(p.token_to_req + t);
    if (keep && (req < 0 || req >= p.n_req)) {
      raise_status(p.status, kStReqRange);
      keep = false;
    }
    int32_t* out = p.out_slots + t * p.out_stride;
    if (keep) {
      const int32_t* row = p.ids + t * p.ids_stride;
      const int32_t* bt = p.block_table + (int64_t)req * p.bt_stride;
      for (int32_t i0 = 0; i0 < p.k; i0 += kLanes) {
        const int32_t i = i0 + lane;
        int32_t slot = -1, bad = 0;
        const int32_t id = i < p.k ? row[i] : -1;
        if (id >= 0) {
          const uint32_t run = (uint32_t)id >> kl;
          const uint32_t turn = run / world;
          if (run - turn * world == rank) {
            const uint32_t u = (turn << kl) | ((uint32_t)id & kmask);
            const int64_t lp = u >> p.page_bits;
            if (lp >= p.bt_stride) {
              bad = kStPtRange;
            } else {
              const int32_t phys = bt[lp];
              if (phys < 0 || phys >= p.num_pages) {
                bad = kStPageRange;
              } else {
                slot = (phys << p.page_bits) | (int32_t)(u & pmask);
              }
            }
          }
        }
        if (bad != 0 && p.status != nullptr) atomicOr(p.status, bad);
        const uint64_t m = __ballot(slot >= 0);
        const int32_t before = (int32_t)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (slot >= 0) out[cnt + before] = slot;
        cnt += (int32_t)__builtin_popcountll(m);
      }
    }
    for (int32_t i = cnt + lane; i < p.k; i += kLanes) out[i] = -1;
    if (lane == 0) p.out_lens[t] = cnt;
  }
}

// ------------------------------------------------------------------ gather
// rows handled together by one wave per loop trip
constexpr int kGatherUnroll = 8;

template <int L> struct LaneCodes;          // this lane's share of a row
template <> struct LaneCodes<kV41> { uint2 codes; uint32_t scale; };
template <> struct LaneCodes<kV41Fp4> { uint32_t codes; uint32_t scale; };
template <> struct LaneCodes<kV4> { uint4 raw; uint32_t scale; };

template <int L>
__device__ __forceinline__ LaneCodes<L> load_lane(const PagedKV<L>& kv, int64_t slot, int lane);

template <>
__device__ __forceinline__ LaneCodes<kV41> load_lane<kV41>(const PagedKV<kV41>& kv, int64_t slot,
                                                           int lane) {
  LaneCodes<kV41> r;
  const u32x2 c = __builtin_nontemporal_load((const u32x2*)(kv.data(slot) + 8 * lane));
  r.codes = make_uint2(c.x, c.y);
  r.scale = __builtin_nontemporal_load(kv.scale(slot) + (lane >> 2));
  return r;
}
template <>
__device__ __forceinline__ LaneCodes<kV41Fp4> load_lane<kV41Fp4>(const PagedKV<kV41Fp4>& kv,
                                                                 int64_t slot, int lane) {
  LaneCodes<kV41Fp4> r;
  r.codes = __builtin_nontemporal_load((const uint32_t*)(kv.data(slot) + 4 * lane));
  r.scale = __builtin_nontemporal_load(kv.scale(slot) + (lane >> 1));
  return r;
}
template <>
__device__ __forceinline__ LaneCodes<kV4> load_lane<kV4>(const PagedKV<kV4>& kv, int64_t slot,
                                                         int lane) {
  LaneCodes<kV4> r;
  const uint8_t* d = kv.data(slot);
  if (lane < kRopeLane0) {
    const u32x2 c = __builtin_nontemporal_load((const u32x2*)(d + 8 * lane));
    r.raw = make_uint4(c.x, c.y, 0u, 0u);
    r.scale = __builtin_nontemporal_load(kv.scale(slot) + (lane >> 3));
  } else {
    r.raw = ld_u4_nt(d + kNope + 16 * (lane - kRopeLane0));
    r.scale = 0;
  }
  return r;
}

template <int L>
__device__ __forceinline__ uint4 decode_lane(const LaneCodes<L>& c, int lane);
template <>
__device__ __forceinline__ uint4 decode_lane<kV41>(const LaneCodes<kV41>& c, int) {
  return dq_fp8x8(c.codes, c.scale);
}
template <>
__device__ __forceinline__ uint4 decode_lane<kV41Fp4>(const LaneCodes<kV41Fp4>& c, int) {
  return dq_fp4x8(c.codes, c.scale);
}
template <>
__device__ __forceinline__ uint4 decode_lane<kV4>(const LaneCodes<kV4>& c, int lane) {
  if (lane >= kRopeLane0) return c.raw;
  return dq_fp8x8(make_uint2(c.raw.x, c.raw.y), c.scale);
}

// A wave takes the rows of the gather 64 at a time: lane i reads id i of the
// batch and resolves it to a physical slot (one vector load of ids, one of
// page-table entries), then the rows are expanded kGatherUnroll at a time,
// their slots broadcast with v_readlane, all their loads issued before any
// store.
template <int L>
__global__ __launch_bounds__(kBlock) void dequant_gather_kernel(GatherParams p) {
  const PagedKV<L> kv = paged<L>(p.cache);
  const int lane = lane_id();
  const int64_t wave0 = uniform64((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int32_t page_mask = (1 << p.cache.page_bits) - 1;

  for (int64_t b0 = wave0 * kLanes; b0 < p.n; b0 += nwaves * kLanes) {
    // ---- resolve this lane's id to a slot (-1: zero row)
    const int64_t r = b0 + lane;
    int32_t slot = -1;
    int32_t bad = 0;
    if (r < p.n) {
      const int32_t id = p.ids[r];
      if (id >= 0) {
        if (p.page_table != nullptr) {
          const int32_t lp = id >> p.cache.page_bits;
          if (lp < p.n_pages) {
            const int32_t phys = p.page_table[lp];
            if (phys >= 0 && phys < kv.num_pages) {
              slot = (phys << p.cache.page_bits) | (id & page_mask);
            } else {
              bad = kStPageRange;
            }
          } else {
            bad = kStIdRange;
          }
        } else if (kv.valid(id)) {
          slot = id;
        } else {
          bad = kStIdRange;
        }
      }
    }
    if (bad != 0 && p.status != nullptr) atomicOr(p.status, bad);

    // ---- expand the batch's rows
    const int cnt = (int)(p.n - b0 < kLanes ? p.n - b0 : kLanes);
    for (int j = 0; j < cnt; j += kGatherUnroll) {
      int32_t s[kGatherUnroll];
      LaneCodes<L> c[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        s[u] = j + u < cnt ? __builtin_amdgcn_readlane(slot, j + u) : -1;
        if (s[u] >= 0) c[u] = load_lane<L>(kv, s[u], lane);
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        if (j + u >= cnt) break;
        const uint4 o = s[u] >= 0 ? decode_lane<L>(c[u], lane) : make_uint4(0u, 0u, 0u, 0u);
        st_u4_nt(p.out + (b0 + j + u) * p.out_stride + kDimsPerLane * lane, o);
      }
    }
  }
}

template <typename K, typename P>
hipError_t launch(K kernel, int blocks, const P& p, hipStream_t stream) {
  hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

int grid_for(int64_t units, int64_t per_block, int cap) {
  int64_t b = (units + per_block - 1) / per_block;
  if (b > cap) b = cap;
  return (int)(b < 1 ? 1 : b);
}

}  // namespace

LaunchTuning& launch_tuning() {
  static LaunchTuning t{0, 0, -1};
  return t;
}

hipError_t launch_store_rows(const StoreParams& p, hipStream_t stream) {
  const int blocks = grid_for(p.n, kWavesPerBlock, 8192);
  const bool rope = p.positions != nullptr;
  switch (p.cache.layout) {
    case kV41:
      return rope ? launch(store_rows_kernel<kV41, true>, blocks, p, stream)
                  : launch(store_rows_kernel<kV41, false>, blocks, p, stream);
    case kV41Fp4:
      return rope ? launch(store_rows_kernel<kV41Fp4, true>, blocks, p, stream)
                  : launch(store_rows_kernel<kV41Fp4, false>, blocks, p, stream);
    default:
      return rope ? launch(store_rows_kernel<kV4, true>, blocks, p, stream)
                  : launch(store_rows_kernel<kV4, false>, blocks, p, stream);
  }
}

hipError_t launch_dcp_filter(const DcpFilterParams& p, hipStream_t stream) {
  return launch(dcp_filter_kernel, grid_for(p.T, kWavesPerBlock, 4096), p, stream);
}

hipError_t launch_dequant_gather(const GatherParams& p, hipStream_t stream) {
  int blocks = grid_for(p.n, (int64_t)kWavesPerBlock * kLanes, 2048);
  if (launch_tuning().gather_blocks > 0) blocks = launch_tuning().gather_blocks;
  switch (p.cache.layout) {
    case kV41: return launch(dequant_gather_kernel<kV41>, blocks, p, stream);
    case kV41Fp4: return launch(dequant_gather_kernel<kV41Fp4>, blocks, p, stream);
    default: return launch(dequant_gather_kernel<kV4>, blocks, p, stream);
  }
}

}  // namespace kvc
