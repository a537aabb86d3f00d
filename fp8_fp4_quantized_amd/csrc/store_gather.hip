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
// A wave stores kStoreRows rows per loop trip: the loads of all of them (row
// bytes, destination, position) are issued before the first is quantized, so
// a wave keeps 4 KiB of reads in flight.  Rows past n reload row n - 1 (a
// fixed count of loads keeps the compiler's waits exact) and store nothing.
// ROPE: rotate the rope dims at positions[i] first (exact, one rounding).
constexpr int kStoreRows = 4;

template <int L, bool ROPE>
__global__ __launch_bounds__(kBlock) void store_rows_kernel(StoreParams p) {
  const PagedKV<L> kv = paged<L>(p.cache);
  const int lane = lane_id();
  const int64_t wave0 = uniform64((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t i0 = wave0 * kStoreRows; i0 < p.n; i0 += nwaves * kStoreRows) {
    uint4 x[kStoreRows];
    int64_t loc[kStoreRows], pos[kStoreRows];
#pragma unroll
    for (int u = 0; u < kStoreRows; ++u) {
      const int64_t i = i0 + u < p.n ? i0 + u : p.n - 1;
      x[u] = ld_u4_nt(p.rows + i * p.row_stride + kDimsPerLane * lane);
      loc[u] = ld_ro(p.out_loc + i);
      pos[u] = ROPE ? ld_ro(p.positions + i) : 0;
    }
#pragma unroll
    for (int u = 0; u < kStoreRows; ++u) {
      if (i0 + u >= p.n) break;
      bool write = loc[u] != 0;
      if constexpr (ROPE) {
        if (write) {
          if (pos[u] < 0 || pos[u] >= p.max_pos) {
            raise_status(p.status, kStPosRange);
            write = false;
          } else {
            x[u] = rope_row_exact(x[u], p.freqs + pos[u] * kRope);
          }
        }
      }
      if (write && !kv.valid(loc[u])) {
        raise_status(p.status, kStPageRange);
        write = false;
      }
      const int64_t slot = write ? loc[u] : 0;
      store_row_wave<L>(x[u], kv.data(slot), kv.scale(slot), write);
    }
  }
}

// ------------------------------------------------------------------ DCP ids
// One workgroup per row of ids, kFilterPerLane consecutive ids per lane
// (2048 ids per pass): every lane tests its ids for ownership and looks up
// their pages (all loads in flight together), the workgroup scans the lanes'
// kept counts (shuffles within a wave, LDS across the four waves),
// and each lane writes its kept slots at its offset; the row ends in -1.
constexpr int kFilterPerLane = 8;
constexpr int kFilterPass = kBlock * kFilterPerLane;

__global__ __launch_bounds__(kBlock) void dcp_filter_kernel(DcpFilterParams p) {
  __shared__ int32_t wave_cnt[kWavesPerBlock];
  const int lane = lane_id(), wid = threadIdx.x >> 6;
  const int kl = p.interleave_log2;
  const uint32_t kmask = (1u << kl) - 1, pmask = (1u << p.page_bits) - 1;
  const uint32_t world = (uint32_t)p.world, rank = (uint32_t)p.rank;
  for (int64_t t = blockIdx.x; t < p.T; t += gridDim.x) {
    bool keep = p.valid == nullptr || ld_ro(p.valid + t) != 0;
    const int32_t req = ld_ro(p.token_to_req + t);
    if (keep && (req < 0 || req >= p.n_req)) {
      if (threadIdx.x == 0 && p.status != nullptr) atomicOr(p.status, kStReqRange);
      keep = false;
    }
    int32_t* out = p.out_slots + t * p.out_stride;
    int32_t cnt = 0;                                   // kept so far (workgroup-uniform)
    if (keep) {
      const int32_t* row = p.ids + t * p.ids_stride;
      const int32_t* bt = p.block_table + (int64_t)req * p.bt_stride;
      for (int32_t s0 = 0; s0 < p.k; s0 += kFilterPass) {
        const int32_t base = s0 + (int32_t)threadIdx.x * kFilterPerLane;
        int32_t id[kFilterPerLane], lp[kFilterPerLane], u[kFilterPerLane], pg[kFilterPerLane];
#pragma unroll
        for (int e = 0; e < kFilterPerLane; ++e) {
          const int32_t i = base + e;
          const int32_t v = row[i < p.k ? i : p.k - 1];
          id[e] = i < p.k ? v : -1;
        }
        // ownership and the page-table entry to read (entry 0 when unused)
#pragma unroll
        for (int e = 0; e < kFilterPerLane; ++e) {
          lp[e] = -1;
          u[e] = 0;
          if (id[e] >= 0) {
            const uint32_t run = (uint32_t)id[e] >> kl;
            const uint32_t turn = run / world;
            if (run - turn * world == rank) {
              u[e] = (int32_t)((turn << kl) | ((uint32_t)id[e] & kmask));
              lp[e] = u[e] >> p.page_bits;
            }
          }
        }
#pragma unroll
        for (int e = 0; e < kFilterPerLane; ++e) pg[e] = bt[lp[e] >= 0 && lp[e] < p.bt_stride ? lp[e] : 0];
        int32_t slot[kFilterPerLane], n = 0, bad = 0;
#pragma unroll
        for (int e = 0; e < kFilterPerLane; ++e) {
          slot[e] = -1;
          if (lp[e] >= 0) {
            if (lp[e] >= p.bt_stride) {
              bad |= kStPtRange;
            } else if (pg[e] < 0 || pg[e] >= p.num_pages) {
              bad |= kStPageRange;
            } else {
              slot[e] = (pg[e] << p.page_bits) | (int32_t)((uint32_t)u[e] & pmask);
              ++n;
            }
          }
        }
        if (bad != 0 && p.status != nullptr) atomicOr(p.status, bad);
        // exclusive offset of this lane's kept ids within the pass
        int32_t inc = n;
#pragma unroll
        for (int d = 1; d < kLanes; d <<= 1) {
          const int32_t v = __shfl_up(inc, d);
          if (lane >= d) inc += v;
        }
        if (lane == kLanes - 1) wave_cnt[wid] = inc;
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
          const int32_t c = wave_cnt[w];
          before += w < wid ? c : 0;
          total += c;
        }
        int32_t o = cnt + before + inc - n;
#pragma unroll
        for (int e = 0; e < kFilterPerLane; ++e) {
          if (slot[e] >= 0) out[o++] = slot[e];
        }
        cnt += total;
        __syncthreads();                                 // wave_cnt is reused
      }
    }
    for (int32_t i = cnt + (int32_t)threadIdx.x; i < p.k; i += kBlock) out[i] = -1;
    if (threadIdx.x == 0) p.out_lens[t] = cnt;
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
  const int blocks = grid_for(p.n, (int64_t)kWavesPerBlock * kStoreRows, 8192);
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
  return launch(dcp_filter_kernel, grid_for(p.T, 1, 16384), p, stream);
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
