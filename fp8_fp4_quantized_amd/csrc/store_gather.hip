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
    float fr[kStoreRows];
#pragma unroll
    for (int u = 0; u < kStoreRows; ++u) {
      const int64_t i = i0 + u < p.n ? i0 + u : p.n - 1;
      x[u] = ld_u4_nt(p.rows + i * p.row_stride + kDimsPerLane * lane);
      loc[u] = ld_ro(p.out_loc + i);
      pos[u] = ROPE ? ld_ro(p.positions + i) : 0;
    }
    if constexpr (ROPE) {
      // every row's table line is requested before the first row is rotated
      // (a position outside the table reads line 0 and is not used)
#pragma unroll
      for (int u = 0; u < kStoreRows; ++u) {
        const int64_t q = pos[u] >= 0 && pos[u] < p.max_pos ? pos[u] : 0;
        fr[u] = p.freqs[q * kRope + lane];
      }
    }
#pragma unroll
    for (int u = 0; u < kStoreRows; ++u) {
      if (i0 + u >= p.n) break;
      bool write = loc[u] != 0;
      if constexpr (ROPE) {
        // rotated whatever the row (a row with no valid position is not
        // stored), so the table loads above stay ahead of every row
        x[u] = rope_row_exact(x[u], fr[u]);
        if (write && (pos[u] < 0 || pos[u] >= p.max_pos)) {
          raise_status(p.status, kStPosRange);
          write = false;
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
// Persistent workgroups walk work units of 2048 ids (a row of k ids is
// ceil(k / 2048) units, taken in order by one workgroup).  Wave w of a
// workgroup takes ids [512 w, 512 w + 512) of the unit, 64 consecutive ids
// per load so every load is one contiguous 256 B.  An id's place among the
// kept ones is its lane count in the chunk's ballot, plus the chunks before
// it in the wave, plus the earlier waves (through LDS), plus the row's
// earlier units.  The ids of the next unit are loaded before the current one
// is processed, so their latency overlaps its page-table reads and stores.
constexpr int kFilterChunks = 8;                          // 64-id loads per lane
constexpr int kFilterUnit = kBlock * kFilterChunks;       // 2048 ids

struct FilterUnit {
  int32_t v[kFilterChunks];   // this lane's ids (-1 past the row)
  int32_t req;                // the row's request
  bool valid;                 // the row is not a padding token
};

// the ids and row data of work unit u, loaded ahead of their use
__device__ __forceinline__ FilterUnit load_unit(const DcpFilterParams& p, int64_t u,
                                                int32_t units_per_row, int wid, int lane) {
  FilterUnit r;
  const int64_t t = u / units_per_row;
  const int32_t s0 = (int32_t)(u - t * units_per_row) * kFilterUnit;
  r.valid = p.valid == nullptr || ld_ro(p.valid + t) != 0;
  r.req = ld_ro(p.token_to_req + t);
  if (p.k == 0) {                                         // no ids: nothing to read
#pragma unroll
    for (int e = 0; e < kFilterChunks; ++e) r.v[e] = -1;
    return r;
  }
  const int32_t* row = p.ids + t * p.ids_stride;
#pragma unroll
  for (int e = 0; e < kFilterChunks; ++e) {
    const int32_t i = s0 + kLanes * (kFilterChunks * wid + e) + lane;
    const int32_t v = __builtin_nontemporal_load(row + (i < p.k ? i : p.k - 1));
    r.v[e] = i < p.k ? v : -1;
  }
  return r;
}

__global__ __launch_bounds__(kBlock) void dcp_filter_kernel(DcpFilterParams p) {
  __shared__ int32_t wave_cnt[2][kWavesPerBlock];
  const int lane = lane_id(), wid = threadIdx.x >> 6;
  const int kl = p.interleave_log2;
  const uint32_t kmask = (1u << kl) - 1, pmask = (1u << p.page_bits) - 1;
  const uint32_t world = (uint32_t)p.world, rank = (uint32_t)p.rank;
  const int32_t units_per_row = p.k > 0 ? (p.k + kFilterUnit - 1) / kFilterUnit : 1;
  const int64_t n_units = p.T * units_per_row;
  int64_t u = blockIdx.x;
  if (u >= n_units) return;
  FilterUnit cur = load_unit(p, u, units_per_row, wid, lane);
  int32_t cnt = 0;                                    // kept so far in the row
  int parity = 0;                                     // LDS buffer of the next scan
  for (; u < n_units; u += gridDim.x) {
    const int64_t t = u / units_per_row;
    const int32_t part = (int32_t)(u - t * units_per_row);
    const int64_t un = u + gridDim.x;                 // next unit: its loads in flight now
    // past the last unit: re-read unit 0, which every workgroup shares in L2
    const FilterUnit nxt = load_unit(p, un < n_units ? un : 0, units_per_row, wid, lane);
    if (part == 0) cnt = 0;
    const int32_t req = cur.req;
    bool keep = cur.valid;
    if (keep && (req < 0 || req >= p.n_req)) {
      if (part == 0 && threadIdx.x == 0 && p.status != nullptr) atomicOr(p.status, kStReqRange);
      keep = false;
    }
    int32_t* out = p.out_slots + t * p.out_stride;
    if (keep && p.k > 0) {
      const int32_t* bt = p.block_table + (int64_t)req * p.bt_stride;
      int32_t lp[kFilterChunks], uo[kFilterChunks], pg[kFilterChunks];
#pragma unroll
      for (int e = 0; e < kFilterChunks; ++e) {
        const int32_t id = cur.v[e];
        lp[e] = -1;
        uo[e] = 0;
        if (id >= 0) {
          const uint32_t run = (uint32_t)id >> kl;
          const uint32_t turn = udiv_magic(run, p.world_div.m, p.world_div.sh1, p.world_div.sh2);
          if (run - turn * world == rank) {
            uo[e] = (int32_t)((turn << kl) | ((uint32_t)id & kmask));
            lp[e] = uo[e] >> p.page_bits;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < kFilterChunks; ++e)
        pg[e] = bt[lp[e] >= 0 && lp[e] < p.bt_stride ? lp[e] : 0];
      int32_t slot[kFilterChunks], bad = 0, wave_total = 0;
      uint64_t m[kFilterChunks];
#pragma unroll
      for (int e = 0; e < kFilterChunks; ++e) {
        slot[e] = -1;
        if (lp[e] >= 0) {
          if (lp[e] >= p.bt_stride) {
            bad |= kStPtRange;
          } else if (pg[e] < 0 || pg[e] >= p.num_pages) {
            bad |= kStPageRange;
          } else {
            slot[e] = (pg[e] << p.page_bits) | (int32_t)((uint32_t)uo[e] & pmask);
          }
        }
        m[e] = __ballot(slot[e] >= 0);
        wave_total += (int32_t)__builtin_popcountll(m[e]);
      }
      if (bad != 0 && p.status != nullptr) atomicOr(p.status, bad);
      if (lane == 0) wave_cnt[parity][wid] = wave_total;
      __syncthreads();
      int32_t before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) {
        const int32_t c = wave_cnt[parity][w];
        before += w < wid ? c : 0;
        total += c;
      }
      int32_t off = cnt + before;
#pragma unroll
      for (int e = 0; e < kFilterChunks; ++e) {
        const int32_t pos = (int32_t)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[e], 0u));
        if (slot[e] >= 0) out[off + pos] = slot[e];
        off += (int32_t)__builtin_popcountll(m[e]);
      }
      cnt += total;
      parity ^= 1;        // the next scan writes the other buffer: a wave that
                          // reaches it has left this one's reads behind
    }
    if (part == units_per_row - 1) {                  // the row is complete
      for (int32_t i = cnt + (int32_t)threadIdx.x; i < p.k; i += kBlock) out[i] = -1;
      if (threadIdx.x == 0) p.out_lens[t] = cnt;
    }
    cur = nxt;
  }
}

// ------------------------------------------------------------------ gather
// rows handled together by one wave per loop trip, and ids one wave
// resolves per batch
constexpr int kGatherUnroll = 8;
constexpr int kGatherBatch = 32;

template <int L> struct LaneCodes;          // this lane's share of a row
template <> struct LaneCodes<kV41> { uint2 codes; uint32_t scale; };
template <> struct LaneCodes<kV41Fp4> { uint32_t codes; uint32_t scale; };
template <> struct LaneCodes<kV4> { uint4 raw; uint32_t scale; };

template <int L>
__device__ __forceinline__ LaneCodes<L> load_lane(const PagedKV<L>& kv, int64_t slot, int lane);

// Plain (cached) loads: a gathered row's scale part shares its cache line
// with the scale parts of the page's other rows, which later ids of the
// batch often select.  (Non-temporal loads measured slower.)
template <>
__device__ __forceinline__ LaneCodes<kV41> load_lane<kV41>(const PagedKV<kV41>& kv, int64_t slot,
                                                           int lane) {
  LaneCodes<kV41> r;
  const u32x2 c = *(const u32x2*)(kv.data(slot) + 8 * lane);
  r.codes = make_uint2(c.x, c.y);
  r.scale = kv.scale(slot)[lane >> 2];
  return r;
}
template <>
__device__ __forceinline__ LaneCodes<kV41Fp4> load_lane<kV41Fp4>(const PagedKV<kV41Fp4>& kv,
                                                                 int64_t slot, int lane) {
  LaneCodes<kV41Fp4> r;
  r.codes = *(const uint32_t*)(kv.data(slot) + 4 * lane);
  r.scale = kv.scale(slot)[lane >> 1];
  return r;
}
template <>
__device__ __forceinline__ LaneCodes<kV4> load_lane<kV4>(const PagedKV<kV4>& kv, int64_t slot,
                                                         int lane) {
  LaneCodes<kV4> r;
  const uint8_t* d = kv.data(slot);
  if (lane < kRopeLane0) {
    const u32x2 c = *(const u32x2*)(d + 8 * lane);
    r.raw = make_uint4(c.x, c.y, 0u, 0u);
    r.scale = kv.scale(slot)[lane >> 3];
  } else {
    r.raw = ld_u4(d + kNope + 16 * (lane - kRopeLane0));
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

// A wave takes the rows of the gather kGatherBatch at a time: lane i reads
// id i of the batch and resolves it to a physical slot (one vector load of
// ids, one of page-table entries), then the rows are expanded kGatherUnroll
// at a time, their slots broadcast with v_readlane, all their loads issued
// before any store.  32-id batches give 8192 waves for 262,144 ids, about
// one resident round of the chip (measured faster than 16, 48 or 64).
template <int L>
__global__ __launch_bounds__(kBlock) void dequant_gather_kernel(GatherParams p) {
  const PagedKV<L> kv = paged<L>(p.cache);
  const int lane = lane_id();
  const int64_t wave0 = uniform64((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int32_t page_mask = (1 << p.cache.page_bits) - 1;

  for (int64_t b0 = wave0 * kGatherBatch; b0 < p.n; b0 += nwaves * kGatherBatch) {
    // ---- resolve this lane's id to a slot (-1: zero row)
    const int64_t r = b0 + lane;
    int32_t slot = -1;
    int32_t bad = 0;
    if (lane < kGatherBatch && r < p.n) {
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
    const int cnt = (int)(p.n - b0 < kGatherBatch ? p.n - b0 : kGatherBatch);
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
  // persistent: six workgroups per compute unit (measured best of 512..4096)
  const int64_t units = p.T * (p.k > 0 ? (p.k + kFilterUnit - 1) / kFilterUnit : 1);
  return launch(dcp_filter_kernel, grid_for(units, 1, 1536), p, stream);
}

hipError_t launch_dequant_gather(const GatherParams& p, hipStream_t stream) {
  int blocks = grid_for(p.n, (int64_t)kWavesPerBlock * kGatherBatch, 8192);
  if (launch_tuning().gather_blocks > 0) blocks = launch_tuning().gather_blocks;
  switch (p.cache.layout) {
    case kV41: return launch(dequant_gather_kernel<kV41>, blocks, p, stream);
    case kV41Fp4: return launch(dequant_gather_kernel<kV41Fp4>, blocks, p, stream);
    default: return launch(dequant_gather_kernel<kV4>, blocks, p, stream);
  }
}

}  // namespace kvc
