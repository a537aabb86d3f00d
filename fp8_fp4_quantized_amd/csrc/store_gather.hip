// store_gather.hip -- plain quantize-store of bf16 rows, the DCP id filter
// and the paged dequant-gather (gfx950).
//
// The store and the gather put one 512-dim row on one 64-lane wave (8 dims
// per lane), so every global access of a row is one contiguous, fully used
// span: the bf16 row (1024 B), the data part (512 / 256 / 576 B) and the
// scale part.  A wave runs several rows per loop trip so that their loads are
// in flight together; the grid strides over the rows.  The filter puts one
// row of global ids on one wave.
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

// ------------------------------------------------------------------ store
// A wave stores kStoreRows rows per loop trip: the loads of all of them (row
// bytes, destination, position) are issued before the first is quantized, so
// a wave keeps 2 KiB of reads in flight.  Rows past n reload row n - 1 (a
// fixed count of loads keeps the compiler's waits exact) and store nothing.
// ROPE: rotate the rope dims at positions[i] first (exact, one rounding).
constexpr int kStoreRows = 2;           // measured faster than 1, 4 or 8

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
// One wave per row of ids, no LDS and no barrier.  A pass takes 2048 ids of
// the row, 32 per lane: all 32 loads are issued together, then the owner
// test, then all 32 page-table loads together, then, 64 ids at a time in the
// row's order, a ballot gives each kept id its place after the ones already
// kept.  A row's tail of -1 goes out in 16-byte stores.  The kernel is bound
// by its per-id arithmetic, which is kept short: a bit-field extract and a
// bit-field insert for a power-of-two group, no clamping on full passes, one
// unsigned test for "kept and inside the page table", status bits worked out
// only for a chunk that drops an id.
constexpr int kFilterChunks = 32;                          // 64-id loads per lane and pass
constexpr int kFilterPass = kLanes * kFilterChunks;        // 2048 ids

template <bool POW2>
__global__ __launch_bounds__(kBlock) void dcp_filter_kernel(DcpFilterParams p) {
  const int lane = lane_id();
  const int kl = p.interleave_log2, wl = p.world_log2, pb = p.page_bits;
  const uint32_t kmask = (1u << kl) - 1, pmask = (1u << pb) - 1;
  const uint32_t world = (uint32_t)p.world, rank = (uint32_t)p.rank;
  // the page index of a kept id is below 2^(31 - pb); a row index of -1
  // (not kept) shifts to 2^(32 - pb) - 1, at or past this bound
  const uint32_t lim = 1u << (31 - pb);
  const uint32_t bts = p.bt_width < (int64_t)lim ? (uint32_t)p.bt_width : lim;
  const uint32_t npg = (uint32_t)(p.num_pages < 0x7FFFFFFF ? p.num_pages : 0x7FFFFFFF);
  const int32_t k = p.k;
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t t = uniform64((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)); t < p.T;
       t += nwaves) {
    int32_t* out = p.out_slots + t * p.out_stride;
    const int32_t req = ld_ro(p.token_to_req + t);
    bool keep = p.valid == nullptr || ld_ro(p.valid + t) != 0;
    uint32_t bad = 0;                                     // status bits of the row
    if (keep && (req < 0 || req >= p.n_req)) {
      bad = kStReqRange;
      keep = false;
    }
    int32_t cnt = 0;                                      // kept so far in the row
    if (keep && k > 0) {
      const int32_t* row = p.ids + t * p.ids_stride;
      const int32_t* bt = p.block_table + (int64_t)req * p.bt_stride;
      for (int32_t s0 = 0; s0 < k; s0 += kFilterPass) {
        int32_t v[kFilterChunks];
        if (s0 + kFilterPass <= k) {
          const int32_t* src = row + s0 + lane;
#pragma unroll
          for (int e = 0; e < kFilterChunks; ++e) v[e] = __builtin_nontemporal_load(src + kLanes * e);
        } else {
          // ids past the row read its last id and are not kept
#pragma unroll
          for (int e = 0; e < kFilterChunks; ++e) {
            const int32_t i = s0 + kLanes * e + lane;
            const int32_t x = __builtin_nontemporal_load(row + (i < k ? i : k - 1));
            v[e] = i < k ? x : -1;
          }
        }
        // owner test: v becomes this rank's row index, or -1
#pragma unroll
        for (int e = 0; e < kFilterChunks; ++e) {
          const uint32_t id = (uint32_t)v[e];
          uint32_t owner, uo;
          if constexpr (POW2) {
            owner = __builtin_amdgcn_ubfe(id, kl, wl);            // (id / K) % world
            uo = (id & kmask) | ((id >> wl) & ~kmask);            // (id / (K world)) K + id % K
          } else {
            const uint32_t run = id >> kl;
            const uint32_t turn = udiv_magic(run, p.world_div.m, p.world_div.sh1, p.world_div.sh2);
            owner = run - turn * world;
            uo = (turn << kl) | (id & kmask);
          }
          v[e] = v[e] >= 0 && owner == rank ? (int32_t)uo : -1;
          // the later tests read v itself (as lane masks, a pass of them
          // would overflow the scalar registers)
          asm volatile("" : "+v"(v[e]));
        }
        // page-table entries (an id not kept, or past the table, reads entry 0)
        int32_t pg[kFilterChunks];
#pragma unroll
        for (int e = 0; e < kFilterChunks; ++e) {
          const uint32_t lp = (uint32_t)v[e] >> pb;
          pg[e] = bt[lp < bts ? lp : 0u];
        }
        // slots, in the row's order.  A kept id whose page index lies past
        // the table, or whose page is out of range, is dropped; the status
        // bits are worked out only for a chunk that drops one.
#pragma unroll
        for (int e = 0; e < kFilterChunks; ++e) {
          const uint32_t lp = (uint32_t)v[e] >> pb;
          const int32_t q = lp < bts ? pg[e] : -1;
          const bool ok = (uint32_t)q < npg;
          const uint64_t m = __ballot(ok);
          if (m != __ballot(v[e] >= 0)) {
            if (__ballot(v[e] >= 0 && lp >= bts) != 0) bad |= kStPtRange;
            if (__ballot(lp < bts && (uint32_t)pg[e] >= npg) != 0) bad |= kStPageRange;
          }
          const int32_t slot = (int32_t)(((uint32_t)pg[e] << pb) | ((uint32_t)v[e] & pmask));
          const int32_t pos = (int32_t)__builtin_amdgcn_mbcnt_hi(
              (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          int32_t* const ob = out + cnt;                  // uniform base, lane offset
          if (ok) ob[(uint32_t)pos] = slot;
          cnt += (int32_t)__builtin_popcountll(m);
        }
      }
    }
    if (bad != 0 && lane == 0 && p.status != nullptr) atomicOr(p.status, (int32_t)bad);
    // -1 over [cnt, k): up to 3 single ids to a 16-byte boundary, 16-byte
    // stores, the last up to 3 ids
    if (k > 0) {
      const int32_t head = (int32_t)(((16u - ((uint32_t)(uintptr_t)(out + cnt) & 15u)) & 15u) >> 2);
      const int32_t a0 = cnt + head < k ? cnt + head : k;
      if (lane < a0 - cnt) out[cnt + lane] = -1;
      const int32_t a1 = a0 + ((k - a0) & ~3);
      for (int32_t i = a0 + 4 * lane; i < a1; i += 4 * kLanes)
        *(int4*)(out + i) = make_int4(-1, -1, -1, -1);
      if (lane < k - a1) out[a1 + lane] = -1;
    }
    if (lane == 0) p.out_lens[t] = cnt;
  }
}

// ------------------------------------------------------------------ gather
// The most ids one wave resolves per batch, and the fewest.
constexpr int kGatherBatch = 32;
constexpr int kGatherMinBatch = 8;
// A large gather (from 2^17 ids: its codes alone fill the chip's 32 MiB of
// L2) streams its codes past the L2 and expands 16 rows per loop trip (0.5%
// faster than 8 on 262,144 V41 ids; 32 needs more registers than eight waves
// per SIMD allow and ran 48% slower); V4 keeps 8, whose 16-byte lane shares
// of 16 rows would not fit those registers.  A smaller gather caches its
// codes and takes 8 rows per trip (its batches hold at most 8 to 16 ids;
// 16-row trips measured 10% slower on 18,642 ids).
constexpr int64_t kLargeGatherIds = int64_t(1) << 17;
template <int L, bool LARGE> constexpr int gather_unroll() { return LARGE && L != kV4 ? 16 : 8; }
// workgroup of a large gather: 8 waves (0.6% faster than 4 on 262,144 V41
// ids; 2 and 16 slower); a smaller gather keeps 4
template <bool LARGE> constexpr int gather_block() { return LARGE ? 512 : kBlock; }
// most waves of a gather's grid (2^20 ids at 32 per batch); rows past them
// take further turns
constexpr int64_t kGatherMaxWaves = 32768;

template <int L> struct LaneCodes;          // this lane's share of a row
template <> struct LaneCodes<kV41> { uint2 codes; uint32_t scale; };
template <> struct LaneCodes<kV41Fp4> { uint32_t codes; uint32_t scale; };
template <> struct LaneCodes<kV4> { uint4 raw; uint32_t scale; };

// Loads from the row's own base (the slot is the same on every lane).  A
// row's scale part shares its cache line with the scale parts of the page's
// other rows, so it is always a cached load (non-temporal: 6% slower on a
// 262,144-id gather).  The codes take CPOL: a large gather reads each row
// once and loads them non-temporally, so that the L2 keeps what the launch
// reads more than once -- the ids, the page-table entries and the scale
// lines (0.75 us faster on 262,144 ids than cached loads); a small gather
// caches them, since the next call may read the same rows again.
template <int L, int CPOL>
__device__ __forceinline__ LaneCodes<L> load_lane(const PagedKV<L>& kv, int64_t slot, int lane) {
  LaneCodes<L> r;
  if constexpr (L == kV41) {
    r.codes = ld_u2_buf<CPOL>(kv.data(slot), 8u * lane);
    r.scale = ld_u8_dev(kv.scale(slot), (uint32_t)lane >> 2);
  } else if constexpr (L == kV41Fp4) {
    r.codes = ld_u32_buf<CPOL>(kv.data(slot), 4u * lane);
    r.scale = ld_u8_dev(kv.scale(slot), (uint32_t)lane >> 1);
  } else {
    const uint8_t* d = kv.data(slot);
    if (lane < kRopeLane0) {
      const uint2 c = ld_u2_buf<CPOL>(d, 8u * lane);
      r.raw = make_uint4(c.x, c.y, 0u, 0u);
      r.scale = ld_u8_dev(kv.scale(slot), (uint32_t)lane >> 3);
    } else {
      r.raw = ld_u4_buf<CPOL>(d, kNope + 16u * (lane - kRopeLane0));
      r.scale = 0;
    }
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

// A wave takes the rows of the gather p.batch at a time: lane i reads id i
// of the batch and resolves it to a physical slot (one vector load of ids,
// one of page-table entries), then the rows are expanded gather_unroll() at
// a time, their slots broadcast with v_readlane, all their loads issued before
// any store.  32-id batches give 8192 waves for 262,144 ids, one resident
// round of the chip at eight waves per SIMD (measured faster than 16, 48 or
// 64); a smaller gather takes smaller batches, so that its rows spread over
// more waves.  Eight waves per SIMD asked of the compiler: it then keeps the
// kernel to 78 scalar registers (93 otherwise), and the launch's 8192 waves
// go through 0.9% faster.
template <int L, bool LARGE>
__global__ __launch_bounds__(gather_block<LARGE>()) __attribute__((amdgpu_waves_per_eu(8, 8)))
void dequant_gather_kernel(GatherParams p) {
  constexpr int CPOL = LARGE ? kCpolNtSc1 : kCpolSc1;
  constexpr int kWaves = gather_block<LARGE>() / kLanes;
  const PagedKV<L> kv = paged<L>(p.cache);
  const int lane = lane_id();
  const int64_t wave0 = uniform64((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int32_t page_mask = (1 << p.cache.page_bits) - 1;

  const int32_t batch = p.batch;
  for (int64_t b0 = wave0 * batch; b0 < p.n; b0 += nwaves * batch) {
    // ---- resolve this lane's id to a slot (-1: zero row)
    const int64_t r = b0 + lane;
    int32_t slot = -1;
    int32_t bad = 0;
    if (lane < batch && r < p.n) {
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
    const int cnt = (int)(p.n - b0 < batch ? p.n - b0 : batch);
    constexpr int U = gather_unroll<L, LARGE>();
    for (int j = 0; j < cnt; j += U) {
      int32_t s[U];
      LaneCodes<L> c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u] = j + u < cnt ? __builtin_amdgcn_readlane(slot, j + u) : -1;
        if (s[u] >= 0) c[u] = load_lane<L, CPOL>(kv, s[u], lane);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j + u >= cnt) break;
        const uint4 o = s[u] >= 0 ? decode_lane<L>(c[u], lane) : make_uint4(0u, 0u, 0u, 0u);
        st_u4_stream(p.out + b0 * p.out_stride,
                     (uint32_t)(((j + u) * p.out_stride + kDimsPerLane * lane) * 2), o);
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
  // one wave per row (rows past the grid's waves take further turns)
  const int blocks = grid_for(p.T, kWavesPerBlock, 1 << 20);
  return p.world_log2 >= 0 ? launch(dcp_filter_kernel<true>, blocks, p, stream)
                           : launch(dcp_filter_kernel<false>, blocks, p, stream);
}

hipError_t launch_dequant_gather(const GatherParams& p_in, hipStream_t stream) {
  // batches of 32 from 2^17 ids up, smaller below: at least 4096 waves
  // where the ids allow, one per 8 ids at the fewest
  GatherParams p = p_in;
  p.batch = kGatherBatch;
  while (p.batch > kGatherMinBatch && p.n < (int64_t)p.batch * 4096) p.batch >>= 1;
  const bool large = p.n >= kLargeGatherIds;
  const int block = large ? gather_block<true>() : gather_block<false>();
  const int64_t waves_per_block = block / kLanes;
  const int blocks = grid_for(p.n, waves_per_block * p.batch,
                              (int)(kGatherMaxWaves / waves_per_block));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(block), 0, stream, p);
    return hipGetLastError();
  };
  switch (p.cache.layout) {
    case kV41:
      return large ? go(dequant_gather_kernel<kV41, true>) : go(dequant_gather_kernel<kV41, false>);
    case kV41Fp4:
      return large ? go(dequant_gather_kernel<kV41Fp4, true>)
                   : go(dequant_gather_kernel<kV41Fp4, false>);
    default:
      return large ? go(dequant_gather_kernel<kV4, true>) : go(dequant_gather_kernel<kV4, false>);
  }
}

}  // namespace kvc
