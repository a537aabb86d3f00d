// compress.hip -- the fused ratio-1 / ratio-2 compressor (gfx950).
//
// One 64-lane wave makes one compressed row at a time: it loads the pair's kv
// and score rows (16 B per lane each), pools them with a per-dim softmax over
// the two scores (ratio 2), RMS-normalises over the 512 dims (one wave sum),
// writes the pre-RoPE latent, rotates the 64 rope dims (lanes 56..63, four
// pairs per lane; the table entries reach them by lane shuffles), rounds to
// bf16 and quantizes the row into its paged slot.  (sglang PR #39652
// "dsv4.1: compression, KV I/O, and metadata kernels", Summary and Review;
// sglang PR #46230, summary.)
//
// Prefill batches are ragged: the int32 [2, S] extend offsets become per-slot
// work counts and latent starts on the device -- up to 256 slots in one
// wave's lanes, one, two or four per lane (a work item finds its slot with
// as many ballots), more with a scan in LDS and a binary search -- so the
// launch needs no host-side knowledge of the row counts (and can be captured
// in a graph).  A work item is a tile of consecutive compressed rows of one
// slot; a wave issues the loads of all its rows before it finishes the first.
//
// Decode and verify batches give one wave per slot, which takes the slot's
// tokens in order, or, when the ring has more entries than a call's pairs,
// one wave per row.  The ratio-2 pending tokens live in a per-slot ring (pair
// k in entry k % ring_slots), and under decode context parallelism the rows
// another rank owns are computed but not stored (flashinfer_sparse.py, DCP
// helpers).
#include "launch.hpp"
#include "row_ops.hpp"

namespace kvc {

namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kLanes;
constexpr int kMaxPrefillSlots = 8191;   // two LDS tables of S + 1 ints fit in 64 KiB
// default rows per prefill work item: 2, or 1 for a batch of at most
// kSmallBatchRows rows (latent capacity), whose rows then spread over more
// waves (measured faster up to 8192 rows, slower from 16384)
constexpr int kTileLog2 = 1;
constexpr int64_t kSmallBatchRows = 8192;
// prefill grid cap: 1024 workgroups of 4 waves (measured best for the
// 32,768-token batch against 512 .. 2048)
constexpr int64_t kMaxPrefillBlocks = 1024;

// One compressed row.  Token rows are indices into the projection buffer;
// `from_state` says the pair's first token is the pending-state entry
// `st_row` (entries counted over all slots: slot b's ring starts at entry
// b * ring_slots).  Indices are 32-bit: positions, offsets and the LDS row
// tables are int32, cache slots are below 2^31 (num_pages * page_size is
// checked on the host) and rings hold at most 8191 * 1024 entries;
// addresses are formed in 64 bits where they are used.
struct RowJob {
  int32_t t1;             // second (or only) token of the row
  int32_t rot_pos;        // rotary position
  int32_t latent_idx;
  int32_t loc;            // destination slot in the cache (0: no write)
  int32_t st_row;
  int32_t loc_err;        // status bit raised instead of the write (0: none)
  bool from_state;
};

// a rotary position held in 32 bits: positions past 2^31 - 1 (beyond any
// table) saturate, so they are reported as outside the table
__device__ __forceinline__ int32_t sat_pos(int64_t q) {
  return q > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)q;
}

// the pending-state entry of pair k of slot b: entry k % ring_slots of the
// slot's ring
__device__ __forceinline__ int32_t ring_row(const CompressParams& p, int32_t b, int32_t k) {
  const uint32_t R = (uint32_t)p.ring_slots;
  return (int32_t)((uint32_t)b * R + (R == 1 ? 0u : (uint32_t)k % R));
}

// registers of one row's inputs: this lane's 16 B of the pair's kv and score
// rows and one entry of the row's rotary-table line (lane k holds entry k;
// the rope lanes gather theirs with lane shuffles when they rotate)
struct RowIn {
  uint4 k0, s0, k1, s1;
  float f;
};

// Every lane issues the same loads whatever the row (the first token comes
// from the pending state or the buffer by an address select), so the count
// of memory operations in flight is fixed and the compiler's waits stay
// exact.  The token rows are read once and loaded non-temporally: they then
// take no cache lines from what earlier kernels left dirty, whose write-back
// would otherwise fall inside this launch (on the 32,768-token prefill after
// a 512 MB write: 26.9 -> 20.5 us; 0.1 us slower with clean caches).
template <int RATIO>
__device__ __forceinline__ RowIn load_row(const CompressParams& p, const RowJob& j) {
  const int lane = lane_id();
  const int dim0 = kDimsPerLane * lane;
  RowIn in;
  in.k1 = ld_u4_nt(p.kv + (int64_t)j.t1 * p.kv_stride + dim0);
  in.k0 = in.s0 = in.s1 = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (RATIO == 2) {
    in.s1 = ld_u4_nt(p.score + (int64_t)j.t1 * p.score_stride + dim0);
    const uint16_t* st = p.state + (int64_t)j.st_row * 2 * kDim;
    const uint16_t* k0 = j.from_state ? st : p.kv + (int64_t)(j.t1 - 1) * p.kv_stride;
    const uint16_t* s0 = j.from_state ? st + kDim : p.score + (int64_t)(j.t1 - 1) * p.score_stride;
    in.k0 = ld_u4_nt(k0 + dim0);
    in.s0 = ld_u4_nt(s0 + dim0);
  }
  const int32_t rp = j.rot_pos < 0 ? 0 : (j.rot_pos >= p.max_pos ? (int32_t)p.max_pos - 1 : j.rot_pos);
  in.f = p.freqs[(int64_t)rp * kRope + lane];
  return in;
}

// The arithmetic of one row, with no memory access and no branch, so that a
// tile's rows can be scheduled together: pooling, RMSNorm, the pre-RoPE
// latent, RoPE and the quantized codes.
template <int L>
struct RowOut {
  uint4 lat;              // pre-RoPE latent, bf16
  uint4 z;                // post-RoPE row fed to the quantizer, bf16
  RowQ<L> q;              // its codes and scale bytes
};

template <int L, int RATIO>
__device__ __forceinline__ RowOut<L> compute_row(const CompressParams& p, const float (&w)[8],
                                                 const RowIn& in) {
  const int lane = lane_id();

  // ---- pooling (ratio 2): softmax over the two scores, per dim
  const uint32_t k1w[4] = {in.k1.x, in.k1.y, in.k1.z, in.k1.w};
  float v[8];
  if constexpr (RATIO == 2) {
    const uint32_t k0w[4] = {in.k0.x, in.k0.y, in.k0.z, in.k0.w};
    const uint32_t s0w[4] = {in.s0.x, in.s0.y, in.s0.z, in.s0.w};
    const uint32_t s1w[4] = {in.s1.x, in.s1.y, in.s1.z, in.s1.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float a0 = h ? bf16_hi(s0w[q]) : bf16_lo(s0w[q]);
        const float a1 = h ? bf16_hi(s1w[q]) : bf16_lo(s1w[q]);
        const float kk0 = h ? bf16_hi(k0w[q]) : bf16_lo(k0w[q]);
        const float kk1 = h ? bf16_hi(k1w[q]) : bf16_lo(k1w[q]);
        // the two-way softmax is a sigmoid of the score difference:
        // v = k1 + (k0 - k1) / (1 + exp(a1 - a0)); exp overflowing to
        // infinity gives weight 0, underflowing to 0 gives weight 1
        const float g = __builtin_amdgcn_rcpf(1.f + __expf(a1 - a0));
        v[2 * q + h] = fmaf(kk0 - kk1, g, kk1);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_lo(k1w[q]);
      v[2 * q + 1] = bf16_hi(k1w[q]);
    }
  }

  // ---- RMSNorm over the 512 dims
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += v[k] * v[k];
  ss = wave_sum_f32(ss);
  const float r = rsqrtf(ss * (1.0f / kDim) + p.eps);
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = v[k] * r * w[k];

  RowOut<L> o;
  o.lat = make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                     pack_bf16(y[6], y[7]));

  // ---- RoPE on the last 64 dims: pairs (2i, 2i+1) times (cos, sin); rope
  // lane 56 + m takes table entries 8m .. 8m + 7 from the lanes holding them
  // (every lane computes, the nope lanes keep the latent)
  float cs[8];
  const int src = kDimsPerLane * ((lane - kRopeLane0) & 7);
#pragma unroll
  for (int i = 0; i < 8; ++i) cs[i] = __int_as_float(__shfl(__float_as_int(in.f), src + i));
  float rot[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = y[2 * i], b = y[2 * i + 1], c = cs[2 * i], s = cs[2 * i + 1];
    rot[2 * i] = a * c - b * s;
    rot[2 * i + 1] = a * s + b * c;
  }
  // per-word selects (a select of the whole vector compiles to an indexed
  // private array)
  const bool rope = lane >= kRopeLane0;
  o.z.x = rope ? pack_bf16(rot[0], rot[1]) : o.lat.x;
  o.z.y = rope ? pack_bf16(rot[2], rot[3]) : o.lat.y;
  o.z.z = rope ? pack_bf16(rot[4], rot[5]) : o.lat.z;
  o.z.w = rope ? pack_bf16(rot[6], rot[7]) : o.lat.w;
  o.q = quantize_row<L>(o.z);
  return o;
}

// The stores of one computed row: latent, pre-quant copy and the quantized
// row at its destination slot (0: padded row, no cache write), with the
// status bits of whatever is out of range.
template <int L>
__device__ __forceinline__ void store_row_out(const CompressParams& p, const PagedKV<L>& kv,
                                              const RowJob& j, const RowOut<L>& o) {
  if (j.rot_pos < 0 || j.rot_pos >= p.max_pos) {
    raise_status(p.status, kStPosRange);
    return;
  }
  const int dim0 = kDimsPerLane * lane_id();
  const bool lat_ok = j.latent_idx < p.max_out_rows;
  if (lat_ok) {
    st_u4_nt(p.latent + (int64_t)j.latent_idx * p.latent_stride + dim0, o.lat);
    if (p.prequant != nullptr)
      st_u4(p.prequant + (int64_t)j.latent_idx * p.prequant_stride + dim0, o.z);
  } else {
    raise_status(p.status, kStLatentRange);
  }
  bool write = j.loc_err == 0 && j.loc != 0;
  if (j.loc_err != 0) raise_status(p.status, j.loc_err);
  if (write && !kv.valid(j.loc)) {
    raise_status(p.status, kStPageRange);
    write = false;
  }
  const int32_t slot = write ? j.loc : 0;
  store_quantized<L>(o.q, o.z, kv.data(slot), kv.scale(slot), write);
}

template <int L, int RATIO>
__device__ __forceinline__ void finish_row(const CompressParams& p, const PagedKV<L>& kv,
                                           const float (&w)[8], const RowJob& j, const RowIn& in) {
  store_row_out<L>(p, kv, j, compute_row<L, RATIO>(p, w, in));
}

// the destination slot of row c of slot b through the page table
__device__ __forceinline__ void page_loc(const CompressParams& p, int32_t b, int32_t c,
                                         int32_t& loc, int32_t& err) {
  loc = 0;
  err = 0;
  const int32_t lp = c >> p.cache.page_bits;
  if (lp >= p.pt_width) {
    err = kStPtRange;
    return;
  }
  const int32_t phys = ld_ro(p.page_table + (int64_t)b * p.pt_stride + lp);
  if (phys < 0 || phys >= p.cache.num_pages) {
    err = kStPageRange;
    return;
  }
  loc = (phys << p.cache.page_bits) | (c & ((1 << p.cache.page_bits) - 1));
}

// the destination of row c of slot b on this rank: with the rows dealt over
// a decode-context-parallel group in runs of K = 2^interleave_log2, run
// c / K belongs to rank (c / K) % world, which keeps it as its row
// (c / (K * world)) * K + c % K; rows of other ranks are not stored (loc 0)
__device__ __forceinline__ void dest_loc(const CompressParams& p, int32_t b, int32_t c,
                                         int32_t& loc, int32_t& err) {
  if (p.dcp_world > 1) {
    const int kl = p.dcp_interleave_log2;
    const uint32_t run = (uint32_t)c >> kl;
    const uint32_t turn = udiv_magic(run, p.dcp_div.m, p.dcp_div.sh1, p.dcp_div.sh2);
    if (run - turn * (uint32_t)p.dcp_world != (uint32_t)p.dcp_rank) {
      loc = 0;
      err = 0;
      return;
    }
    c = (int32_t)((turn << kl) | ((uint32_t)c & ((1u << kl) - 1)));
  }
  page_loc(p, b, c, loc, err);
}

// write a token's kv and score (this lane's 16 B of each) into pending-state
// entry st_row
__device__ __forceinline__ void write_state_regs(const CompressParams& p, int32_t st_row,
                                                 uint4 kvv, uint4 scv) {
  const int dim0 = kDimsPerLane * lane_id();
  uint16_t* st = p.state + (int64_t)st_row * 2 * kDim;
  st_u4(st + dim0, kvv);
  st_u4(st + kDim + dim0, scv);
}

// copy a token's kv and score rows into pending-state entry st_row
__device__ __forceinline__ void write_state(const CompressParams& p, int32_t st_row, int32_t tok) {
  const int dim0 = kDimsPerLane * lane_id();
  uint16_t* st = p.state + (int64_t)st_row * 2 * kDim;
  const uint4 kvv = ld_u4_nt(p.kv + (int64_t)tok * p.kv_stride + dim0);
  const uint4 scv = ld_u4_nt(p.score + (int64_t)tok * p.score_stride + dim0);
  st_u4(st + dim0, kvv);
  st_u4(st + kDim + dim0, scv);
}

// Per-slot work of a prefill batch.  The slot's compressed rows c0 .. c0 +
// rows - 1 are cut into tiles aligned to multiples of T in c, so every tile
// stays inside one page (T divides the page size) and the rows that share a
// scale cache line are written by one wave.  A last token at an even
// position becomes the pending state (ratio 2); the slot's first tile does
// that after its first row, which may read the old state.  A slot with such a
// tail and no rows gets one work item for it.
struct SlotWork {
  int32_t rows, items, c0;
  bool tail;
};
template <int RATIO>
__device__ __forceinline__ SlotWork slot_work(int32_t n, int32_t P, int32_t tile_log2) {
  SlotWork s{0, 0, 0, false};
  if (n <= 0 || P < 0) return s;
  // positions are int32: a slot running past 2^31 - 1 is cut there (its
  // result is unspecified, but every index stays in range)
  const int32_t end = (int64_t)P + n > 0x7FFFFFFF ? 0x7FFFFFFF : P + n;
  if constexpr (RATIO == 1) {
    s.rows = end - P;
    s.c0 = P;
  } else {
    s.rows = (end >> 1) - (P >> 1);          // odd positions in [P, end)
    s.c0 = P >> 1;                           // row of the first odd position
    s.tail = (end & 1) != 0;                 // last position end - 1 is even
  }
  if (s.rows > 0) {
    s.items = ((s.c0 + s.rows - 1) >> tile_log2) - (s.c0 >> tile_log2) + 1;
  } else {
    s.items = s.tail ? 1 : 0;
  }
  return s;
}

// a slot's token rows first .. first + n - 1 lie in the projection buffer
// (a slot with no tokens is always in range); a slot outside it is skipped
// whole and flagged
__device__ __forceinline__ bool slot_in_buffer(int32_t first, int32_t n, int64_t kv_rows) {
  return n <= 0 || (first >= 0 && (int64_t)first + n <= kv_rows);
}

// exclusive scans of work items and rows over the slots, into LDS
template <int RATIO>
__device__ void build_tables(const CompressParams& p, int32_t* item_start, int32_t* row_start) {
  __shared__ int32_t tot_i[kWavesPerBlock], tot_r[kWavesPerBlock];
  const int S = p.num_slots;
  const int lane = lane_id(), wid = threadIdx.x >> 6;
  int32_t carry_i = 0, carry_r = 0;
  for (int base = 0; base < S; base += kBlock) {
    const int b = base + threadIdx.x;
    SlotWork sw{0, 0, 0, false};
    if (b < S) {
      const int32_t n = p.offsets[S + b];
      const bool in_buf = slot_in_buffer(p.offsets[b], n, p.kv_rows);
      if (!in_buf && blockIdx.x == 0 && p.status != nullptr) atomicOr(p.status, kStTokenRange);
      sw = slot_work<RATIO>(in_buf ? n : 0, p.start_pos[b], p.tile_log2);
    }
    const int32_t si = wave_incl_scan_i32(sw.items), sr = wave_incl_scan_i32(sw.rows);
    if (lane == kLanes - 1) {
      tot_i[wid] = si;
      tot_r[wid] = sr;
    }
    __syncthreads();
    int32_t oi = carry_i, orr = carry_r;
    for (int q = 0; q < wid; ++q) {
      oi += tot_i[q];
      orr += tot_r[q];
    }
    if (b < S) {
      item_start[b] = oi + si - sw.items;
      row_start[b] = orr + sr - sw.rows;
    }
    for (int q = 0; q < kWavesPerBlock; ++q) {
      carry_i += tot_i[q];
      carry_r += tot_r[q];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    item_start[S] = carry_i;
    row_start[S] = carry_r;
  }
  __syncthreads();
}

// One prefill work item: the tile kt of slot b (slot data already at hand).
template <int L, int RATIO, int kTileRows>
__device__ __forceinline__ void run_tile(const CompressParams& p, const PagedKV<L>& kv,
                                         const float (&w)[8], int32_t b, int32_t kt, int32_t lat0,
                                         int32_t rows, int32_t first, int32_t n, int32_t P) {
  const int tl = p.tile_log2;
  const int32_t page_mask = (1 << p.cache.page_bits) - 1;
  const int32_t c0 = RATIO == 1 ? P : (P >> 1);
  const int32_t tbase = ((c0 >> tl) + kt) << tl;
  const int32_t c_lo = c0 > tbase ? c0 : tbase;
  const int32_t c_end = c0 + rows, t_end = tbase + (1 << tl);
  const int32_t c_hi = c_end < t_end ? c_end : t_end;

  if (c_lo < c_hi) {
    // all loads of the tile's rows are issued before the first row is
    // finished; a tile shorter than kTileRows reloads its last row
    RowJob j[kTileRows];
    RowIn in[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const int32_t c = c_lo + r < c_hi ? c_lo + r : c_hi - 1;
      j[r].st_row = 0;
      j[r].latent_idx = lat0 + (c - c0);
      if constexpr (RATIO == 1) {
        j[r].t1 = first + (c - P);
        j[r].rot_pos = c;
        j[r].from_state = false;
      } else {
        const int64_t q = 2 * (int64_t)c + 1;    // odd position closing the pair
        j[r].t1 = first + (int32_t)(q - P);
        j[r].rot_pos = sat_pos(q - 1);
        j[r].from_state = q - 1 < P;             // first token precedes the extend
        if (j[r].from_state) j[r].st_row = ring_row(p, b, c);
      }
      in[r] = load_row<RATIO>(p, j[r]);
    }
    if (p.dcp_world > 1) {
      // rows dealt over a context-parallel group: each row has its own owner
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) {
        const int32_t c = c_lo + r < c_hi ? c_lo + r : c_hi - 1;
        dest_loc(p, b, c, j[r].loc, j[r].loc_err);
      }
    } else {
      // the tile's rows share one page (aligned, no larger than a page): one
      // page-table lookup, needed only when the rows are stored
      int32_t loc0;
      int32_t loc_err;
      page_loc(p, b, c_lo, loc0, loc_err);
      const int32_t page_base = loc0 - (c_lo & page_mask);
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) {
        j[r].loc_err = loc_err;
        j[r].loc = loc_err ? 0 : page_base + ((c_lo + r) & page_mask);
      }
    }
    // the tile's arithmetic as one block (the rows' instruction streams
    // interleave), then its stores
    RowOut<L> o[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) o[r] = compute_row<L, RATIO>(p, w, in[r]);
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      if (c_lo + r < c_hi) store_row_out<L>(p, kv, j[r], o[r]);
    }
  }
  if constexpr (RATIO == 2) {
    if (kt == 0 && (((int64_t)P + n) & 1))
      write_state(p, ring_row(p, b, (int32_t)(((int64_t)P + n - 1) >> 1)), first + n - 1);
  }
}

// The work item of wave `wave0` in pass `k` of a prefill grid (nwaves items per
// pass, items 0 .. total - 1), or -1 when the wave has none left.  The first
// pass goes in wave order, every later pass in reverse wave order, so that
// the waves dispatched first take a pass's last items (0.8% faster on the
// 32,768-token batch than every pass in wave order: 16.95 against 17.08 us,
// 60 samples each).  Each pass covers its items once.
__device__ __forceinline__ int32_t pass_item(int32_t k, int32_t wave0, int32_t nwaves,
                                             int32_t total) {
  const int64_t base = (int64_t)k * nwaves;
  if (base >= total) return -1;
  const int32_t span = total - base < nwaves ? (int32_t)(total - base) : nwaves;
  if (wave0 >= span) return -1;
  return (int32_t)base + (k == 0 ? wave0 : span - 1 - wave0);
}

// Prefill with up to 64 slots: every lane holds one slot's work counts and
// their inclusive prefix sums, and a work item finds its slot with one
// ballot -- no LDS, no barrier.
template <int L, int RATIO, int kTileRows>
__global__ __launch_bounds__(kBlock) void compress_prefill_small_kernel(CompressParams p) {
  const PagedKV<L> kv{p.cache.base, p.cache.page_stride, p.cache.num_pages, p.cache.page_bits};
  const int lane = lane_id();
  const int S = p.num_slots;
  int32_t first = 0, n = 0, P = 0;
  if (lane < S) {
    first = p.offsets[lane];
    n = p.offsets[S + lane];
    P = p.start_pos[lane];
  }
  const uint4 wr = ld_u4(p.norm_w + kDimsPerLane * lane);
  if (!slot_in_buffer(first, n, p.kv_rows)) {
    n = 0;
    if (blockIdx.x == 0 && p.status != nullptr) atomicOr(p.status, kStTokenRange);
  }
  const SlotWork sw = lane < S ? slot_work<RATIO>(n, P, p.tile_log2) : SlotWork{0, 0, 0, false};
  // inclusive sums over the slots (DPP scan: the first item's loads wait on it)
  const int32_t inc_i = wave_incl_scan_i32(sw.items), inc_r = wave_incl_scan_i32(sw.rows);
  const float w[8] = {bf16_lo(wr.x), bf16_hi(wr.x), bf16_lo(wr.y), bf16_hi(wr.y),
                      bf16_lo(wr.z), bf16_hi(wr.z), bf16_lo(wr.w), bf16_hi(wr.w)};
  const int32_t total = __builtin_amdgcn_readlane(inc_i, kLanes - 1);
  const int32_t wave0 = uniform((int32_t)blockIdx.x * kWavesPerBlock + (int32_t)(threadIdx.x >> 6));
  const int32_t nwaves = (int32_t)gridDim.x * kWavesPerBlock;
  for (int32_t pass = 0;; ++pass) {
    const int32_t item = pass_item(pass, wave0, nwaves, total);
    if (item < 0) break;
    // slot b = number of slots whose items all come before this one
    const int32_t b = __builtin_popcountll(__ballot(inc_i <= item));
    const int32_t kt = item - (__builtin_amdgcn_readlane(inc_i, b) - __builtin_amdgcn_readlane(sw.items, b));
    const int32_t rows = __builtin_amdgcn_readlane(sw.rows, b);
    const int32_t lat0 = __builtin_amdgcn_readlane(inc_r, b) - rows;
    run_tile<L, RATIO, kTileRows>(p, kv, w, b, kt, lat0, rows, __builtin_amdgcn_readlane(first, b),
                                  __builtin_amdgcn_readlane(n, b), __builtin_amdgcn_readlane(P, b));
  }
}

// Prefill with 65 to 64 * SPL slots (SPL = 2 or 4): lane l holds slots
// l * SPL .. l * SPL + SPL - 1 (their work counts and inclusive prefix sums,
// in slot order), and a work item finds its slot with SPL ballots -- no LDS,
// no barrier.  The one-slot kernel above stays separate: this form at
// SPL = 1 compiled to code measured slightly slower on the 16-request batch.
template <int L, int RATIO, int kTileRows, int SPL>
__global__ __launch_bounds__(kBlock) void compress_prefill_multi_kernel(CompressParams p) {
  const PagedKV<L> kv{p.cache.base, p.cache.page_stride, p.cache.num_pages, p.cache.page_bits};
  const int lane = lane_id();
  const int S = p.num_slots;
  int32_t first[SPL], n[SPL], P[SPL], items[SPL], rows[SPL];
#pragma unroll
  for (int k = 0; k < SPL; ++k) {
    const int s = lane * SPL + k;
    first[k] = n[k] = P[k] = 0;
    if (s < S) {
      first[k] = p.offsets[s];
      n[k] = p.offsets[S + s];
      P[k] = p.start_pos[s];
    }
  }
  const uint4 wr = ld_u4(p.norm_w + kDimsPerLane * lane);
#pragma unroll
  for (int k = 0; k < SPL; ++k) {
    if (!slot_in_buffer(first[k], n[k], p.kv_rows)) {
      n[k] = 0;
      if (blockIdx.x == 0 && p.status != nullptr) atomicOr(p.status, kStTokenRange);
    }
  }
  int32_t tot_i = 0, tot_r = 0;
#pragma unroll
  for (int k = 0; k < SPL; ++k) {
    const SlotWork sw = lane * SPL + k < S ? slot_work<RATIO>(n[k], P[k], p.tile_log2)
                                           : SlotWork{0, 0, 0, false};
    items[k] = sw.items;
    rows[k] = sw.rows;
    tot_i += sw.items;
    tot_r += sw.rows;
  }
  // inclusive scan of the lanes' totals, then each slot's inclusive sums
  const int32_t inc_i = wave_incl_scan_i32(tot_i), inc_r = wave_incl_scan_i32(tot_r);
  int32_t ci[SPL], cr[SPL];
  {
    int32_t ri = inc_i - tot_i, rr = inc_r - tot_r;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      ri += items[k];
      rr += rows[k];
      ci[k] = ri;
      cr[k] = rr;
    }
  }
  const float w[8] = {bf16_lo(wr.x), bf16_hi(wr.x), bf16_lo(wr.y), bf16_hi(wr.y),
                      bf16_lo(wr.z), bf16_hi(wr.z), bf16_lo(wr.w), bf16_hi(wr.w)};
  const int32_t total = __builtin_amdgcn_readlane(inc_i, kLanes - 1);
  const int32_t wave0 = uniform((int32_t)blockIdx.x * kWavesPerBlock + (int32_t)(threadIdx.x >> 6));
  const int32_t nwaves = (int32_t)gridDim.x * kWavesPerBlock;
  for (int32_t pass = 0;; ++pass) {
    const int32_t item = pass_item(pass, wave0, nwaves, total);
    if (item < 0) break;
    // slot b = number of slots whose items all come before this one
    int32_t b = 0;
#pragma unroll
    for (int k = 0; k < SPL; ++k) b += __builtin_popcountll(__ballot(ci[k] <= item));
    const int32_t bl = b / SPL, bk = b % SPL;              // its lane and register
    int32_t v_rows = rows[0], v_ci = ci[0], v_items = items[0], v_cr = cr[0];
    int32_t v_first = first[0], v_n = n[0], v_P = P[0];
#pragma unroll
    for (int k = 1; k < SPL; ++k) {
      if (bk == k) {
        v_rows = rows[k];
        v_ci = ci[k];
        v_items = items[k];
        v_cr = cr[k];
        v_first = first[k];
        v_n = n[k];
        v_P = P[k];
      }
    }
    const int32_t nrows = __builtin_amdgcn_readlane(v_rows, bl);
    const int32_t kt = item - (__builtin_amdgcn_readlane(v_ci, bl) - __builtin_amdgcn_readlane(v_items, bl));
    const int32_t lat0 = __builtin_amdgcn_readlane(v_cr, bl) - nrows;
    run_tile<L, RATIO, kTileRows>(p, kv, w, b, kt, lat0, nrows, __builtin_amdgcn_readlane(v_first, bl),
                                  __builtin_amdgcn_readlane(v_n, bl), __builtin_amdgcn_readlane(v_P, bl));
  }
}

// Prefill with any number of slots (up to kMaxPrefillSlots; used above 256):
// the per-slot prefix sums go to LDS and work items find their slot by
// binary search.
template <int L, int RATIO, int kTileRows>
__global__ __launch_bounds__(kBlock) void compress_prefill_kernel(CompressParams p) {
  extern __shared__ int32_t tables[];
  const PagedKV<L> kv{p.cache.base, p.cache.page_stride, p.cache.num_pages, p.cache.page_bits};
  const int lane = lane_id();
  const uint4 wr = ld_u4(p.norm_w + kDimsPerLane * lane);
  const float w[8] = {bf16_lo(wr.x), bf16_hi(wr.x), bf16_lo(wr.y), bf16_hi(wr.y),
                      bf16_lo(wr.z), bf16_hi(wr.z), bf16_lo(wr.w), bf16_hi(wr.w)};
  const int32_t wave0 = uniform((int32_t)blockIdx.x * kWavesPerBlock + (int32_t)(threadIdx.x >> 6));
  const int32_t nwaves = (int32_t)gridDim.x * kWavesPerBlock;
  const int S = p.num_slots;

  int32_t* item_start = tables;
  int32_t* row_start = tables + (S + 1);
  build_tables<RATIO>(p, item_start, row_start);
  const int32_t total = uniform(item_start[S]);

  for (int32_t pass = 0;; ++pass) {
    const int32_t item = pass_item(pass, wave0, nwaves, total);
    if (item < 0) break;
    int lo = 0, hi = S;                          // item_start[lo] <= item < item_start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (uniform(item_start[mid]) <= item) lo = mid; else hi = mid;
    }
    const int32_t b = lo;
    const int32_t lat0 = uniform(row_start[b]);
    run_tile<L, RATIO, kTileRows>(p, kv, w, b, item - uniform(item_start[b]), lat0,
                                  uniform(row_start[b + 1]) - lat0, ld_ro(p.offsets + b),
                                  ld_ro(p.offsets + S + b), ld_ro(p.start_pos + b));
  }
}

// Decode and verify: one wave per slot takes the slot's D tokens (D = 1 for
// decode) in order, as D single decode tokens.  Rows first: a ratio-2 token
// at an odd position pools with the previous draft token, or for the first
// token with the ring entry an earlier call left; the ring entries are
// written after every row of the slot has read its inputs.  SPLIT (ratio 1,
// or ring_slots > D / 2): the pairs of one call then span fewer ring entries
// than the ring has, so no ring write can reach the entry the first row
// reads, and each row takes a wave of its own.
template <int L, int RATIO, bool SPLIT>
__global__ __launch_bounds__(kBlock) void compress_tokens_kernel(CompressParams p) {
  const PagedKV<L> kv{p.cache.base, p.cache.page_stride, p.cache.num_pages, p.cache.page_bits};
  const int lane = lane_id();
  // SPLIT: wave r of a slot takes the slot's row r alone (and wave 0 the
  // last pending token); otherwise one wave takes all of the slot's rows
  const int32_t per_slot = SPLIT ? (RATIO == 2 ? (p.draft_len + 1) >> 1 : p.draft_len) : 1;
  const int64_t w64 = uniform64((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (w64 >= (int64_t)p.num_slots * per_slot) return;
  const int32_t b = (int32_t)(w64 / per_slot);
  const int32_t r_only = (int32_t)(w64 - (int64_t)b * per_slot);
  const int64_t P = ld_ro(p.start_pos + b);
  if (P < 0) return;
  const int32_t D = p.draft_len;
  const int64_t t0 = (int64_t)b * D;
  const uint4 wr = ld_u4(p.norm_w + kDimsPerLane * lane);
  const float w[8] = {bf16_lo(wr.x), bf16_hi(wr.x), bf16_lo(wr.y), bf16_hi(wr.y),
                      bf16_lo(wr.z), bf16_hi(wr.z), bf16_lo(wr.w), bf16_hi(wr.w)};
  // the slot's rows two at a time, the loads of both issued before either
  // is computed
  auto job = [&](int32_t jj) {
    const int64_t q = P + jj;
    RowJob r;
    r.t1 = (int32_t)(t0 + jj);
    r.latent_idx = (int32_t)(t0 + jj);
    r.from_state = RATIO == 2 && jj == 0;
    r.st_row = r.from_state ? ring_row(p, b, (int32_t)(q >> 1)) : 0;
    r.rot_pos = sat_pos(RATIO == 2 ? q - 1 : q);
    // destination: the caller's out_loc (0 = padded row) or the page table
    if (p.out_loc != nullptr) {
      r.loc = ld_ro(p.out_loc + t0 + jj);
      r.loc_err = 0;
    } else {
      const int64_t c = RATIO == 2 ? (q >> 1) : q;
      if (c > 0x7FFFFFFF) {
        r.loc = 0;
        r.loc_err = kStPtRange;
      } else {
        dest_loc(p, b, (int32_t)c, r.loc, r.loc_err);
      }
    }
    return r;
  };
  // Pending tokens (ratio 2): an even position's token becomes the pending
  // token of its pair, unless a later token of this call takes the same ring
  // entry.  A token followed by the odd token of its pair is already in that
  // row's registers (its first token) and is written from there after the
  // row; a last token at an even position is loaded up front and written at
  // the end.  Every ring write follows the row that reads the ring.
  const int64_t last_pair = (P + D - 1) >> 1;
  const bool tail = RATIO == 2 && ((P + D - 1) & 1) == 0 && (!SPLIT || r_only == 0);
  uint4 tail_kv = make_uint4(0u, 0u, 0u, 0u), tail_sc = tail_kv;
  if (tail) {
    const int dim0 = kDimsPerLane * lane;
    tail_kv = ld_u4_nt(p.kv + (t0 + D - 1) * p.kv_stride + dim0);
    tail_sc = ld_u4_nt(p.score + (t0 + D - 1) * p.score_stride + dim0);
  }
  auto pend_from_row = [&](const RowJob& j, const RowIn& in) {
    if constexpr (RATIO == 2) {
      const int64_t q = P + (j.t1 - t0);       // the row's odd position
      const int64_t k = (q - 1) >> 1;
      if (!j.from_state && k + p.ring_slots > last_pair)
        write_state_regs(p, ring_row(p, b, (int32_t)k), in.k0, in.s0);
    }
  };
  // tokens that close a row: every token (ratio 1), odd positions (ratio 2)
  const int32_t first = (RATIO == 2 && (P & 1) == 0) ? 1 : 0;
  const int32_t step = RATIO == 2 ? 2 : 1;
  if constexpr (SPLIT) {
    // this wave's row alone: with more ring entries than pairs in a call,
    // no other row's ring write can touch the entry the first row reads
    const int32_t jj = first + step * r_only;
    if (jj < D) {
      const RowJob j0 = job(jj);
      const RowIn in0 = load_row<RATIO>(p, j0);
      finish_row<L, RATIO>(p, kv, w, j0, in0);
      pend_from_row(j0, in0);
    }
    if (tail) write_state_regs(p, ring_row(p, b, (int32_t)last_pair), tail_kv, tail_sc);
    return;
  }
  for (int32_t jj = first; jj < D; jj += 2 * step) {
    const bool two = jj + step < D;
    const RowJob j0 = job(jj);
    if (two) {
      const RowJob j1 = job(jj + step);
      const RowIn in0 = load_row<RATIO>(p, j0);
      const RowIn in1 = load_row<RATIO>(p, j1);
      finish_row<L, RATIO>(p, kv, w, j0, in0);
      finish_row<L, RATIO>(p, kv, w, j1, in1);
      pend_from_row(j0, in0);
      pend_from_row(j1, in1);
    } else {
      const RowIn in0 = load_row<RATIO>(p, j0);
      finish_row<L, RATIO>(p, kv, w, j0, in0);
      pend_from_row(j0, in0);
    }
  }
  if (tail) write_state_regs(p, ring_row(p, b, (int32_t)last_pair), tail_kv, tail_sc);
}

template <int L, int RATIO>
hipError_t launch_one(const CompressParams& p, hipStream_t stream) {
  if (p.mode == 0) {
    // an upper bound on the work items: full tiles of the latent capacity plus
    // up to two partial tiles (or one tail item) per slot
    const int64_t items_hint = (p.max_out_rows >> p.tile_log2) + 2 * (int64_t)p.num_slots + 1;
    int64_t blocks = (items_hint + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > kMaxPrefillBlocks) blocks = kMaxPrefillBlocks;
    if (blocks < 1) blocks = 1;
    const size_t lds = sizeof(int32_t) * 2 * (size_t)(p.num_slots + 1);
    // up to 256 slots: slot lookup by ballots over 1, 2 or 4 slots per lane
    const int spl = p.num_slots <= kLanes ? 1 : p.num_slots <= 2 * kLanes ? 2
                  : p.num_slots <= 4 * kLanes ? 4 : 0;
#define KVC_PREFILL_LAUNCH(R)                                                                     \
  if (spl == 1)                                                                                   \
    hipLaunchKernelGGL((compress_prefill_small_kernel<L, RATIO, R>), dim3((int)blocks),           \
                       dim3(kBlock), 0, stream, p);                                               \
  else if (spl == 2)                                                                              \
    hipLaunchKernelGGL((compress_prefill_multi_kernel<L, RATIO, R, 2>), dim3((int)blocks),        \
                       dim3(kBlock), 0, stream, p);                                               \
  else if (spl == 4)                                                                              \
    hipLaunchKernelGGL((compress_prefill_multi_kernel<L, RATIO, R, 4>), dim3((int)blocks),        \
                       dim3(kBlock), 0, stream, p);                                               \
  else                                                                                            \
    hipLaunchKernelGGL((compress_prefill_kernel<L, RATIO, R>), dim3((int)blocks), dim3(kBlock),  \
                       lds, stream, p);
    switch (p.tile_log2) {
      case 0: KVC_PREFILL_LAUNCH(1) break;
      case 1: KVC_PREFILL_LAUNCH(2) break;
      default: KVC_PREFILL_LAUNCH(4) break;
    }
#undef KVC_PREFILL_LAUNCH
  } else {
    // rows of a slot in waves of their own when the ring has more entries
    // than a call's pairs (ratio 2) -- the rows are then independent
    const bool split = p.draft_len > 1 && (RATIO == 1 || 2 * p.ring_slots > p.draft_len);
    const int64_t per_slot = split ? (RATIO == 2 ? (p.draft_len + 1) / 2 : p.draft_len) : 1;
    const int blocks = (int)(((int64_t)p.num_slots * per_slot + kWavesPerBlock - 1) / kWavesPerBlock);
    if (split)
      hipLaunchKernelGGL((compress_tokens_kernel<L, RATIO, true>), dim3(blocks), dim3(kBlock), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((compress_tokens_kernel<L, RATIO, false>), dim3(blocks), dim3(kBlock), 0,
                         stream, p);
  }
  return hipGetLastError();
}

template <int L>
hipError_t launch_layout(const CompressParams& p, hipStream_t stream) {
  return p.ratio == 1 ? launch_one<L, 1>(p, stream) : launch_one<L, 2>(p, stream);
}

}  // namespace

int max_prefill_slots() { return kMaxPrefillSlots; }

hipError_t launch_compress(const CompressParams& p_in, hipStream_t stream) {
  CompressParams p = p_in;
  // rows per work item: the caller's 1, 2 or 4, else by batch size; no more
  // than a page
  int tl = p.tile_rows == 1 ? 0 : p.tile_rows == 2 ? 1 : p.tile_rows == 4 ? 2
           : p.max_out_rows <= kSmallBatchRows ? 0 : kTileLog2;
  p.tile_log2 = tl < p.cache.page_bits ? tl : p.cache.page_bits;
  switch (p.cache.layout) {
    case kV41: return launch_layout<kV41>(p, stream);
    case kV41Fp4: return launch_layout<kV41Fp4>(p, stream);
    default: return launch_layout<kV4>(p, stream);
  }
}

}  // namespace kvc
