// compress.hip -- the fused ratio-1 / ratio-2 compressor (gfx950).
//
// One 64-lane wave makes one compressed row: it loads the pair's kv and score
// rows (16 B per lane each), pools them with a per-dim softmax over the two
// scores (ratio 2), RMS-normalises over the 512 dims (one wave sum), writes
// the pre-RoPE latent, rotates the 64 rope dims (lanes 56..63, four pairs per
// lane, no cross-lane traffic), rounds to bf16 and quantizes the row into its
// paged slot.  (sglang PR #39652 "dsv4.1: compression, KV I/O, and metadata
// kernels", Summary and Review; sglang PR #46230, summary.)
//
// Prefill batches are ragged: each workgroup turns the int32 [2, S] extend
// offsets into per-slot work and latent starts with a scan in LDS, then its
// waves look their work items up by binary search, so the launch needs no
// host-side knowledge of the row counts (and can be captured in a graph).
#include "launch.hpp"
#include "row_ops.hpp"

namespace kvc {

namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kLanes;
constexpr int kMaxPrefillSlots = 8191;   // two LDS tables of S + 1 ints fit in 64 KiB

__device__ __forceinline__ void raise_status(int32_t* status, int32_t bit) {
  if (status != nullptr && lane_id() == 0) atomicOr(status, bit);
}

struct RowJob {
  const uint16_t* k0;     // first token of the pair (ratio 2)
  const uint16_t* s0;
  const uint16_t* k1;     // second (or only) token
  const uint16_t* s1;
  int64_t rot_pos;        // rotary position
  int64_t c;              // compressed row index within the slot
  int32_t slot;
  int64_t latent_idx;
};

template <int L, int RATIO, int MODE>
__device__ __forceinline__ void compress_row(const CompressParams& p, const PagedKV<L>& kv,
                                             const float (&w)[8], const RowJob& j) {
  const int lane = lane_id();
  if (j.rot_pos < 0 || j.rot_pos >= p.max_pos) {
    raise_status(p.status, kStPosRange);
    return;
  }
  // ---- loads: the pair's rows and this lane's slice of the rotary table
  const int dim0 = kDimsPerLane * lane;
  const uint4 xk1 = ld_u4_nt(j.k1 + dim0);
  uint4 xk0 = make_uint4(0u, 0u, 0u, 0u), xs0 = xk0, xs1 = xk0;
  if constexpr (RATIO == 2) {
    xk0 = ld_u4_nt(j.k0 + dim0);
    xs0 = ld_u4_nt(j.s0 + dim0);
    xs1 = ld_u4_nt(j.s1 + dim0);
  }
  float4 f0 = make_float4(1.f, 0.f, 1.f, 0.f), f1 = f0;
  if (lane >= kRopeLane0) {
    const float* fr = p.freqs + j.rot_pos * kRope + kDimsPerLane * (lane - kRopeLane0);
    f0 = *(const float4*)fr;
    f1 = *(const float4*)(fr + 4);
  }

  // ---- pooling (ratio 2): softmax over the two scores, per dim
  const uint32_t k1w[4] = {xk1.x, xk1.y, xk1.z, xk1.w};
  float v[8];
  if constexpr (RATIO == 2) {
    const uint32_t k0w[4] = {xk0.x, xk0.y, xk0.z, xk0.w};
    const uint32_t s0w[4] = {xs0.x, xs0.y, xs0.z, xs0.w};
    const uint32_t s1w[4] = {xs1.x, xs1.y, xs1.z, xs1.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float a0 = h ? bf16_hi(s0w[q]) : bf16_lo(s0w[q]);
        const float a1 = h ? bf16_hi(s1w[q]) : bf16_lo(s1w[q]);
        const float kk0 = h ? bf16_hi(k0w[q]) : bf16_lo(k0w[q]);
        const float kk1 = h ? bf16_hi(k1w[q]) : bf16_lo(k1w[q]);
        const float m = fmaxf(a0, a1);
        const float e0 = __expf(a0 - m), e1 = __expf(a1 - m);
        v[2 * q + h] = (e0 * kk0 + e1 * kk1) * __builtin_amdgcn_rcpf(e0 + e1);
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

  // ---- pre-RoPE latent
  const uint4 lat = make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]),
                               pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7]));
  const bool lat_ok = j.latent_idx < p.max_out_rows;
  if (lat_ok) {
    st_u4(p.latent + j.latent_idx * p.latent_stride + dim0, lat);
  } else {
    raise_status(p.status, kStLatentRange);
  }

  // ---- RoPE on the last 64 dims: pairs (2i, 2i+1) times (cos, sin)
  uint4 z = lat;
  if (lane >= kRopeLane0) {
    const float cs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    float o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = y[2 * i], b = y[2 * i + 1], c = cs[2 * i], s = cs[2 * i + 1];
      o[2 * i] = a * c - b * s;
      o[2 * i + 1] = a * s + b * c;
    }
    z = make_uint4(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]),
                   pack_bf16(o[6], o[7]));
  }
  if (p.prequant != nullptr && lat_ok) st_u4(p.prequant + j.latent_idx * p.prequant_stride + dim0, z);

  // ---- destination slot (out_loc == 0: padded row, no write)
  int64_t loc;
  bool write = true;
  if (MODE == 1 && p.out_loc != nullptr) {
    loc = uniform(p.out_loc[j.slot]);
  } else {
    const int64_t lp = j.c >> p.cache.page_bits;
    if (lp >= p.pt_stride) {
      raise_status(p.status, kStPtRange);
      write = false;
      loc = 0;
    } else {
      const int64_t phys = uniform(p.page_table[(int64_t)j.slot * p.pt_stride + lp]);
      if (phys < 0 || phys >= kv.num_pages) {
        raise_status(p.status, kStPageRange);
        write = false;
        loc = 0;
      } else {
        loc = (phys << p.cache.page_bits) | (j.c & ((int64_t(1) << p.cache.page_bits) - 1));
      }
    }
  }
  if (write && loc == 0) write = false;
  if (write && !kv.valid(loc)) {
    raise_status(p.status, kStPageRange);
    write = false;
  }
  const int64_t slot = write ? loc : 0;
  store_row_wave<L>(z, kv.data(slot), kv.scale(slot), write);
}

// copy a token's kv and score rows into the slot's pending state
__device__ __forceinline__ void write_state(const CompressParams& p, int32_t b, int64_t tok) {
  const int dim0 = kDimsPerLane * lane_id();
  uint16_t* st = p.state + (int64_t)b * 2 * kDim;
  const uint4 kvv = ld_u4_nt(p.kv + tok * p.kv_stride + dim0);
  const uint4 scv = ld_u4_nt(p.score + tok * p.score_stride + dim0);
  st_u4(st + dim0, kvv);
  st_u4(st + kDim + dim0, scv);
}

// per-slot work of a prefill batch: compressed rows, and whether the last
// token becomes the pending state (ratio 2); a slot with a tail and rows does
// the tail in its first work item, after that item has read the old state
struct SlotWork {
  int32_t rows, items;
  bool tail;
};
template <int RATIO>
__device__ __forceinline__ SlotWork slot_work(int32_t n, int32_t P) {
  SlotWork s{0, 0, false};
  if (n <= 0 || P < 0) return s;
  if constexpr (RATIO == 1) {
    s.rows = n;
    s.items = n;
  } else {
    s.rows = ((P + n) >> 1) - (P >> 1);      // odd positions in [P, P + n)
    s.tail = ((P + n) & 1) != 0;             // last position P + n - 1 is even
    s.items = s.rows > 0 ? s.rows : (s.tail ? 1 : 0);
  }
  return s;
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
    SlotWork sw{0, 0, false};
    if (b < S) sw = slot_work<RATIO>(p.offsets[S + b], p.start_pos[b]);
    int32_t si = sw.items, sr = sw.rows;
#pragma unroll
    for (int d = 1; d < kLanes; d <<= 1) {
      const int32_t ti = __shfl_up(si, d), tr = __shfl_up(sr, d);
      if (lane >= d) {
        si += ti;
        sr += tr;
      }
    }
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

template <int L, int RATIO, int MODE>
__global__ __launch_bounds__(kBlock) void compress_kernel(CompressParams p) {
  extern __shared__ int32_t tables[];
  const PagedKV<L> kv{p.cache.base, p.cache.page_stride, p.cache.num_pages, p.cache.page_bits};
  const int lane = lane_id();
  const uint4 wr = ld_u4(p.norm_w + kDimsPerLane * lane);
  const float w[8] = {bf16_lo(wr.x), bf16_hi(wr.x), bf16_lo(wr.y), bf16_hi(wr.y),
                      bf16_lo(wr.z), bf16_hi(wr.z), bf16_lo(wr.w), bf16_hi(wr.w)};
  const int64_t wave0 = uniform64((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int S = p.num_slots;

  if constexpr (MODE == 0) {
    int32_t* item_start = tables;
    int32_t* row_start = tables + (S + 1);
    build_tables<RATIO>(p, item_start, row_start);
    const int64_t total = item_start[S];
    for (int64_t item = wave0; item < total; item += nwaves) {
      int lo = 0, hi = S;                        // item_start[lo] <= item < item_start[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (item_start[mid] <= item) lo = mid; else hi = mid;
      }
      const int32_t b = uniform(lo);
      const int64_t k = item - uniform(item_start[b]);
      const int32_t rows = uniform(row_start[b + 1]) - uniform(row_start[b]);
      const int64_t first = uniform(p.offsets[b]);
      const int32_t n = uniform(p.offsets[S + b]);
      const int64_t P = uniform(p.start_pos[b]);
      RowJob j;
      j.slot = b;
      j.latent_idx = uniform(row_start[b]) + k;
      if constexpr (RATIO == 1) {
        j.k0 = j.s0 = nullptr;
        j.k1 = p.kv + (first + k) * p.kv_stride;
        j.s1 = nullptr;
        j.c = P + k;
        j.rot_pos = P + k;
        compress_row<L, RATIO, MODE>(p, kv, w, j);
      } else {
        if (k < rows) {
          const int64_t q = (P | 1) + 2 * k;     // odd position closing the pair
          const int64_t t1 = first + (q - P);
          j.k1 = p.kv + t1 * p.kv_stride;
          j.s1 = p.score + t1 * p.score_stride;
          if (q - 1 >= P) {
            j.k0 = j.k1 - p.kv_stride;
            j.s0 = j.s1 - p.score_stride;
          } else {                               // first token is the pending state
            j.k0 = p.state + (int64_t)b * 2 * kDim;
            j.s0 = j.k0 + kDim;
          }
          j.c = q >> 1;
          j.rot_pos = q - 1;
          compress_row<L, RATIO, MODE>(p, kv, w, j);
        }
        if (k == 0 && ((P + n) & 1)) write_state(p, b, first + n - 1);
      }
    }
  } else {
    const int64_t b64 = wave0;
    if (b64 >= S) return;
    const int32_t b = (int32_t)b64;
    const int64_t pos = uniform(p.start_pos[b]);
    if (pos < 0) return;
    RowJob j;
    j.slot = b;
    j.latent_idx = b;
    j.k1 = p.kv + (int64_t)b * p.kv_stride;
    if constexpr (RATIO == 1) {
      j.k0 = j.s0 = j.s1 = nullptr;
      j.c = pos;
      j.rot_pos = pos;
      compress_row<L, RATIO, MODE>(p, kv, w, j);
    } else {
      j.s1 = p.score + (int64_t)b * p.score_stride;
      if (pos & 1) {
        j.k0 = p.state + (int64_t)b * 2 * kDim;
        j.s0 = j.k0 + kDim;
        j.c = pos >> 1;
        j.rot_pos = pos - 1;
        compress_row<L, RATIO, MODE>(p, kv, w, j);
      } else {
        write_state(p, b, b);
      }
    }
  }
}

template <int L, int RATIO, int MODE>
hipError_t launch_one(const CompressParams& p, hipStream_t stream) {
  int blocks;
  size_t lds = 0;
  if (MODE == 0) {
    const int64_t items_hint = p.max_out_rows + p.num_slots;
    int64_t b = (items_hint + kWavesPerBlock - 1) / kWavesPerBlock;
    const int cap = launch_tuning().compress_blocks > 0 ? launch_tuning().compress_blocks : 4096;
    if (b > cap) b = cap;
    blocks = (int)(b < 1 ? 1 : b);
    lds = sizeof(int32_t) * 2 * (size_t)(p.num_slots + 1);
  } else {
    blocks = (p.num_slots + kWavesPerBlock - 1) / kWavesPerBlock;
  }
  hipLaunchKernelGGL((compress_kernel<L, RATIO, MODE>), dim3(blocks), dim3(kBlock), lds, stream, p);
  return hipGetLastError();
}

template <int L>
hipError_t launch_layout(const CompressParams& p, hipStream_t stream) {
  if (p.ratio == 1) {
    return p.mode == 0 ? launch_one<L, 1, 0>(p, stream) : launch_one<L, 1, 1>(p, stream);
  }
  return p.mode == 0 ? launch_one<L, 2, 0>(p, stream) : launch_one<L, 2, 1>(p, stream);
}

}  // namespace

int max_prefill_slots() { return kMaxPrefillSlots; }

hipError_t launch_compress(const CompressParams& p, hipStream_t stream) {
  switch (p.cache.layout) {
    case kV41: return launch_layout<kV41>(p, stream);
    case kV41Fp4: return launch_layout<kV41Fp4>(p, stream);
    default: return launch_layout<kV4>(p, stream);
  }
}

}  // namespace kvc
