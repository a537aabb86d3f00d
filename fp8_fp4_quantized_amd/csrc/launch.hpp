// launch.hpp -- parameter blocks and launchers shared by the C ABI and the
// kernel translation units (host-side declarations only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// Division of a uint32 by an invariant d >= 1 as a multiply-high and shifts
// (the round-down method for unsigned invariant divisors of Granlund and
// Montgomery, 1994): with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
// q = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0), t = mulhi(m, n).
struct DivMagic {
  uint32_t m;
  int32_t sh1, sh2;
};

inline DivMagic div_magic(uint32_t d) {
  int l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  DivMagic r;
  r.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  r.sh1 = l < 1 ? l : 1;
  r.sh2 = l > 1 ? l - 1 : 0;
  return r;
}

struct CacheView {
  uint8_t* base;
  int64_t page_stride;
  int64_t num_pages;
  int32_t page_bits;
  int32_t layout;
};

struct StoreParams {
  CacheView cache;
  const uint16_t* rows;
  int64_t row_stride;          // elements
  const int32_t* out_loc;
  int64_t n;
  int32_t* status;
  const int32_t* positions;    // rotary positions (NULL: plain store)
  const float* freqs;          // [max_pos, 64]
  int64_t max_pos;
};

struct DcpFilterParams {
  const int32_t* ids;
  int64_t T;
  int32_t k;
  int64_t ids_stride;
  const int32_t* token_to_req;
  int32_t n_req;
  const int32_t* block_table;
  int64_t bt_stride;           // entries between block-table rows
  int64_t bt_width;            // valid entries per row (the bound)
  const int32_t* valid;        // nullable
  int32_t page_bits;
  int64_t num_pages;
  int32_t world;
  DivMagic world_div;
  int32_t world_log2;          // log2(world) for a power of two, else -1
  int32_t rank;
  int32_t interleave_log2;
  int32_t* out_slots;
  int64_t out_stride;
  int32_t* out_lens;
  int32_t* status;
};

struct GatherParams {
  CacheView cache;
  const int32_t* page_table;   // nullable
  int64_t n_pages;
  const int32_t* ids;
  int64_t n;
  uint16_t* out;
  int64_t out_stride;          // elements
  int32_t* status;
  int32_t batch;               // ids a wave resolves at once: 8, 16 or 32 (set by the launcher)
};

struct CompressParams {
  CacheView cache;
  int32_t ratio;
  int32_t mode;                // 0 prefill, 1 decode, 2 verify
  const uint16_t* kv;
  int64_t kv_stride;
  const uint16_t* score;
  int64_t score_stride;
  int64_t kv_rows;             // token rows kv and score hold
  int32_t num_slots;
  const int32_t* offsets;
  const int32_t* start_pos;
  const int32_t* page_table;
  int64_t pt_stride;           // entries between page-table rows
  int64_t pt_width;            // valid entries per row (the bound)
  const int32_t* out_loc;
  uint16_t* state;
  const uint16_t* norm_w;
  float eps;
  const float* freqs;
  int64_t max_pos;
  uint16_t* latent;
  int64_t latent_stride;
  int64_t max_out_rows;
  uint16_t* prequant;
  int64_t prequant_stride;
  int32_t* status;
  int32_t draft_len;           // tokens per slot in decode / verify (decode: 1)
  int32_t ring_slots;          // pending-state entries per slot (>= 1)
  int32_t dcp_world;           // context-parallel ranks (1: none)
  DivMagic dcp_div;            // division by dcp_world
  int32_t dcp_rank;
  int32_t dcp_interleave_log2; // log2 of the rows per rank turn
  int32_t tile_rows;           // prefill rows per work item: 1, 2, 4 (0: by batch size)
  int32_t tile_log2;           // set by the launcher: log2 of rows per prefill work item
};

// Each launcher enqueues one kernel on `stream` and returns the HIP error of
// the launch (hipSuccess on success).
hipError_t launch_store_rows(const StoreParams& p, hipStream_t stream);
hipError_t launch_dequant_gather(const GatherParams& p, hipStream_t stream);
hipError_t launch_compress(const CompressParams& p, hipStream_t stream);
hipError_t launch_dcp_filter(const DcpFilterParams& p, hipStream_t stream);

// largest num_slots a prefill compress accepts (its LDS tables)
int max_prefill_slots();

}  // namespace kvc
