// kvc_api.cpp -- the C ABI (include/kvc.h): argument checks from host
// scalars, dispatch to the kernel launchers, error strings and the host-side
// dequant-reuse head.  Nothing here touches device memory or synchronises.
#include "../../include/kvc.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <new>
#include <cstring>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return KVC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool layout_info(int32_t layout, kvc_layout_info* info) {
  switch (layout) {
    case KVC_LAYOUT_V4: *info = {576, 8, 584, 64, 448}; return true;
    case KVC_LAYOUT_V41: *info = {512, 16, 528, 32, 512}; return true;
    case KVC_LAYOUT_V41_FP4: *info = {256, 32, 288, 16, 512}; return true;
    default: return false;
  }
}

int page_bits_of(int32_t page_size) {
  int b = 0;
  while ((1 << b) < page_size) ++b;
  return b;
}

// checks the cache descriptor and fills the device view
int check_cache(const kvc_cache* c, kvc::CacheView* v, const char* who) {
  if (c == nullptr) return fail(KVC_EINVAL, "%s: cache descriptor is NULL", who);
  kvc_layout_info li;
  if (!layout_info(c->layout, &li)) return fail(KVC_EUNSUPPORTED, "%s: unknown layout %d", who, c->layout);
  if (c->base == nullptr) return fail(KVC_EINVAL, "%s: cache base is NULL", who);
  if (!aligned16(c->base)) return fail(KVC_EINVAL, "%s: cache base is not 16-byte aligned", who);
  if (c->page_size < 1 || c->page_size > 4096 || (c->page_size & (c->page_size - 1)) != 0)
    return fail(KVC_EINVAL, "%s: page_size %d is not a power of two in [1, 4096]", who, c->page_size);
  if (c->page_stride < (int64_t)c->page_size * li.row_bytes || c->page_stride % 16 != 0)
    return fail(KVC_EINVAL, "%s: page_stride %lld must be >= page_size * %d and a multiple of 16",
                who, (long long)c->page_stride, li.row_bytes);
  if (c->num_pages < 1) return fail(KVC_EINVAL, "%s: num_pages must be >= 1", who);
  if (c->num_pages > ((int64_t)1 << 31) / c->page_size)
    return fail(KVC_EINVAL, "%s: num_pages * page_size must fit in int32 slots", who);
  v->base = static_cast<uint8_t*>(c->base);
  v->page_stride = c->page_stride;
  v->num_pages = c->num_pages;
  v->page_bits = page_bits_of(c->page_size);
  v->layout = c->layout;
  return KVC_OK;
}

bool row_stride_ok(int64_t s) { return s >= 512 && s % 8 == 0; }

int launched(hipError_t e, const char* who) {
  if (e != hipSuccess) return fail(KVC_ELAUNCH, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // namespace

// --------------------------------------------------------------------------
struct kvc_kvbuf {
  bool valid;
  void* base;
  int32_t layout;
  int32_t page_size;
  int64_t page_stride;
  const int32_t* page_table;
  int64_t n_pages;
  const int32_t* ids;
  int64_t n;
  void* out;
  int64_t out_stride;
};

extern "C" {

int kvc_version(void) { return 3; }

const char* kvc_last_error(void) { return g_last_error.c_str(); }

int kvc_layout_query(int32_t layout, kvc_layout_info* info) {
  if (info == nullptr) return fail(KVC_EINVAL, "kvc_layout_query: info is NULL");
  if (!layout_info(layout, info)) return fail(KVC_EUNSUPPORTED, "kvc_layout_query: unknown layout %d", layout);
  return ok();
}

int kvc_store_rows(const kvc_cache* cache, const void* rows_bf16, int64_t row_stride,
                   const int32_t* out_loc, int64_t n, int32_t* status, void* stream) {
  const char* who = "kvc_store_rows";
  kvc::StoreParams p{};
  int rc = check_cache(cache, &p.cache, who);
  if (rc) return rc;
  if (n < 0) return fail(KVC_EINVAL, "%s: n < 0", who);
  if (n == 0) return ok();
  if (rows_bf16 == nullptr || out_loc == nullptr) return fail(KVC_EINVAL, "%s: NULL rows or out_loc", who);
  if (!aligned16(rows_bf16) || !row_stride_ok(row_stride))
    return fail(KVC_EINVAL, "%s: rows must be 16-byte aligned with row_stride >= 512, a multiple of 8", who);
  p.rows = static_cast<const uint16_t*>(rows_bf16);
  p.row_stride = row_stride;
  p.out_loc = out_loc;
  p.n = n;
  p.status = status;
  return launched(kvc::launch_store_rows(p, static_cast<hipStream_t>(stream)), who);
}

int kvc_store_rows_rope(const kvc_cache* cache, const void* rows_bf16, int64_t row_stride,
                        const int32_t* positions, const float* freqs, int64_t max_pos,
                        const int32_t* out_loc, int64_t n, int32_t* status, void* stream) {
  const char* who = "kvc_store_rows_rope";
  kvc::StoreParams p{};
  int rc = check_cache(cache, &p.cache, who);
  if (rc) return rc;
  if (n < 0) return fail(KVC_EINVAL, "%s: n < 0", who);
  if (n == 0) return ok();
  if (rows_bf16 == nullptr || out_loc == nullptr || positions == nullptr)
    return fail(KVC_EINVAL, "%s: NULL rows, out_loc or positions", who);
  if (!aligned16(rows_bf16) || !row_stride_ok(row_stride))
    return fail(KVC_EINVAL, "%s: rows must be 16-byte aligned with row_stride >= 512, a multiple of 8", who);
  if (freqs == nullptr || !aligned16(freqs) || max_pos < 1)
    return fail(KVC_EINVAL, "%s: freqs must be non-NULL, 16-byte aligned, max_pos >= 1", who);
  p.rows = static_cast<const uint16_t*>(rows_bf16);
  p.row_stride = row_stride;
  p.out_loc = out_loc;
  p.n = n;
  p.status = status;
  p.positions = positions;
  p.freqs = freqs;
  p.max_pos = max_pos;
  return launched(kvc::launch_store_rows(p, static_cast<hipStream_t>(stream)), who);
}

int kvc_dcp_filter_ids(const int32_t* ids, int64_t T, int32_t k, int64_t ids_stride,
                       const int32_t* token_to_req, int32_t n_req, const int32_t* block_table,
                       int64_t bt_stride, int64_t bt_width, const int32_t* valid, int32_t page_size,
                       int64_t num_pages, int32_t world, int32_t rank, int32_t interleave,
                       int32_t* out_slots, int64_t out_stride, int32_t* out_lens,
                       int32_t* status, void* stream) {
  const char* who = "kvc_dcp_filter_ids";
  if (T < 0 || k < 0 || k > 65536) return fail(KVC_EINVAL, "%s: T < 0 or k outside [0, 65536]", who);
  if (T == 0) return ok();
  if (page_size < 1 || page_size > 4096 || (page_size & (page_size - 1)) != 0)
    return fail(KVC_EINVAL, "%s: page_size %d is not a power of two in [1, 4096]", who, page_size);
  if (world < 1 || world > 1024 || rank < 0 || rank >= world)
    return fail(KVC_EINVAL, "%s: world %d / rank %d (1 <= world <= 1024, 0 <= rank < world)", who,
                world, rank);
  if (interleave < 1 || page_size % interleave != 0)
    return fail(KVC_EINVAL, "%s: interleave %d must be >= 1 and divide page_size %d", who,
                interleave, page_size);
  if (token_to_req == nullptr || out_lens == nullptr)
    return fail(KVC_EINVAL, "%s: NULL token_to_req or out_lens", who);
  if (k > 0 && (ids == nullptr || out_slots == nullptr || ids_stride < k || out_stride < k))
    return fail(KVC_EINVAL, "%s: NULL ids or out_slots, or a row stride below k", who);
  if (k > 0 && ((uintptr_t)out_slots & 3u) != 0)
    return fail(KVC_EINVAL, "%s: out_slots is not 4-byte aligned", who);
  if (n_req < 0 || (n_req > 0 && (block_table == nullptr || bt_width < 1 || bt_stride < bt_width)))
    return fail(KVC_EINVAL, "%s: n_req < 0, or no block table, or not 1 <= bt_width <= bt_stride",
                who);
  if (num_pages < 1 || num_pages > ((int64_t)1 << 31) / page_size)
    return fail(KVC_EINVAL, "%s: num_pages must be >= 1 with num_pages * page_size in int32", who);
  kvc::DcpFilterParams p{};
  p.ids = ids;
  p.T = T;
  p.k = k;
  p.ids_stride = ids_stride;
  p.token_to_req = token_to_req;
  p.n_req = n_req;
  p.block_table = block_table;
  p.bt_stride = bt_stride;
  p.bt_width = bt_width;
  p.valid = valid;
  p.page_bits = page_bits_of(page_size);
  p.num_pages = num_pages;
  p.world = world;
  p.world_div = kvc::div_magic((uint32_t)world);
  p.world_log2 = -1;
  if ((world & (world - 1)) == 0) {
    p.world_log2 = 0;
    while ((1 << p.world_log2) < world) ++p.world_log2;
  }
  p.rank = rank;
  p.interleave_log2 = page_bits_of(interleave);
  p.out_slots = out_slots;
  p.out_stride = out_stride;
  p.out_lens = out_lens;
  p.status = status;
  return launched(kvc::launch_dcp_filter(p, static_cast<hipStream_t>(stream)), who);
}

int kvc_dequant_gather(const kvc_cache* cache, const int32_t* page_table, int64_t n_pages,
                       const int32_t* ids, int64_t n, void* out_bf16, int64_t out_row_stride,
                       int32_t* status, void* stream) {
  const char* who = "kvc_dequant_gather";
  kvc::GatherParams p{};
  int rc = check_cache(cache, &p.cache, who);
  if (rc) return rc;
  if (n < 0) return fail(KVC_EINVAL, "%s: n < 0", who);
  if (n == 0) return ok();
  if (ids == nullptr || out_bf16 == nullptr) return fail(KVC_EINVAL, "%s: NULL ids or output", who);
  if (page_table != nullptr && n_pages < 1) return fail(KVC_EINVAL, "%s: page table with n_pages < 1", who);
  if (!aligned16(out_bf16) || !row_stride_ok(out_row_stride) || out_row_stride > (1 << 25))
    return fail(KVC_EINVAL, "%s: output must be 16-byte aligned with out_row_stride in [512, 2^25], "
                            "a multiple of 8", who);
  p.page_table = page_table;
  p.n_pages = page_table ? n_pages : 0;
  p.ids = ids;
  p.n = n;
  p.out = static_cast<uint16_t*>(out_bf16);
  p.out_stride = out_row_stride;
  p.status = status;
  return launched(kvc::launch_dequant_gather(p, static_cast<hipStream_t>(stream)), who);
}

int kvc_compress_store(const kvc_compress_args* a, void* stream) {
  const char* who = "kvc_compress_store";
  if (a == nullptr) return fail(KVC_EINVAL, "%s: args is NULL", who);
  kvc::CompressParams p{};
  int rc = check_cache(&a->cache, &p.cache, who);
  if (rc) return rc;
  if (a->ratio != 1 && a->ratio != 2) return fail(KVC_EUNSUPPORTED, "%s: ratio %d (1 or 2)", who, a->ratio);
  if (a->mode != KVC_MODE_PREFILL && a->mode != KVC_MODE_DECODE && a->mode != KVC_MODE_VERIFY)
    return fail(KVC_EUNSUPPORTED, "%s: mode %d", who, a->mode);
  if (a->mode == KVC_MODE_VERIFY && (a->draft_len < 1 || a->draft_len > 64))
    return fail(KVC_EINVAL, "%s: verify draft_len %d outside [1, 64]", who, a->draft_len);
  if (a->ring_slots < 0 || a->ring_slots > 1024)
    return fail(KVC_EINVAL, "%s: ring_slots %d outside [0, 1024]", who, a->ring_slots);
  const int32_t world = a->dcp_world > 1 ? a->dcp_world : 1;
  if (a->dcp_world < 0 || world > 1024 || a->dcp_rank < 0 || a->dcp_rank >= world)
    return fail(KVC_EINVAL, "%s: dcp_world %d / dcp_rank %d (world <= 1024, 0 <= rank < world)",
                who, a->dcp_world, a->dcp_rank);
  if (world > 1 && (a->dcp_interleave < 1 || a->cache.page_size % a->dcp_interleave != 0))
    return fail(KVC_EINVAL, "%s: dcp_interleave %d must be >= 1 and divide page_size %d", who,
                a->dcp_interleave, a->cache.page_size);
  if (a->num_slots < 0) return fail(KVC_EINVAL, "%s: num_slots < 0", who);
  if (a->tile_rows != 0 && a->tile_rows != 1 && a->tile_rows != 2 && a->tile_rows != 4)
    return fail(KVC_EINVAL, "%s: tile_rows %d (0, 1, 2 or 4)", who, a->tile_rows);
  if (a->num_slots == 0) return ok();
  if (a->mode == KVC_MODE_VERIFY && (int64_t)a->num_slots * a->draft_len > 0x7FFFFFFF)
    return fail(KVC_EINVAL, "%s: num_slots * draft_len must be below 2^31 (token indices are int32)",
                who);
  if (a->mode == KVC_MODE_PREFILL && a->num_slots > kvc::max_prefill_slots())
    return fail(KVC_EINVAL, "%s: prefill num_slots %d > %d", who, a->num_slots, kvc::max_prefill_slots());
  if (a->kv == nullptr || !aligned16(a->kv) || !row_stride_ok(a->kv_stride))
    return fail(KVC_EINVAL, "%s: kv must be non-NULL, 16-byte aligned, kv_stride >= 512 and a multiple of 8", who);
  {
    // decode / verify read token rows 0 .. num_slots * D - 1; prefill checks
    // each slot's rows against kv_rows on the device
    const int64_t need = a->mode == KVC_MODE_PREFILL ? 1
                       : (int64_t)a->num_slots * (a->mode == KVC_MODE_VERIFY ? a->draft_len : 1);
    if (a->kv_rows < need)
      return fail(KVC_EINVAL, "%s: kv_rows %lld, need at least %lld", who, (long long)a->kv_rows,
                  (long long)need);
  }
  if (a->ratio == 2) {
    if (a->score == nullptr || !aligned16(a->score) || a->score_stride < 512 || a->score_stride % 8)
      return fail(KVC_EINVAL, "%s: ratio 2 needs an aligned score buffer with score_stride >= 512, a multiple of 8", who);
    if (a->state == nullptr || !aligned16(a->state))
      return fail(KVC_EINVAL, "%s: ratio 2 needs a 16-byte aligned pending-state buffer", who);
  }
  if (a->start_pos == nullptr) return fail(KVC_EINVAL, "%s: start_pos is NULL", who);
  if (a->mode == KVC_MODE_PREFILL) {
    if (a->offsets == nullptr) return fail(KVC_EINVAL, "%s: prefill needs offsets", who);
    if (a->page_table == nullptr)
      return fail(KVC_EINVAL, "%s: prefill needs a page table", who);
  } else if (a->out_loc == nullptr && a->page_table == nullptr) {
    return fail(KVC_EINVAL, "%s: decode and verify need out_loc or a page table", who);
  }
  if (a->page_table != nullptr && (a->pt_width < 1 || a->pt_stride < a->pt_width))
    return fail(KVC_EINVAL, "%s: page table needs 1 <= pt_width <= pt_stride (%lld, %lld)", who,
                (long long)a->pt_width, (long long)a->pt_stride);
  if (a->norm_w == nullptr || !aligned16(a->norm_w)) return fail(KVC_EINVAL, "%s: norm_w NULL or misaligned", who);
  if (a->freqs == nullptr || !aligned16(a->freqs) || a->max_pos < 1)
    return fail(KVC_EINVAL, "%s: freqs must be non-NULL, 16-byte aligned, max_pos >= 1", who);
  if (a->latent_out == nullptr || !aligned16(a->latent_out) || !row_stride_ok(a->latent_stride))
    return fail(KVC_EINVAL, "%s: latent_out must be aligned with latent_stride >= 512, a multiple of 8", who);
  if (a->max_out_rows < 0) return fail(KVC_EINVAL, "%s: max_out_rows < 0", who);
  if (a->prequant_out != nullptr && (!aligned16(a->prequant_out) || !row_stride_ok(a->prequant_stride)))
    return fail(KVC_EINVAL, "%s: prequant_out misaligned or bad prequant_stride", who);
  if (!(a->eps >= 0.0f)) return fail(KVC_EINVAL, "%s: eps must be >= 0", who);
  p.ratio = a->ratio;
  p.mode = a->mode;
  p.kv = static_cast<const uint16_t*>(a->kv);
  p.kv_stride = a->kv_stride;
  p.score = static_cast<const uint16_t*>(a->score);
  p.score_stride = a->score_stride;
  p.kv_rows = a->kv_rows;
  p.num_slots = a->num_slots;
  p.offsets = a->offsets;
  p.start_pos = a->start_pos;
  p.page_table = a->page_table;
  p.pt_stride = a->page_table ? a->pt_stride : 0;
  p.pt_width = a->page_table ? a->pt_width : 0;
  p.out_loc = a->mode != KVC_MODE_PREFILL ? a->out_loc : nullptr;
  p.state = static_cast<uint16_t*>(a->state);
  p.norm_w = static_cast<const uint16_t*>(a->norm_w);
  p.eps = a->eps;
  p.freqs = a->freqs;
  p.max_pos = a->max_pos;
  p.latent = static_cast<uint16_t*>(a->latent_out);
  p.latent_stride = a->latent_stride;
  p.max_out_rows = a->max_out_rows;
  p.prequant = static_cast<uint16_t*>(a->prequant_out);
  p.prequant_stride = a->prequant_stride;
  p.status = a->status;
  p.draft_len = a->mode == KVC_MODE_VERIFY ? a->draft_len : 1;
  p.ring_slots = a->ring_slots > 1 ? a->ring_slots : 1;
  p.dcp_world = world;
  p.dcp_div = kvc::div_magic((uint32_t)world);
  p.dcp_rank = world > 1 ? a->dcp_rank : 0;
  p.dcp_interleave_log2 = world > 1 ? page_bits_of(a->dcp_interleave) : 0;
  p.tile_rows = a->tile_rows;
  return launched(kvc::launch_compress(p, static_cast<hipStream_t>(stream)), who);
}

// ---------------------------------------------------------------- reuse head
kvc_kvbuf* kvc_kvbuf_create(void) {
  kvc_kvbuf* kb = new (std::nothrow) kvc_kvbuf;
  if (kb) std::memset(kb, 0, sizeof *kb);
  return kb;
}

void kvc_kvbuf_destroy(kvc_kvbuf* kb) { delete kb; }

void kvc_kvbuf_forget(kvc_kvbuf* kb) {
  if (kb) kb->valid = false;
}

void kvc_kvbuf_begin_forward(kvc_kvbuf* kb) {
  if (kb) kb->valid = false;
}

int kvc_dequant_gather_reuse(kvc_kvbuf* kb, const kvc_cache* cache, const int32_t* page_table,
                             int64_t n_pages, const int32_t* ids, int64_t n, void* out_bf16,
                             int64_t out_row_stride, int32_t* status, int32_t* hit,
                             void* stream) {
  const char* who = "kvc_dequant_gather_reuse";
  if (kb == nullptr || hit == nullptr || cache == nullptr)
    return fail(KVC_EINVAL, "%s: NULL kvbuf, hit or cache", who);
  *hit = 0;
  const int64_t np = page_table ? n_pages : 0;
  if (kb->valid && kb->base == cache->base && kb->layout == cache->layout &&
      kb->page_size == cache->page_size && kb->page_stride == cache->page_stride &&
      kb->page_table == page_table && kb->n_pages == np && kb->ids == ids && kb->n == n &&
      kb->out == out_bf16 && kb->out_stride == out_row_stride) {
    *hit = 1;
    return ok();
  }
  kb->valid = false;
  const int rc = kvc_dequant_gather(cache, page_table, n_pages, ids, n, out_bf16, out_row_stride,
                                    status, stream);
  if (rc != KVC_OK) return rc;
  kb->valid = true;
  kb->base = cache->base;
  kb->layout = cache->layout;
  kb->page_size = cache->page_size;
  kb->page_stride = cache->page_stride;
  kb->page_table = page_table;
  kb->n_pages = np;
  kb->ids = ids;
  kb->n = n;
  kb->out = out_bf16;
  kb->out_stride = out_row_stride;
  return KVC_OK;
}

}  // extern "C"
