/*
 * kvc.h -- C ABI of the MI355X (gfx950) compressed-KV library for the
 * DeepSeek-V4.1 low-ratio (ratio 1 / ratio 2) layers: the fused compressor
 * that pools, normalises, rotates and quantizes latent rows into a paged
 * main-KV cache, and the paged dequant-gather used by sparse prefill.
 *
 * Sources of the operations (web pages; cited by title and section):
 *  - sglang PR #39652 "dsv4.1: compression, KV I/O, and metadata kernels",
 *    Summary: the KVLayout formats V4 (584 B/token), V41 (528 B/token) and
 *    V41_FP4 (288 B/token); one row quantizer for V4.1 rows; shared paged
 *    address arithmetic for every writer; the ratio-1 / ratio-2 compressors
 *    that pool (ratio 2), RMSNorm, RoPE and write the main KV in one launch
 *    and return the pre-RoPE latent, with out_loc == 0 marking a padded row;
 *    the V4.1 dequantizers.
 *  - same page, Review: the ue8m0 exponent formula of the fp8 quantizer, the
 *    decode compressor reading its rotary table at pos - 1, its pair-state
 *    ring and the normalisation eps.
 *  - sglang PR #46230, summary: int32 [2, request slots] extend offsets
 *    (first row, row count) read on device so the call can sit in a graph,
 *    and the fused |kv|score| projection buffer.
 *  - sglang PR #45909, summary: one dequant per kv source reused by the
 *    layers that read it, keyed by (source cache, gather ids, row count) and
 *    forgotten on a plain get, a reallocation or a new forward.
 *  - flashinfer_sparse.py (vLLM DeepSeek-V4.1 sparse MLA backend),
 *    _compressed_topk_to_slots: request-local compressed ids mapped to
 *    physical slots through the block table, -1 marking empty entries; its
 *    DCP helpers (the same function for more than one rank, and
 *    _dcp_prefill_gather): global compressed ids dealt to the ranks of a
 *    decode-context-parallel group in runs of the interleave size, pages of
 *    block_size states per rank, the other ranks' ids dropped and this
 *    rank's slots compacted to a prefix.
 *
 * Conventions shared by every entry point
 *  - Pointers named "device" are HIP device memory (or memory the device can
 *    read and write); "host" pointers are read on the calling thread before
 *    the call returns.  The caller owns every buffer; the library allocates
 *    no device memory in any call.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *    asynchronous on that stream and performs no host <-> device
 *    synchronisation, so calls can be captured in a HIP graph.
 *  - bf16 values are 16-bit bfloat16 bit patterns.
 *  - A row is 512 latent dims: dims 0..447 "nope", 448..511 "rope".
 *  - Return codes: KVC_OK, or a negative KVC_E* code with a message in
 *    kvc_last_error() (thread-local).  Arguments are validated from host
 *    scalars only; nothing is launched when validation fails.
 *  - Device-side problems (an id, page or position outside its table) are
 *    reported through an optional device `status` word: the kernel ORs a
 *    KVC_STATUS_* bit into it and skips the write (stores) or writes a zero
 *    row (gather).  The caller zeroes the word before the call.
 */
#ifndef KVC_H
#define KVC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- codes */
enum {
  KVC_OK = 0,
  KVC_EINVAL = -1,        /* null pointer, bad size, stride or alignment  */
  KVC_EUNSUPPORTED = -2,  /* layout, ratio or mode not supported          */
  KVC_ELAUNCH = -3        /* a HIP error when launching                   */
};

enum {
  KVC_STATUS_ID_RANGE = 1,     /* gather id (or its logical page) beyond the table / cache */
  KVC_STATUS_PAGE_RANGE = 2,   /* physical page < 0 or >= num_pages                       */
  KVC_STATUS_PT_RANGE = 4,     /* compressed row beyond its slot's page-table row          */
  KVC_STATUS_LATENT_RANGE = 8, /* latent row index >= max_out_rows                         */
  KVC_STATUS_POS_RANGE = 16,   /* rotary position < 0 or >= max_pos: row skipped           */
  KVC_STATUS_REQ_RANGE = 32,   /* request index outside the block table: row dropped        */
  KVC_STATUS_TOKEN_RANGE = 64  /* prefill slot's token rows outside [0, kv_rows): slot skipped */
};

/* ---------------------------------------------------------------- layouts
 * KVLayout of sglang PR #39652, Summary.  Per row:
 *   V4       data 576 B = 448 fp8 e4m3fn codes (dims 0..447) + 64 bf16 (dims
 *            448..511, little endian); scale 8 B = 7 ue8m0 bytes (one per 64
 *            nope dims) + 1 zero pad byte.                       584 B.
 *   V41      data 512 B = 512 fp8 e4m3fn codes; scale 16 B = one ue8m0 byte
 *            per 32 dims.                                        528 B.
 *   V41_FP4  data 256 B = 512 e2m1 codes, dim 2k in the low nibble of byte k;
 *            scale 32 B = one e4m3fn byte per 16 dims.           288 B.
 * Page layout: page p starts at base + p * page_stride; the data parts of its
 * page_size rows come first (row r at r * data_bytes), then their scale
 * parts (row r at page_size * data_bytes + r * scale_bytes).  Slot s lives in
 * page s / page_size, row s % page_size.  Physical page 0 is the padding page:
 * slot 0 (out_loc == 0) is never written.
 */
typedef enum kvc_layout {
  KVC_LAYOUT_V4 = 0,
  KVC_LAYOUT_V41 = 1,
  KVC_LAYOUT_V41_FP4 = 2
} kvc_layout;

typedef struct kvc_layout_info {
  int32_t data_bytes;    /* per row, data part  (576 / 512 / 256) */
  int32_t scale_bytes;   /* per row, scale part (8 / 16 / 32)     */
  int32_t row_bytes;     /* data + scale        (584 / 528 / 288) */
  int32_t group;         /* dims per scale      (64 / 32 / 16)    */
  int32_t quant_dims;    /* quantized dims      (448 / 512 / 512) */
} kvc_layout_info;

/* A paged main-KV cache.  page_size: power of two, 1..4096 rows.
 * page_stride: bytes between pages, >= page_size * row_bytes and a multiple
 * of 16.  base: device, 16-byte aligned.  num_pages >= 1. */
typedef struct kvc_cache {
  void* base;
  int32_t layout;        /* kvc_layout */
  int32_t page_size;
  int64_t page_stride;
  int64_t num_pages;
} kvc_cache;

/* Fill *info for `layout`.  Returns KVC_EUNSUPPORTED for an unknown layout.
 * Host only; launches nothing. */
int kvc_layout_query(int32_t layout, kvc_layout_info* info);

/* ---------------------------------------------------------------- store
 * Quantize n bf16 rows into the cache: row i goes to slot out_loc[i]
 * (sglang PR #39652, Summary: the V4.1 row quantizer and the paged writers).
 *   rows_bf16   device, n rows of 512 bf16, row i at rows_bf16 + i*row_stride
 *               elements; row_stride >= 512 and a multiple of 8; 16-B aligned
 *   out_loc     device int32 [n]; 0 = padded row (nothing written); a slot
 *               outside the cache sets KVC_STATUS_PAGE_RANGE and is skipped
 *   status      device int32 or NULL
 * Quantization per layout:
 *   fp8 groups (V41: 32 dims, V4: 64 nope dims): E = 127 +
 *     ceil(log2(max(amax / 448, 1e-4))) (sglang PR #39652, Review), stored
 *     as the scale byte; code = e4m3fn(x * 2^(127 - E)), nearest even.
 *   fp4 groups (16 dims): s = e4m3fn(amax / 6 in fp32, nearest even,
 *     clamped at 448) stored as the scale byte; code = e2m1(x / s in fp32,
 *     nearest even, clamped at 6); s == 0 gives code 0.
 *   Codes keep the sign of x (a negative value that rounds to zero gives the
 *   negative-zero code).  V4 rope dims are stored as their bf16 bytes.
 * Rows with the same non-zero out_loc race (undefined which one lands). */
int kvc_store_rows(const kvc_cache* cache, const void* rows_bf16, int64_t row_stride,
                   const int32_t* out_loc, int64_t n, int32_t* status, void* stream);

/* kvc_store_rows with the rotary embedding applied in the kernel (sglang PR
 * #39652, Summary: the cache writer with an optional in-kernel RoPE for the
 * V4.1 layouts; accepted for every layout here).  Before row i is quantized,
 * its dims (448 + 2j, 449 + 2j), j = 0..31, are rotated by (cos, sin) =
 * (freqs[positions[i]][2j], freqs[positions[i]][2j + 1]); the products are
 * formed in fp64 and the rotated value is rounded once to bf16 (nearest
 * even), so the result does not depend on the evaluation order.  The other
 * dims are stored as given.
 *   positions  device int32 [n]; a position < 0 or >= max_pos skips the row
 *              with KVC_STATUS_POS_RANGE (checked after out_loc == 0)
 *   freqs      device fp32 [max_pos, 64], 16-byte aligned
 * Other arguments and rules as kvc_store_rows. */
int kvc_store_rows_rope(const kvc_cache* cache, const void* rows_bf16, int64_t row_stride,
                        const int32_t* positions, const float* freqs, int64_t max_pos,
                        const int32_t* out_loc, int64_t n, int32_t* status, void* stream);

/* ---------------------------------------------------------------- compress
 * The ratio-1 / ratio-2 compressor (sglang PR #39652, Summary; sglang PR
 * #46230, summary), per output row:
 *   v   = ratio 2: per dim d, the softmax over the pair's two scores weights
 *         their two kv values: v_d = (e^(s0_d - m) k0_d + e^(s1_d - m) k1_d)
 *         / (e^(s0_d - m) + e^(s1_d - m)), m = max(s0_d, s1_d);
 *         ratio 1: the token's kv row;
 *   y   = v * rsqrt(mean(v^2) + eps) * norm_w            (fp32)
 *   latent_out row = bf16(y)                              (pre-RoPE latent)
 *   z   = y, with dims (448 + 2j, 449 + 2j), j = 0..31, rotated by
 *         (cos, sin) = (freqs[p][2j], freqs[p][2j + 1])
 *   bf16(z) is quantized as kvc_store_rows does into slot out_loc (skipped
 *   when out_loc == 0).
 *
 * PREFILL mode (ragged extend batch):
 *   offsets   device int32 [2, num_slots]: offsets[b] = first token row of
 *             slot b in the projection buffer, offsets[num_slots + b] = its
 *             token count (<= 0: the slot has no tokens)
 *   start_pos device int32 [num_slots]: position of slot b's first token
 *             (< 0: the slot is skipped)
 *   kv_rows   token rows the kv (and score) buffers hold: a slot whose rows
 *             offsets[b] .. offsets[b] + count - 1 do not lie in [0, kv_rows)
 *             is skipped whole (no rows, no pending-state write) with
 *             KVC_STATUS_TOKEN_RANGE
 *   Ratio 1: every token at position q gives compressed row c = q.
 *   Ratio 2: every token at an odd position q closes the pair (q - 1, q) and
 *   gives row c = q / 2; the pair's first token is the previous token, or
 *   the slot's pending state when q - 1 precedes the extend.  A last token
 *   at an even position is written to the pending state (after it is read).
 *   The rotary position of a row is p = c for ratio 1 and p = 2c (the pair's
 *   first position) for ratio 2.  out_loc = page_table[b][c / page_size] *
 *   page_size + c % page_size; a logical page c / page_size >= pt_width sets
 *   KVC_STATUS_PT_RANGE and the row is not stored.  Latent rows are numbered
 *   consecutively over the batch in slot order.
 * DECODE mode (one new token per slot):
 *   slot b's token is row b of the projection buffer at position
 *   start_pos[b] (< 0: skipped); kv_rows >= num_slots.  Ratio 1: row c =
 *   pos.  Ratio 2: an odd position pools the pending state with the token
 *   into row c = pos / 2 (rotary position pos - 1); an even position writes
 *   the token to the pending state and emits no row.  out_loc = out_loc[b]
 *   when out_loc is given (0 = no cache write, a padded row), otherwise from
 *   the page table as in prefill.  The latent row of slot b is b (written
 *   only when a row is emitted).
 * VERIFY mode (speculative decoding: draft_len = D tokens per slot; sglang
 *   PR #39652, Summary and Review, the decode-or-verify ratio-2 compressor):
 *   slot b's tokens are rows b*D .. b*D + D - 1 at positions start_pos[b] ..
 *   start_pos[b] + D - 1 (start_pos[b] < 0: the slot is skipped; kv_rows >=
 *   num_slots * D), taken in
 *   order as D decode tokens: token j's latent row and out_loc entry are
 *   b*D + j, and a ratio-2 token at an odd position pools with the previous
 *   draft token (j > 0) or with the ring entry (j = 0).  DECODE is VERIFY
 *   with D = 1.
 *
 * Pending-state ring (ratio 2, every mode): state holds ring_slots entries
 * per slot, entry e of slot b at state + (b*ring_slots + e)*1024 elements
 * (kv then score, 512 each); the pending first token of pair k (positions
 * 2k, 2k + 1) lives in entry k % ring_slots.  One entry is the plain decode
 * state.  A verify step that accepts only the first a drafts is followed by
 * a step at start_pos + a; that step finds its pending token intact when
 * ring_slots > D / 2 (the entries one step writes then never reach the one
 * an earlier step left).  When two even positions of one call share an
 * entry, the later token's is the one written.
 *
 * Decode context parallelism (dcp_world W > 1; flashinfer_sparse.py, DCP
 * helpers): the compressed rows of a request are dealt to the W ranks in
 * runs of dcp_interleave (K) consecutive rows, round robin (row c belongs to
 * rank (c / K) % W), and every rank keeps its own rows densely: row c is the
 * u-th row of its rank, u = (c / (K*W))*K + c % K, stored through this
 * rank's page table at page_table[b][u / page_size] * page_size + u %
 * page_size.  This call stores only the rows of rank dcp_rank; the other
 * rows are still computed and their latent rows written.  page_size must be
 * a multiple of K.  An explicit out_loc (decode, verify) is used as given.
 */
typedef enum kvc_mode {
  KVC_MODE_PREFILL = 0,
  KVC_MODE_DECODE = 1,
  KVC_MODE_VERIFY = 2
} kvc_mode;

typedef struct kvc_compress_args {
  int32_t ratio;              /* 1 or 2 */
  int32_t mode;               /* kvc_mode */
  const void* kv;             /* device bf16: token t's kv row at kv + t*kv_stride */
  int64_t kv_stride;          /* elements, multiple of 8, >= 512 */
  const void* score;          /* device bf16, ratio 2 (fused buffer: kv + 512) */
  int64_t score_stride;       /* elements, multiple of 8 */
  int32_t num_slots;          /* S >= 0; prefill: S <= 8191 */
  const int32_t* offsets;     /* device int32 [2, S], prefill */
  const int32_t* start_pos;   /* device int32 [S] */
  const int32_t* page_table;  /* device int32 [S, pt_stride]; may be NULL only
                                 in decode / verify mode with out_loc */
  int64_t pt_stride;          /* entries between page-table rows (addressing) */
  const int32_t* out_loc;     /* device int32 [S * D], decode / verify only, or NULL */
  void* state;                /* device bf16 [S, ring_slots, 2, 512]: pending (kv, score), ratio 2 */
  const void* norm_w;         /* device bf16 [512] */
  float eps;
  const float* freqs;         /* device fp32 [max_pos, 64] */
  int64_t max_pos;
  void* latent_out;           /* device bf16, row i at latent_out + i*latent_stride */
  int64_t latent_stride;      /* elements, multiple of 8, >= 512 */
  int64_t max_out_rows;       /* rows latent_out can hold; prefill also sizes the grid */
  void* prequant_out;         /* device bf16 or NULL: bf16(z), indexed like latent */
  int64_t prequant_stride;
  kvc_cache cache;
  int32_t* status;            /* device int32 or NULL */
  int32_t draft_len;          /* VERIFY: tokens per slot, 1..64 (other modes: ignored) */
  int32_t ring_slots;         /* pending-state entries per slot, 1..1024 (0: 1) */
  int32_t dcp_world;          /* decode-context-parallel ranks, 0 or 1: none; <= 1024 */
  int32_t dcp_rank;           /* 0 .. dcp_world - 1 */
  int32_t dcp_interleave;     /* consecutive rows per rank turn, >= 1, divides page_size */
  int32_t tile_rows;          /* prefill: consecutive rows per work item, 1, 2 or 4 (0:
                                 the library's choice, 1 for max_out_rows <= 8192, else 2);
                                 results do not depend on it */
  int64_t kv_rows;            /* token rows in kv and score, >= 1 */
  int64_t pt_width;           /* valid entries per page-table row, 1 .. pt_stride (the
                                 bound; pt_stride only addresses the rows) */
} kvc_compress_args;
/* Index ranges: token positions (start_pos + i) stay below 2^31, the rows a
 * prefill batch emits and the token rows of a decode / verify batch (num_slots
 * * draft_len) number fewer than 2^31 (a verify batch past that is rejected
 * with KVC_EINVAL).  Beyond them the results are unspecified; no access
 * leaves the buffers the other arguments describe. */

int kvc_compress_store(const kvc_compress_args* args, void* stream);

/* ---------------------------------------------------------------- gather
 * Expand n cached rows to bf16 (sglang PR #39652, Summary: V4.1
 * dequantizers; sglang PR #45909, summary: the sparse-prefill dequant).
 *   page_table  device int32 [n_pages] or NULL.  Given: ids are logical rows
 *               and id maps to slot page_table[id / page_size] * page_size +
 *               id % page_size (flashinfer_sparse.py,
 *               _compressed_topk_to_slots).  NULL: ids are physical slots.
 *   ids         device int32 [n]; id < 0 gives a zero row; an id past the
 *               table or cache, or a page outside the cache, gives a zero row
 *               and a status bit
 *   out_bf16    device, row j at out_bf16 + j*out_row_stride elements;
 *               out_row_stride in [512, 2^25], multiple of 8; 16-B aligned
 * Values: fp8 code times 2^(E - 127) (V41, V4 nope dims), e2m1 code times
 * the e4m3 scale (V41_FP4), V4 rope dims copied; each product is exact in
 * bf16.  A NaN code, a ue8m0 byte of 255 or a NaN e4m3 scale gives NaN. */
int kvc_dequant_gather(const kvc_cache* cache, const int32_t* page_table, int64_t n_pages,
                       const int32_t* ids, int64_t n, void* out_bf16, int64_t out_row_stride,
                       int32_t* status, void* stream);

/* ---------------------------------------------------------------- DCP ids
 * One rank's share of the gather ids of a decode-context-parallel group
 * (flashinfer_sparse.py, DCP helpers: the ids of the indexer are GLOBAL
 * compressed row ids; the states other ranks own are dropped and this rank's
 * slots compacted to a prefix with a -1 tail and a count).  Row t of `ids`
 * (k ids at ids + t*ids_stride) belongs to request token_to_req[t].  Each id
 * c >= 0 that rank `rank` owns (the dealing of kvc_compress_store: run c / K
 * goes to rank (c / K) % world; this rank's ordinal u = (c / (K*world))*K +
 * c % K) becomes the physical slot block_table[req][u / page_size] *
 * page_size + u % page_size.  The slots of a row are written, in the order
 * of their ids, to out_slots + t*out_stride, followed by -1 up to k entries;
 * out_lens[t] = their count.  The output is a physical-slot id list for
 * kvc_dequant_gather with page_table = NULL.
 *   ids          device int32, rows of k entries, ids_stride >= k
 *   token_to_req device int32 [T]; a request outside [0, n_req) drops the
 *                row (count 0) with KVC_STATUS_REQ_RANGE
 *   block_table  device int32, n_req rows of bt_width valid entries, rows
 *                bt_stride entries apart (1 <= bt_width <= bt_stride): this
 *                rank's pages
 *   valid        device int32 [T] or NULL; 0 = a padding token: count 0
 *   out_slots    device int32, 4-byte aligned, out_stride >= k; must not
 *                overlap ids (may be NULL when k = 0)
 *   out_lens     device int32 [T]
 * A page index >= bt_width (KVC_STATUS_PT_RANGE) or a page < 0 or >=
 * num_pages (KVC_STATUS_PAGE_RANGE) drops that id.  world = 1 (rank 0) maps
 * through the block table with the -1 entries squeezed out.  page_size is a
 * power of two in [1, 4096] and a multiple of interleave; 1 <= world <= 1024;
 * 0 <= k <= 65536. */
int kvc_dcp_filter_ids(const int32_t* ids, int64_t T, int32_t k, int64_t ids_stride,
                       const int32_t* token_to_req, int32_t n_req, const int32_t* block_table,
                       int64_t bt_stride, int64_t bt_width, const int32_t* valid, int32_t page_size,
                       int64_t num_pages, int32_t world, int32_t rank, int32_t interleave,
                       int32_t* out_slots, int64_t out_stride, int32_t* out_lens,
                       int32_t* status, void* stream);

/* ---------------------------------------------------------------- reuse
 * Dequant reuse across the layers that read one kv source (sglang PR #45909,
 * summary).  A kvc_kvbuf is a small host object that remembers the head: the
 * arguments of the last gather it ran.  kvc_dequant_gather_reuse runs the
 * gather unless the head matches (cache base, layout, page size, page stride,
 * page table, n_pages, ids pointer, n, output pointer, output stride), in
 * which case it launches nothing and sets *hit = 1.  The key compares
 * pointers, not contents: the caller must not rewrite the ids, the page
 * table, the cache rows or the output behind a head it still relies on;
 * that is what kvc_kvbuf_forget / kvc_kvbuf_begin_forward are for.  A hit
 * launches nothing, so a reader on another stream must still be ordered
 * after the gather that filled the output.
 *   kvc_kvbuf_forget         a plain get or a reallocation: drop the head
 *   kvc_kvbuf_begin_forward  a new forward pass: drop the head
 * A kvc_kvbuf is not thread-safe; it owns no device memory. */
typedef struct kvc_kvbuf kvc_kvbuf;

kvc_kvbuf* kvc_kvbuf_create(void);
void kvc_kvbuf_destroy(kvc_kvbuf* kb);
void kvc_kvbuf_forget(kvc_kvbuf* kb);
void kvc_kvbuf_begin_forward(kvc_kvbuf* kb);
int kvc_dequant_gather_reuse(kvc_kvbuf* kb, const kvc_cache* cache, const int32_t* page_table,
                             int64_t n_pages, const int32_t* ids, int64_t n, void* out_bf16,
                             int64_t out_row_stride, int32_t* status, int32_t* hit,
                             void* stream);

/* ---------------------------------------------------------------- misc */
/* Message of the last failed call on this thread ("" if none). */
const char* kvc_last_error(void);

/* Library ABI version (this header: 3). */
int kvc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
