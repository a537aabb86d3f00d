/*
 * kvc_oracle.h -- plain CPU reference of the DeepSeek-V4.1 low-ratio
 * compressed-KV path (compress-store and dequant-gather).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library) never calls it and shares no code, header or table with it.
 *
 * Everything here is host memory.  bf16 values are carried as uint16 bit
 * patterns.  Floating-point work of the compressor is done in fp64 and
 * rounded once to bf16 where the method stores bf16.  Number formats are
 * produced by their definitions (nearest representable value, ties to even),
 * not by bit tricks.
 *
 * Sources (the web pages this library is written from):
 *  [PR39652-S]  sglang PR #39652 "dsv4.1: compression, KV I/O, and metadata
 *               kernels", Summary: the three paged layouts and their byte
 *               counts, the single V4.1 row quantizer, the ratio-1/ratio-2
 *               compressors (pooling, RMSNorm, RoPE, store, pre-RoPE latent
 *               returned, out_loc == 0 = padded row).
 *  [PR39652-R]  same page, Review: the ue8m0 scale exponent
 *               ceil(log2(max(amax/448, 1e-4))); the decode kernel reading
 *               the rotary table at position pos-1 on the rope lanes; the
 *               pair-state ring and the eps of the normalisation.
 *  [PR46230-S]  sglang PR #46230, summary: int32 [2, slots] extend offsets
 *               (first row, row count) and the fused |kv|score| projection.
 *  [PR45909-S]  sglang PR #45909, summary: reuse of one dequant per source.
 *  [FI-topk]    flashinfer_sparse.py, _compressed_topk_to_slots: request
 *               ids mapped to physical slots through the block table.
 *  [FI-dcp]     flashinfer_sparse.py, DCP helpers (_compressed_topk_to_slots
 *               for more than one rank, _dcp_prefill_gather): global
 *               compressed ids dealt to the ranks in runs of the interleave
 *               size, pages of block_size states per rank, the ids other
 *               ranks own dropped and this rank's slots compacted to a prefix.
 * Where the pages leave a step open, the reading taken is stated beside the
 * function.  Functions whose exact results have no pin of their own say
 * "parity unpinned".
 */
#ifndef KVC_ORACLE_H
#define KVC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { KVO_V4 = 0, KVO_V41 = 1, KVO_V41_FP4 = 2 };
enum { KVO_PREFILL = 0, KVO_DECODE = 1, KVO_VERIFY = 2 };

/* status bits (the values documented for the device status word) */
enum {
  KVO_ST_ID_RANGE = 1,      /* gather id / logical page beyond the table   */
  KVO_ST_PAGE_RANGE = 2,    /* physical page outside the cache             */
  KVO_ST_PT_RANGE = 4,      /* compressed row beyond the slot's page table */
  KVO_ST_LATENT_RANGE = 8,  /* latent ordinal beyond the output capacity   */
  KVO_ST_POS_RANGE = 16,    /* rotary position outside the table           */
  KVO_ST_REQ_RANGE = 32,    /* request index outside the block table       */
  KVO_ST_TOKEN_RANGE = 64   /* prefill slot's token rows outside the buffer */
};

typedef struct {
  uint8_t* base;        /* host image: page p starts at base + p*page_stride */
  int32_t layout;
  int32_t page_size;    /* rows per page */
  int64_t page_stride;  /* bytes per page */
  int64_t num_pages;
} kvo_cache;

typedef struct {
  int32_t ratio;              /* 1 or 2 */
  int32_t mode;               /* KVO_PREFILL, KVO_DECODE or KVO_VERIFY */
  const uint16_t* kv;         /* token rows, kv part (bf16) */
  int64_t kv_stride;          /* elements between token rows */
  const uint16_t* score;      /* token rows, score part (ratio 2) */
  int64_t score_stride;
  int32_t num_slots;
  const int32_t* offsets;     /* prefill: [2, S] first token row, token count */
  const int32_t* start_pos;   /* [S] position of the slot's first (or only) token */
  const int32_t* page_table;  /* [S, pt_stride] compressed-row pages, or NULL */
  int64_t pt_stride;
  const int32_t* out_loc;     /* decode / verify: [S * draft_len] destination slot,
                                 0 = no write; or NULL */
  uint16_t* state;            /* [S, ring, 2, 512] pending tokens (kv, score), ratio 2 */
  const uint16_t* norm_w;     /* [512] bf16 */
  float eps;
  const float* freqs;         /* [max_pos, 64] fp32 (cos, sin) pairs */
  int64_t max_pos;
  uint16_t* latent;           /* pre-RoPE latent rows (bf16) */
  int64_t latent_stride;
  int64_t max_out_rows;
  uint16_t* prequant;         /* post-RoPE rows fed to the quantizer, or NULL */
  int64_t prequant_stride;
  kvo_cache cache;
  int32_t* status;
  int32_t draft_len;          /* verify: tokens per slot */
  int32_t ring_slots;         /* pending-state entries per slot (<= 1: one) */
  int32_t dcp_world;          /* context-parallel ranks (<= 1: none) */
  int32_t dcp_rank;
  int32_t dcp_interleave;     /* consecutive compressed rows per rank turn */
  int64_t kv_rows;            /* token rows the kv / score buffers hold */
} kvo_compress_args;

/* layouts */
int kvo_layout_bytes(int32_t layout, int32_t* data_bytes, int32_t* scale_bytes,
                     int32_t* row_bytes, int32_t* group);

/* number formats */
double   kvo_round_to_grid(double a, int mant_bits, int emin);
uint8_t  kvo_e4m3_encode(double v, int satfinite);
double   kvo_e4m3_decode(uint8_t c);
uint8_t  kvo_e2m1_encode(double v);
double   kvo_e2m1_decode(uint8_t c);
uint16_t kvo_bf16_encode(double v);
double   kvo_bf16_decode(uint16_t b);
int      kvo_ue8m0(float amax);
uint8_t  kvo_fp4_scale(float amax);
uint8_t  kvo_fp8_code(uint16_t x, int E);
uint8_t  kvo_fp4_code(uint16_t x, uint8_t sc);

/* one row */
void kvo_store_row(int32_t layout, const uint16_t* x, uint8_t* data, uint8_t* scale);
void kvo_dequant_row(int32_t layout, const uint8_t* data, const uint8_t* scale,
                     uint16_t* out);

/* paged cache */
void kvo_store_rows(const kvo_cache* c, const uint16_t* rows, int64_t row_stride,
                    const int32_t* out_loc, int64_t n, int32_t* status);
void kvo_dequant_gather(const kvo_cache* c, const int32_t* page_table,
                        int64_t n_pages, const int32_t* ids, int64_t n,
                        uint16_t* out, int64_t out_stride, int32_t* status);

/* store with the rotary embedding applied first */
void kvo_store_rows_rope(const kvo_cache* c, const uint16_t* rows, int64_t row_stride,
                         const int32_t* positions, const float* freqs, int64_t max_pos,
                         const int32_t* out_loc, int64_t n, uint16_t* rotated,
                         int32_t* status);

/* compressor */
void kvo_compress(const kvo_compress_args* a);
int64_t kvo_count_rows(const kvo_compress_args* a);

/* decode context parallelism: owner rank and per-rank ordinal of a
 * compressed row, and one rank's share of a list of global row ids */
int32_t kvo_dcp_owner(int64_t c, int32_t world, int32_t interleave, int64_t* local);
void kvo_dcp_filter_ids(const int32_t* ids, int64_t T, int32_t k, int64_t ids_stride,
                        const int32_t* token_to_req, int32_t n_req,
                        const int32_t* block_table, int64_t bt_stride,
                        const int32_t* valid, int32_t page_size, int64_t num_pages,
                        int32_t world, int32_t rank, int32_t interleave,
                        int32_t* out_slots, int64_t out_stride, int32_t* out_lens,
                        int32_t* status);

/* array forms (for sweeps in tests) */
void kvo_e4m3_encode_n(const double* v, int64_t n, int satfinite, uint8_t* out);
void kvo_e2m1_encode_n(const double* v, int64_t n, uint8_t* out);
void kvo_bf16_encode_n(const double* v, int64_t n, uint16_t* out);
void kvo_ue8m0_n(const float* amax, int64_t n, int32_t* out);
void kvo_fp4_scale_n(const float* amax, int64_t n, uint8_t* out);
void kvo_fp8_code_n(const uint16_t* x, const int32_t* E, int64_t n, uint8_t* out);
void kvo_fp4_code_n(const uint16_t* x, const uint8_t* sc, int64_t n, uint8_t* out);
void kvo_store_row_n(int32_t layout, const uint16_t* x, int64_t n,
                     uint8_t* data, uint8_t* scale);
void kvo_dequant_row_n(int32_t layout, const uint8_t* data, const uint8_t* scale,
                       int64_t n, uint16_t* out);

int kvo_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
