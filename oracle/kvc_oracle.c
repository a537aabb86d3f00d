/*
 * kvc_oracle.c -- plain CPU reference of the DeepSeek-V4.1 low-ratio
 * compressed-KV path.  TEST INFRASTRUCTURE ONLY (see kvc_oracle.h): nothing
 * in the product library calls, links or includes this file.
 *
 * Style: scalar loops, fp64 arithmetic, number formats by definition.  OpenMP
 * splits independent rows over threads and nothing else.
 */
#include "kvc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KVO_D 512
#define KVO_ROPE 64
#define KVO_NOPE (KVO_D - KVO_ROPE)

int kvo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Layouts [PR39652-S]: per token, V4 = 448 fp8 nope dims + 64 bf16 rope dims
 * + ue8m0 scales = 584 B; V41 = 512 fp8 dims + one ue8m0 scale per 32 dims =
 * 528 B; V41_FP4 = 512 e2m1 codes + one e4m3 scale per 16 dims = 288 B.
 * Reading: V4 keeps one ue8m0 scale per 64 nope dims (7 bytes) and pads its
 * scale part to 8 bytes with a zero byte, which is what 584 - 448 - 128
 * leaves.  A page holds the data parts of all its rows first, then their
 * scale parts (the pages list data and scale bytes per token separately and
 * fix only the per-token totals).
 * ---------------------------------------------------------------------- */
int kvo_layout_bytes(int32_t layout, int32_t* data_bytes, int32_t* scale_bytes,
                     int32_t* row_bytes, int32_t* group) {
  int32_t d, s, g;
  switch (layout) {
    case KVO_V4:      d = KVO_NOPE * 1 + KVO_ROPE * 2; s = KVO_NOPE / 64 + 1; g = 64; break;
    case KVO_V41:     d = KVO_D * 1;                   s = KVO_D / 32;         g = 32; break;
    case KVO_V41_FP4: d = KVO_D / 2;                   s = KVO_D / 16;         g = 16; break;
    default: return -1;
  }
  if (data_bytes) *data_bytes = d;
  if (scale_bytes) *scale_bytes = s;
  if (row_bytes) *row_bytes = d + s;
  if (group) *group = g;
  return 0;
}

/* ------------------------------------------------------------------------
 * Number formats.
 *
 * kvo_round_to_grid: nearest value to a >= 0 among the numbers of a binary
 * floating-point format with `mant_bits` stored mantissa bits whose smallest
 * normal binade starts at 2^emin (below it the spacing stays that of the
 * smallest binade: subnormals), ties to the even multiple of the spacing.
 * The exponent range is unbounded above; callers apply overflow rules.
 * a / q is exact (q is a power of two) and nearbyint rounds half to even in
 * the default rounding mode.
 * ---------------------------------------------------------------------- */
double kvo_round_to_grid(double a, int mant_bits, int emin) {
  if (a == 0.0) return 0.0;
  int e;
  (void)frexp(a, &e);          /* a in [2^(e-1), 2^e) */
  int lead = e - 1;
  if (lead < emin) lead = emin;
  double q = ldexp(1.0, lead - mant_bits);
  return nearbyint(a / q) * q;
}

/* OCP fp8 e4m3fn: bias 7, 3 mantissa bits, subnormals down to 2^-9, largest
 * finite 448, 0x7F/0xFF are NaN, no infinity.  A value whose magnitude
 * rounds above 448 becomes 448 when `satfinite`, NaN otherwise.  The sign of
 * a value that rounds to zero is kept (0x80 for negative). */
uint8_t kvo_e4m3_encode(double v, int satfinite) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  if (isnan(v)) return 0x7F | sign;
  double r = isinf(v) ? INFINITY : kvo_round_to_grid(fabs(v), 3, -6);
  if (r > 448.0) {
    if (!satfinite) return 0x7F | sign;
    r = 448.0;
  }
  uint8_t code;
  if (r < ldexp(1.0, -6)) {
    code = (uint8_t)(r / ldexp(1.0, -9));          /* r = k * 2^-9, k = 0..7 */
  } else {
    int e;
    double f = frexp(r, &e);                       /* r = f * 2^e, f in [0.5, 1) */
    int biased = (e - 1) + 7;
    int mant = (int)((2.0 * f - 1.0) * 8.0);
    code = (uint8_t)((biased << 3) | mant);
  }
  return code | sign;
}

double kvo_e4m3_decode(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

/* OCP fp4 e2m1: bias 1, 1 mantissa bit, values 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 * Magnitudes that round above 6 saturate to 6; the sign is kept. */
uint8_t kvo_e2m1_encode(double v) {
  uint8_t sign = signbit(v) ? 0x8 : 0x0;
  double r = kvo_round_to_grid(fabs(v), 1, 0);
  if (!(r <= 6.0)) r = 6.0;
  uint8_t code;
  if (r < 1.0) {
    code = (uint8_t)(r / 0.5);                     /* 0 or 1 */
  } else {
    int e;
    double f = frexp(r, &e);
    int biased = (e - 1) + 1;
    int mant = (int)((2.0 * f - 1.0) * 2.0);
    code = (uint8_t)((biased << 1) | mant);
  }
  return code | sign;
}

double kvo_e2m1_decode(uint8_t c) {
  int e = (c >> 1) & 3, m = c & 1;
  double v = (e == 0) ? 0.5 * m : ldexp((double)(2 + m), e - 2);
  return (c & 0x8) ? -v : v;
}

/* bfloat16 = the upper 16 bits of an IEEE binary32.  Encoding rounds to
 * nearest even with subnormals; magnitudes that round to 2^128 or above
 * become infinity; NaN becomes the quiet NaN 0x7FC0. */
uint16_t kvo_bf16_encode(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
  if (isnan(v)) return 0x7FC0;
  if (isinf(v)) return sign | 0x7F80;
  double r = kvo_round_to_grid(fabs(v), 7, -126);
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
  uint16_t code;
  if (r < ldexp(1.0, -126)) {
    code = (uint16_t)(r / ldexp(1.0, -133));
  } else {
    int e;
    double f = frexp(r, &e);
    int biased = (e - 1) + 127;
    int mant = (int)((2.0 * f - 1.0) * 128.0);
    code = (uint16_t)((biased << 7) | mant);
  }
  return code | sign;
}

double kvo_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ue8m0 scale of a group [PR39652-R]: the biased exponent
 * 127 + ceil(log2(max(amax / 448, 1e-4))).  Written as its definition: the
 * smallest integer k with 2^k >= amax/448 and 2^k >= 1e-4.  Since
 * 2^-14 < 1e-4 <= 2^-13 the second condition is k >= -13, and the first is
 * 448 * 2^k >= amax, compared exactly in fp64. */
int kvo_ue8m0(float amax) {
  double a = (double)amax;
  int k = -13;
  while (k < 128 && 448.0 * ldexp(1.0, k) < a) k++;
  return 127 + k;
}

/* e4m3 scale of one V41_FP4 group of 16.  The pages say only that each 16
 * dims share one e4m3 scale [PR39652-S].  Reading: the scale is amax / 6 (6 = the
 * largest e2m1 magnitude) divided in fp32, rounded to nearest even into
 * e4m3 and clamped at 448. */
uint8_t kvo_fp4_scale(float amax) {
  float q = amax / 6.0f;
  return kvo_e4m3_encode((double)q, 1);
}

/* ------------------------------------------------------------------------
 * store_row: quantize one bf16 row of 512 dims into its data and scale parts.
 * [PR39652-S] names a single V4.1 row quantizer; the V4 row keeps the rope
 * dims as bf16.
 * ---------------------------------------------------------------------- */
static double group_amax(const uint16_t* x, int lo, int n) {
  double m = 0.0;
  for (int d = lo; d < lo + n; ++d) {
    double a = fabs(kvo_bf16_decode(x[d]));
    if (a > m) m = a;
  }
  return m;
}

/* fp8 code of one bf16 element under ue8m0 exponent E: x * 2^(127-E) is
 * exact in fp64 and, with E from the element's group, at most 448. */
uint8_t kvo_fp8_code(uint16_t x, int E) {
  return kvo_e4m3_encode(ldexp(kvo_bf16_decode(x), 127 - E), 0);
}

/* e2m1 code of one bf16 element under the e4m3 scale code sc: the quotient
 * x / s is formed in fp32 (as the device does) and rounded to nearest even
 * into e2m1, saturating at 6.  Reading: a zero scale gives code 0. */
uint8_t kvo_fp4_code(uint16_t x, uint8_t sc) {
  float s = (float)kvo_e4m3_decode(sc);
  if (s == 0.0f) return 0;
  float y = (float)kvo_bf16_decode(x) / s;
  return kvo_e2m1_encode((double)y);
}

static void store_fp8_groups(const uint16_t* x, int dims, int group,
                             uint8_t* data, uint8_t* scale) {
  for (int g = 0; g < dims / group; ++g) {
    int E = kvo_ue8m0((float)group_amax(x, g * group, group));
    scale[g] = (uint8_t)E;
    for (int d = g * group; d < (g + 1) * group; ++d) data[d] = kvo_fp8_code(x[d], E);
  }
}

void kvo_store_row(int32_t layout, const uint16_t* x, uint8_t* data, uint8_t* scale) {
  switch (layout) {
    case KVO_V41:
      store_fp8_groups(x, KVO_D, 32, data, scale);
      break;
    case KVO_V4:
      store_fp8_groups(x, KVO_NOPE, 64, data, scale);
      scale[KVO_NOPE / 64] = 0;                    /* pad byte */
      for (int k = 0; k < KVO_ROPE; ++k) {         /* rope dims: bf16, little endian */
        data[KVO_NOPE + 2 * k] = (uint8_t)(x[KVO_NOPE + k] & 0xFF);
        data[KVO_NOPE + 2 * k + 1] = (uint8_t)(x[KVO_NOPE + k] >> 8);
      }
      break;
    case KVO_V41_FP4:
      memset(data, 0, KVO_D / 2);
      for (int g = 0; g < KVO_D / 16; ++g) {
        float amax = (float)group_amax(x, g * 16, 16);
        uint8_t sc = kvo_fp4_scale(amax);
        scale[g] = sc;
        for (int d = g * 16; d < (g + 1) * 16; ++d) {
          uint8_t q = kvo_fp4_code(x[d], sc);
          /* reading: dim 2k in the low nibble of byte k, dim 2k+1 in the high */
          data[d / 2] |= (uint8_t)((d & 1) ? (q << 4) : q);
        }
      }
      break;
    default:
      break;
  }
}

/* Dequantize one row into bf16.  V41 / V4: fp8 value times 2^(E-127);
 * V41_FP4: e2m1 value times the e4m3 scale.  Both products are formed
 * exactly in fp64 and rounded once to bf16.  Reading: a ue8m0 byte of 255
 * (the NaN of the e8m0 format) or a NaN e4m3 scale turns its group into NaN;
 * NaN fp8 codes give NaN. */
static uint16_t dq_fp8(uint8_t code, uint8_t E) {
  if (E == 255) return 0x7FC0;
  double v = kvo_e4m3_decode(code);
  if (isnan(v)) return 0x7FC0;
  return kvo_bf16_encode(ldexp(v, (int)E - 127));
}

void kvo_dequant_row(int32_t layout, const uint8_t* data, const uint8_t* scale,
                     uint16_t* out) {
  switch (layout) {
    case KVO_V41:
      for (int d = 0; d < KVO_D; ++d) out[d] = dq_fp8(data[d], scale[d / 32]);
      break;
    case KVO_V4:
      for (int d = 0; d < KVO_NOPE; ++d) out[d] = dq_fp8(data[d], scale[d / 64]);
      for (int k = 0; k < KVO_ROPE; ++k)
        out[KVO_NOPE + k] = (uint16_t)(data[KVO_NOPE + 2 * k] |
                                       (data[KVO_NOPE + 2 * k + 1] << 8));
      break;
    case KVO_V41_FP4:
      for (int d = 0; d < KVO_D; ++d) {
        double s = kvo_e4m3_decode(scale[d / 16]);
        uint8_t q = (d & 1) ? (data[d / 2] >> 4) : (data[d / 2] & 0xF);
        out[d] = isnan(s) ? 0x7FC0 : kvo_bf16_encode(kvo_e2m1_decode(q) * s);
      }
      break;
    default:
      break;
  }
}

/* ------------------------------------------------------------------------
 * Paged addressing: slot -> (page, row in page).  Data part of row r of page
 * p at p*page_stride + r*data_bytes; scale part at
 * p*page_stride + page_size*data_bytes + r*scale_bytes.
 * ---------------------------------------------------------------------- */
static uint8_t* row_data(const kvo_cache* c, int64_t slot) {
  int32_t db;
  kvo_layout_bytes(c->layout, &db, NULL, NULL, NULL);
  int64_t page = slot / c->page_size, r = slot % c->page_size;
  return c->base + page * c->page_stride + r * db;
}

static uint8_t* row_scale(const kvo_cache* c, int64_t slot) {
  int32_t db, sb;
  kvo_layout_bytes(c->layout, &db, &sb, NULL, NULL);
  int64_t page = slot / c->page_size, r = slot % c->page_size;
  return c->base + page * c->page_stride + (int64_t)c->page_size * db + r * sb;
}

static void set_status(int32_t* status, int32_t bit) {
  if (!status) return;
#pragma omp atomic
  *status |= bit;
}

/* Store bf16 rows at caller-given slots; slot 0 marks a padded row and is
 * skipped [PR39652-S]. */
void kvo_store_rows(const kvo_cache* c, const uint16_t* rows, int64_t row_stride,
                    const int32_t* out_loc, int64_t n, int32_t* status) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int32_t loc = out_loc[i];
    if (loc == 0) continue;
    if (loc < 0 || loc / c->page_size >= c->num_pages) {
      set_status(status, KVO_ST_PAGE_RANGE);
      continue;
    }
    kvo_store_row(c->layout, rows + i * row_stride, row_data(c, loc), row_scale(c, loc));
  }
}

/* Store with an in-kernel rotary embedding [PR39652-S: the cache writer
 * with optional RoPE for the V4.1 layouts]: row i's dims (448+2j, 449+2j)
 * are rotated by (cos, sin) = (freqs[positions[i]][2j], freqs[positions[i]][2j+1])
 * in fp64 and rounded once to bf16, the other dims pass unchanged, and the
 * result is stored as kvo_store_rows stores (any layout).  Readings: the
 * rotation is the one the compressors apply (interleaved pairs of the last
 * 64 dims); a padded row (out_loc 0) is skipped before its position is
 * looked at; a position outside the table skips the row with
 * KVO_ST_POS_RANGE.  `rotated` (NULL or n x 512) receives the rotated bf16
 * rows of the rows that are stored. */
void kvo_store_rows_rope(const kvo_cache* c, const uint16_t* rows, int64_t row_stride,
                         const int32_t* positions, const float* freqs, int64_t max_pos,
                         const int32_t* out_loc, int64_t n, uint16_t* rotated,
                         int32_t* status) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int32_t loc = out_loc[i];
    if (loc == 0) continue;
    int64_t p = positions[i];
    if (p < 0 || p >= max_pos) {
      set_status(status, KVO_ST_POS_RANGE);
      continue;
    }
    if (loc < 0 || loc / c->page_size >= c->num_pages) {
      set_status(status, KVO_ST_PAGE_RANGE);
      continue;
    }
    const uint16_t* x = rows + i * row_stride;
    uint16_t z[KVO_D];
    memcpy(z, x, sizeof z);
    const float* f = freqs + p * KVO_ROPE;
    for (int j = 0; j < KVO_ROPE / 2; ++j) {
      double xr = kvo_bf16_decode(x[KVO_NOPE + 2 * j]), xi = kvo_bf16_decode(x[KVO_NOPE + 2 * j + 1]);
      double cs = f[2 * j], sn = f[2 * j + 1];
      z[KVO_NOPE + 2 * j] = kvo_bf16_encode(xr * cs - xi * sn);
      z[KVO_NOPE + 2 * j + 1] = kvo_bf16_encode(xr * sn + xi * cs);
    }
    if (rotated) memcpy(rotated + i * KVO_D, z, sizeof z);
    kvo_store_row(c->layout, z, row_data(c, loc), row_scale(c, loc));
  }
}

/* Gather rows by id and expand them to bf16.  With a page table the ids are
 * logical rows mapped through it [FI-topk]; without one they are physical
 * slots.  A negative id yields a zero row (reading: the -1 padding of top-k
 * id lists).  Out-of-range ids or pages yield a zero row and a status bit. */
void kvo_dequant_gather(const kvo_cache* c, const int32_t* page_table,
                        int64_t n_pages, const int32_t* ids, int64_t n,
                        uint16_t* out, int64_t out_stride, int32_t* status) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    uint16_t* o = out + j * out_stride;
    memset(o, 0, KVO_D * sizeof(uint16_t));
    int64_t id = ids[j];
    if (id < 0) continue;
    int64_t slot;
    if (page_table) {
      int64_t lp = id / c->page_size;
      if (lp >= n_pages) { set_status(status, KVO_ST_ID_RANGE); continue; }
      int64_t phys = page_table[lp];
      if (phys < 0 || phys >= c->num_pages) { set_status(status, KVO_ST_PAGE_RANGE); continue; }
      slot = phys * c->page_size + id % c->page_size;
    } else {
      if (id / c->page_size >= c->num_pages) { set_status(status, KVO_ST_ID_RANGE); continue; }
      slot = id;
    }
    kvo_dequant_row(c->layout, row_data(c, slot), row_scale(c, slot), o);
  }
}

/* ------------------------------------------------------------------------
 * Compressor [PR39652-S, PR39652-R, PR46230-S].
 *
 * Per output row (fp64 throughout):
 *   ratio 2: per channel d, a softmax over the pair's two scores weights the
 *            pair's two kv values;  ratio 1: the token's kv row itself;
 *   RMSNorm over the 512 dims with weight w and eps;
 *   latent = bf16(y)  (the pre-RoPE latent that is returned);
 *   RoPE on dims 448..511, pairs (448+2j, 449+2j) rotated by the table entry
 *   (cos, sin) = (freqs[p][2j], freqs[p][2j+1]);
 *   z = bf16(rotated y), quantized by store_row into slot out_loc unless
 *   out_loc == 0.
 * Readings: the softmax is per channel over the two tokens; the norm covers
 * all 512 dims and the weight multiplies after the rsqrt; RoPE acts on the
 * unrounded y; the rotary position of a ratio-2 row is that of the first
 * token of its pair (pos - 1 of the completing token, as the decode kernel
 * reads its table), of a ratio-1 row the token's own position.
 * Parity unpinned: the fp32 rounding of exp / rsqrt on the device side is
 * covered by a tolerance, not by a value from the pages.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t slot;          /* request slot b */
  int64_t c;             /* compressed row index within the request */
  int64_t p;             /* rotary position */
  const uint16_t* k0;    /* first token of the pair (NULL for ratio 1) */
  const uint16_t* s0;
  const uint16_t* k1;    /* second (or only) token */
  const uint16_t* s1;
  int64_t latent_idx;
  int64_t token;         /* decode / verify: the token's index into out_loc */
} kvo_row;

static void pool_norm_rope(const kvo_compress_args* a, const kvo_row* r,
                           uint16_t* latent_out, uint16_t* z_out) {
  double v[KVO_D], y[KVO_D], z[KVO_D];
  for (int d = 0; d < KVO_D; ++d) {
    if (r->k0 == NULL) {
      v[d] = kvo_bf16_decode(r->k1[d]);
    } else {
      double s0 = kvo_bf16_decode(r->s0[d]), s1 = kvo_bf16_decode(r->s1[d]);
      double m = s0 > s1 ? s0 : s1;
      double e0 = exp(s0 - m), e1 = exp(s1 - m);
      v[d] = (e0 * kvo_bf16_decode(r->k0[d]) + e1 * kvo_bf16_decode(r->k1[d])) / (e0 + e1);
    }
  }
  double ss = 0.0;
  for (int d = 0; d < KVO_D; ++d) ss += v[d] * v[d];
  double inv = 1.0 / sqrt(ss / KVO_D + (double)a->eps);
  for (int d = 0; d < KVO_D; ++d) y[d] = v[d] * inv * kvo_bf16_decode(a->norm_w[d]);
  for (int d = 0; d < KVO_D; ++d) latent_out[d] = kvo_bf16_encode(y[d]);
  for (int d = 0; d < KVO_NOPE; ++d) z[d] = y[d];
  const float* f = a->freqs + r->p * KVO_ROPE;
  for (int j = 0; j < KVO_ROPE / 2; ++j) {
    double xr = y[KVO_NOPE + 2 * j], xi = y[KVO_NOPE + 2 * j + 1];
    double cs = f[2 * j], sn = f[2 * j + 1];
    z[KVO_NOPE + 2 * j] = xr * cs - xi * sn;
    z[KVO_NOPE + 2 * j + 1] = xr * sn + xi * cs;
  }
  for (int d = 0; d < KVO_D; ++d) z_out[d] = kvo_bf16_encode(z[d]);
}

/* ------------------------------------------------------------------------
 * Decode context parallelism [FI-dcp].  The compressed rows of a request
 * are dealt to the `world` ranks in runs of `interleave` consecutive rows,
 * round robin: run u = c / interleave goes to rank u % world.  Each rank
 * numbers the rows it owns consecutively (its ordinal `local`), and its
 * pages hold page_size of its own rows, so page-table entry local /
 * page_size and row local % page_size place row c on its owner.  This is the
 * pages' de-interleave (virtual block of page_size * world states, owner from
 * the offset in it) whenever page_size is a multiple of the interleave.
 * ---------------------------------------------------------------------- */
int32_t kvo_dcp_owner(int64_t c, int32_t world, int32_t interleave, int64_t* local) {
  if (world <= 1) {
    if (local) *local = c;
    return 0;
  }
  int64_t u = c / interleave;
  if (local) *local = (u / world) * interleave + c % interleave;
  return (int32_t)(u % world);
}

/* destination slot of a row, or 0 when nothing is written */
static int64_t row_out_loc(const kvo_compress_args* a, const kvo_row* r) {
  const kvo_cache* c = &a->cache;
  int64_t loc;
  if (a->mode != KVO_PREFILL && a->out_loc) {
    loc = a->out_loc[r->token];
  } else {
    int64_t local = r->c;
    if (a->dcp_world > 1) {
      /* rows other ranks own are not stored here */
      if (kvo_dcp_owner(r->c, a->dcp_world, a->dcp_interleave, &local) != a->dcp_rank) return 0;
    }
    int64_t lp = local / c->page_size;
    if (lp >= a->pt_stride) { set_status(a->status, KVO_ST_PT_RANGE); return 0; }
    int64_t phys = a->page_table[(int64_t)r->slot * a->pt_stride + lp];
    if (phys < 0 || phys >= c->num_pages) { set_status(a->status, KVO_ST_PAGE_RANGE); return 0; }
    loc = phys * c->page_size + local % c->page_size;
  }
  if (loc == 0) return 0;                         /* padded row */
  if (loc < 0 || loc / c->page_size >= c->num_pages) {
    set_status(a->status, KVO_ST_PAGE_RANGE);
    return 0;
  }
  return loc;
}

static const uint16_t* tok_kv(const kvo_compress_args* a, int64_t row) {
  return a->kv + row * a->kv_stride;
}
static const uint16_t* tok_score(const kvo_compress_args* a, int64_t row) {
  return a->score ? a->score + row * a->score_stride : NULL;
}

/* The pending-state ring of slot b: `ring` entries of (kv, score).  The
 * first token of pair k (positions 2k, 2k+1) waits in entry k % ring.  One
 * entry is the single pending token of plain decode [PR39652-R]; more
 * entries let a verify step that rejects drafts find the pending token an
 * earlier step left (reading: the multi-slot ring of the verify mode, its
 * indexing unstated on the pages). */
static int64_t ring_of(const kvo_compress_args* a) {
  return a->ring_slots > 1 ? a->ring_slots : 1;
}
static uint16_t* state_kv(const kvo_compress_args* a, int32_t b, int64_t pair) {
  int64_t e = pair % ring_of(a);
  return a->state + ((int64_t)b * ring_of(a) + e) * 2 * KVO_D;
}
static uint16_t* state_score(const kvo_compress_args* a, int32_t b, int64_t pair) {
  return state_kv(a, b, pair) + KVO_D;
}

typedef struct {
  uint16_t* kv_dst;
  uint16_t* score_dst;
  const uint16_t* kv;
  const uint16_t* score;
} kvo_state_write;

/* The row plan.  Prefill: slot b holds n tokens at rows first..first+n-1 of
 * the projection buffer with positions P..P+n-1 [PR46230-S]; a slot with
 * n <= 0 (or a negative position) has no rows.  Ratio 1: one row per token,
 * compressed index = position.  Ratio 2: the pair (2c, 2c+1) yields row c
 * when its second position lies in the extend; its first token comes from
 * the slot's pending state when it precedes the extend; a last token at an
 * even position becomes the new pending state (the pair-state ring
 * [PR39652-R]).  Latent rows are numbered consecutively in slot order.
 * Decode and verify: slot b holds D tokens (D = 1 for decode, draft_len for
 * verify) at rows b*D..b*D+D-1 with positions start_pos[b]..start_pos[b]+D-1,
 * taken in order as single decode tokens: ratio 1 emits a row per token;
 * ratio 2 makes a token at an even position pending and pools a token at an
 * odd position with the pending one (the previous token of the slot, or the
 * ring's entry when the pair began before this call).  Token j's latent row
 * and out_loc entry are b*D + j (reading: the verify batch laid out as D
 * decode tokens per slot). */
static int64_t build_plan(const kvo_compress_args* a, kvo_row* rows,
                          kvo_state_write* sw, int64_t* n_sw) {
  int64_t nr = 0, ns = 0;
  const int32_t S = a->num_slots;
  for (int32_t b = 0; b < S; ++b) {
    if (a->mode == KVO_PREFILL) {
      int64_t first = a->offsets[b], n = a->offsets[S + b], P = a->start_pos[b];
      if (n <= 0 || P < 0) continue;
      /* reading: a slot whose extend rows are not all inside the projection
       * buffer is skipped whole and flagged (the pages index the buffer with
       * the offsets and give no rule for rows outside it) */
      if (first < 0 || first + n > a->kv_rows) {
        if (rows) set_status(a->status, KVO_ST_TOKEN_RANGE);
        continue;
      }
      if (a->ratio == 1) {
        for (int64_t t = 0; t < n; ++t) {
          if (rows) {
            kvo_row r = {b, P + t, P + t, NULL, NULL, tok_kv(a, first + t),
                         tok_score(a, first + t), nr, -1};
            rows[nr] = r;
          }
          ++nr;
        }
      } else {
        for (int64_t q = P; q < P + n; ++q) {
          if (q % 2 != 1) continue;
          if (rows) {
            kvo_row r;
            r.slot = b;
            r.c = q / 2;
            r.p = q - 1;
            if (q - 1 >= P) {
              r.k0 = tok_kv(a, first + (q - 1 - P));
              r.s0 = tok_score(a, first + (q - 1 - P));
            } else {
              r.k0 = state_kv(a, b, q / 2);
              r.s0 = state_score(a, b, q / 2);
            }
            r.k1 = tok_kv(a, first + (q - P));
            r.s1 = tok_score(a, first + (q - P));
            r.latent_idx = nr;
            r.token = -1;
            rows[nr] = r;
          }
          ++nr;
        }
        int64_t last = P + n - 1;
        if (last % 2 == 0) {
          if (sw) {
            kvo_state_write w = {state_kv(a, b, last / 2), state_score(a, b, last / 2),
                                 tok_kv(a, first + n - 1), tok_score(a, first + n - 1)};
            sw[ns] = w;
          }
          ++ns;
        }
      }
    } else {
      const int64_t D = a->mode == KVO_VERIFY ? a->draft_len : 1;
      int64_t P = a->start_pos[b];
      if (P < 0) continue;
      for (int64_t j = 0; j < D; ++j) {
        int64_t q = P + j, t = (int64_t)b * D + j;
        if (a->ratio == 1) {
          if (rows) {
            kvo_row r = {b, q, q, NULL, NULL, tok_kv(a, t), tok_score(a, t), t, t};
            rows[nr] = r;
          }
          ++nr;
        } else if (q % 2 == 1) {
          if (rows) {
            kvo_row r = {b, q / 2, q - 1, NULL, NULL, tok_kv(a, t), tok_score(a, t), t, t};
            if (j > 0) {
              r.k0 = tok_kv(a, t - 1);
              r.s0 = tok_score(a, t - 1);
            } else {
              r.k0 = state_kv(a, b, q / 2);
              r.s0 = state_score(a, b, q / 2);
            }
            rows[nr] = r;
          }
          ++nr;
        } else {
          if (sw) {
            kvo_state_write w = {state_kv(a, b, q / 2), state_score(a, b, q / 2),
                                 tok_kv(a, t), tok_score(a, t)};
            sw[ns] = w;
          }
          ++ns;
        }
      }
    }
  }
  if (n_sw) *n_sw = ns;
  return nr;
}

int64_t kvo_count_rows(const kvo_compress_args* a) {
  return build_plan(a, NULL, NULL, NULL);
}

void kvo_compress(const kvo_compress_args* a) {
  int64_t ns = 0;
  int64_t nr = build_plan(a, NULL, NULL, &ns);
  kvo_row* rows = (kvo_row*)malloc(sizeof(kvo_row) * (size_t)(nr > 0 ? nr : 1));
  kvo_state_write* sw = (kvo_state_write*)malloc(sizeof(kvo_state_write) * (size_t)(ns > 0 ? ns : 1));
  build_plan(a, rows, sw, &ns);

#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < nr; ++i) {
    const kvo_row* r = &rows[i];
    if (r->p < 0 || r->p >= a->max_pos) {
      set_status(a->status, KVO_ST_POS_RANGE);
      continue;
    }
    uint16_t lat[KVO_D], z[KVO_D];
    pool_norm_rope(a, r, lat, z);
    if (r->latent_idx < a->max_out_rows) {
      memcpy(a->latent + r->latent_idx * a->latent_stride, lat, sizeof lat);
      if (a->prequant)
        memcpy(a->prequant + r->latent_idx * a->prequant_stride, z, sizeof z);
    } else {
      set_status(a->status, KVO_ST_LATENT_RANGE);
    }
    int64_t loc = row_out_loc(a, r);
    if (loc != 0)
      kvo_store_row(a->cache.layout, z, row_data(&a->cache, loc), row_scale(&a->cache, loc));
  }

  /* pending-state writes come after every row that may read the old state,
   * in token order (a later token of a slot overwrites an earlier one that
   * shares its ring entry) */
  for (int64_t i = 0; i < ns; ++i) {
    memcpy(sw[i].kv_dst, sw[i].kv, KVO_D * sizeof(uint16_t));
    if (sw[i].score)
      memcpy(sw[i].score_dst, sw[i].score, KVO_D * sizeof(uint16_t));
  }
  free(rows);
  free(sw);
}

/* ------------------------------------------------------------------------
 * One rank's share of global compressed ids [FI-dcp]: per token row t, the
 * ids of request token_to_req[t] that this rank owns, in their order,
 * mapped through the request's block-table row to this rank's physical
 * slots, written as a prefix of out_slots[t] followed by -1, with the prefix
 * length in out_lens[t].  Negative ids and other ranks' ids are dropped; a
 * row whose `valid` entry is 0 (a graph padding token) keeps nothing.
 * Readings: a request index outside the table drops the whole row
 * (KVO_ST_REQ_RANGE); a page beyond the block-table row or outside the
 * cache drops the id (KVO_ST_PT_RANGE / KVO_ST_PAGE_RANGE).  With world = 1
 * this is the single-rank mapping with the -1 entries squeezed out.
 * ---------------------------------------------------------------------- */
void kvo_dcp_filter_ids(const int32_t* ids, int64_t T, int32_t k, int64_t ids_stride,
                        const int32_t* token_to_req, int32_t n_req,
                        const int32_t* block_table, int64_t bt_stride,
                        const int32_t* valid, int32_t page_size, int64_t num_pages,
                        int32_t world, int32_t rank, int32_t interleave,
                        int32_t* out_slots, int64_t out_stride, int32_t* out_lens,
                        int32_t* status) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    int32_t* o = out_slots + t * out_stride;
    int32_t cnt = 0;
    int32_t req = token_to_req[t];
    int keep_row = !(valid && valid[t] == 0);
    if (keep_row && (req < 0 || req >= n_req)) {
      set_status(status, KVO_ST_REQ_RANGE);
      keep_row = 0;
    }
    for (int32_t i = 0; keep_row && i < k; ++i) {
      int64_t id = ids[t * ids_stride + i];
      if (id < 0) continue;
      int64_t local;
      if (kvo_dcp_owner(id, world, interleave, &local) != rank) continue;
      int64_t lp = local / page_size;
      if (lp >= bt_stride) { set_status(status, KVO_ST_PT_RANGE); continue; }
      int64_t phys = block_table[(int64_t)req * bt_stride + lp];
      if (phys < 0 || phys >= num_pages) { set_status(status, KVO_ST_PAGE_RANGE); continue; }
      o[cnt++] = (int32_t)(phys * page_size + local % page_size);
    }
    for (int32_t i = cnt; i < k; ++i) o[i] = -1;
    out_lens[t] = cnt;
  }
}

/* ------------------------------------------------------------------------
 * Array forms of the scalar functions, so that tests can sweep whole format
 * ranges without one foreign call per value.
 * ---------------------------------------------------------------------- */
void kvo_e4m3_encode_n(const double* v, int64_t n, int satfinite, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_e4m3_encode(v[i], satfinite);
}

void kvo_e2m1_encode_n(const double* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_e2m1_encode(v[i]);
}

void kvo_bf16_encode_n(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_bf16_encode(v[i]);
}

void kvo_ue8m0_n(const float* amax, int64_t n, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_ue8m0(amax[i]);
}

void kvo_fp4_scale_n(const float* amax, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_fp4_scale(amax[i]);
}

/* n rows of 512 bf16 -> n data parts (row-major) and n scale parts */
void kvo_store_row_n(int32_t layout, const uint16_t* x, int64_t n,
                     uint8_t* data, uint8_t* scale) {
  int32_t db, sb;
  if (kvo_layout_bytes(layout, &db, &sb, NULL, NULL)) return;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    kvo_store_row(layout, x + i * KVO_D, data + i * db, scale + i * sb);
}

void kvo_dequant_row_n(int32_t layout, const uint8_t* data, const uint8_t* scale,
                       int64_t n, uint16_t* out) {
  int32_t db, sb;
  if (kvo_layout_bytes(layout, &db, &sb, NULL, NULL)) return;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    kvo_dequant_row(layout, data + i * db, scale + i * sb, out + i * KVO_D);
}

void kvo_fp8_code_n(const uint16_t* x, const int32_t* E, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_fp8_code(x[i], E[i]);
}

void kvo_fp4_code_n(const uint16_t* x, const uint8_t* sc, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_fp4_code(x[i], sc[i]);
}
