/*
 * mla_oracle.c -- CPU fp64 oracle for multi-head latent attention (MLA) decode
 * over a paged KV cache, and for the packed top-k FP8 variant.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or constant generator with the HIP library, and the
 * library never calls it.
 *
 * What it computes (all arithmetic in IEEE double, inputs decoded exactly):
 *
 *   For request r, new token i in [0, s_q), head h:
 *     visible keys  j in [0, n),  n = seqlen[r]                       (non-causal)
 *                                 n = clamp(seqlen[r] - s_q + i + 1)  (causal, bottom-right)
 *     key j         = kcache[block_table[r][j / 64]][j % 64][0][0:576]
 *     score s_j     = scale * sum_{d<576} q[r][i][h][d] * key_j[d]
 *     m = max_j s_j,  l = sum_j exp(s_j - m),  lse = m + log(l)
 *     out[v]        = sum_j exp(s_j - m) / l * key_j[v]      for v < 512 (V is the
 *                                                            first 512 dims of K)
 *     n == 0  ->  out = 0, lse = -inf
 *
 *   This is the plain two-pass softmax(scale * q K^T) V of the dense MLA decode
 *   described on "Add SM80 (Ampere/A100) dense MLA decode kernel" (FlashMLA
 *   pull request 183, Summary and Design sections: 576-dim latent K shared by all
 *   query heads, 512 V columns, causal mask for multi-token queries, split-K
 *   merged by a combine step).  The split/online-softmax of the GPU path reaches
 *   the same value up to rounding, so the oracle does no splitting.
 *
 *   Sparse FP8 variant ("[SM90] Add packed selected-KV sparse decode", FlashMLA
 *   pull request 200, sections "SM90 packing kernel" and "Packed attention
 *   specialization"): a 656-byte record per token holds 512 E4M3 NoPE bytes,
 *   4 little-endian fp32 scales (one per 128 NoPE dims) and 64 little-endian
 *   bf16 RoPE values.  Key d < 512 = e4m3fn(byte d) * scale[d / 128];
 *   key 512 + e = bf16 RoPE e.  Keys are the records named by indices[r][i][k]
 *   (physical token id = page * 64 + slot) for k < topk_length[r]; no causal mask.
 *
 *   Several KV heads (the dense page's Test plan sweeps hk = 1..4): the cache
 *   is [pages][64][h_kv][576] and query head h reads KV head h / (h_q / h_kv),
 *   the query heads being grouped contiguously.
 *
 *   fp16 variant (the dense page's Summary and Test plan verify BF16 and FP16
 *   instantiations): q and the cache rows are IEEE binary16 bit patterns
 *   instead of bf16; everything else is the same.
 *
 *   Pack: workspace[row][t][s][0:656] = record(indices[row][t*64+s]) when
 *   t*64+s < topk_length, else 656 zero bytes (byte copy, no arithmetic).
 *
 *   Split partial: the same attention restricted to keys j in [j0, j1), giving
 *   a normalised partial output o and its lse; combine merges partials by
 *   L = log(sum_i exp(lse_i)), out = sum_i exp(lse_i - L) * o_i (empty parts
 *   have lse = -inf and weight 0).
 *
 * Every entry point validates indices before reading and returns a nonzero
 * status instead of reading out of range.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D_QK 576
#define D_V 512
#define PAGE 64
#define REC_BYTES 656
#define REC_NOPE 512
#define REC_SCALE_OFF 512
#define REC_ROPE_OFF 528

enum { OR_OK = 0, OR_BAD_ARG = 1, OR_BAD_PAGE = 2, OR_BAD_INDEX = 3, OR_NOMEM = 4 };

/* bf16 is the upper half of an IEEE binary32; widening it is exact. */
static double bf16_bits_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits.  Exponent 0 encodes subnormals f * 2^-24; exponent 31 encodes
 * infinities (f = 0) and NaNs. */
double oracle_f16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 10) & 0x1F;
  int f = b & 0x3FF;
  double v;
  if (e == 0x1F) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -24);          /* (f / 1024) * 2^(1 - 15) */
  else v = ldexp(1.0 + (double)f / 1024.0, e - 15);
  return sign ? -v : v;
}

static double f32le_to_f64(const uint8_t* p) {
  uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3 ("FN": finite + NaN only): 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 encodes
 * subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities. */
double oracle_e4m3fn_to_f64(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);                 /* (m / 8) * 2^(1 - 7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* ------------------------------------------------------------------ key sources */

typedef struct {
  int fp8;                   /* 0: 16-bit rows of 576; 1: 656-byte FP8 records */
  const uint16_t* kc_bf16;   /* [num_pages][64][576], bf16 or (f16 set) binary16 */
  const uint8_t* kc_rec;     /* [num_pages][64][656] */
  int64_t num_pages;
  int f16;                   /* 16-bit rows (and q) are binary16 */
  int h_kv;                  /* 16-bit rows per token (KV heads); 0 is read as 1 */
} kv_pool;

static double half_bits_to_f64(const kv_pool* p, uint16_t b) {
  return p->f16 ? oracle_f16_to_f64(b) : bf16_bits_to_f64(b);
}

/* Decode key `phys` into k[0:576]: a physical token id, or for 16-bit rows
 * with h_kv > 1 the row (token id * h_kv + KV head). */
static int load_key(const kv_pool* p, int64_t phys, double* k) {
  const int64_t rows_per_token = (!p->fp8 && p->h_kv > 1) ? p->h_kv : 1;
  if (phys < 0 || phys >= p->num_pages * PAGE * rows_per_token) return OR_BAD_INDEX;
  if (!p->fp8) {
    const uint16_t* row = p->kc_bf16 + phys * D_QK;
    for (int d = 0; d < D_QK; ++d) k[d] = half_bits_to_f64(p, row[d]);
  } else {
    const uint8_t* rec = p->kc_rec + phys * REC_BYTES;
    for (int d = 0; d < REC_NOPE; ++d) {
      double scale = f32le_to_f64(rec + REC_SCALE_OFF + 4 * (d / 128));
      k[d] = oracle_e4m3fn_to_f64(rec[d]) * scale;
    }
    for (int e = 0; e < D_QK - REC_NOPE; ++e) {
      uint16_t b = (uint16_t)(rec[REC_ROPE_OFF + 2 * e] | (rec[REC_ROPE_OFF + 2 * e + 1] << 8));
      k[REC_NOPE + e] = bf16_bits_to_f64(b);
    }
  }
  return OR_OK;
}

/* Attention of one query row over an explicit list of physical key ids.
 * Two passes: scores (kept), then the weighted sum of V = K[0:512]. */
static int attend(const kv_pool* pool, const double* q, const int64_t* keys, int64_t n, double scale,
                  double* score_buf, double* out, double* lse) {
  double k[D_QK];
  for (int v = 0; v < D_V; ++v) out[v] = 0.0;
  if (n <= 0) {
    *lse = -INFINITY;
    return OR_OK;
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    int st = load_key(pool, keys[j], k);
    if (st) return st;
    double s = 0.0;
    for (int d = 0; d < D_QK; ++d) s += q[d] * k[d];
    s *= scale;
    score_buf[j] = s;
    if (s > m) m = s;
  }
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) l += exp(score_buf[j] - m);
  for (int64_t j = 0; j < n; ++j) {
    double p = exp(score_buf[j] - m) / l;
    int st = load_key(pool, keys[j], k);
    if (st) return st;
    for (int v = 0; v < D_V; ++v) out[v] += p * k[v];
  }
  *lse = m + log(l);
  return OR_OK;
}

/* ------------------------------------------------------------------ threading */

typedef struct job job;
typedef int (*row_fn)(const job* jb, int64_t row, int64_t* key_buf, double* score_buf);

struct job {
  row_fn fn;
  int64_t rows;
  int nthreads;
  int tid;
  int status;
  const void* ctx;
  int64_t max_keys;
};

static void* worker(void* arg) {
  job* jb = (job*)arg;
  int64_t* key_buf = (int64_t*)malloc(sizeof(int64_t) * (size_t)(jb->max_keys > 0 ? jb->max_keys : 1));
  double* score_buf = (double*)malloc(sizeof(double) * (size_t)(jb->max_keys > 0 ? jb->max_keys : 1));
  if (!key_buf || !score_buf) {
    jb->status = OR_NOMEM;
  } else {
    for (int64_t row = jb->tid; row < jb->rows; row += jb->nthreads) {
      int st = jb->fn(jb, row, key_buf, score_buf);
      if (st) {
        jb->status = st;
        break;
      }
    }
  }
  free(key_buf);
  free(score_buf);
  return NULL;
}

static int run_rows(row_fn fn, const void* ctx, int64_t rows, int64_t max_keys, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 1024) nthreads = 1024;
  if ((int64_t)nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
  job* jobs = (job*)calloc((size_t)nthreads, sizeof(job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return OR_NOMEM;
  }
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].rows = rows;
    jobs[t].nthreads = nthreads;
    jobs[t].tid = t;
    jobs[t].ctx = ctx;
    jobs[t].max_keys = max_keys;
  }
  int status = OR_OK;
  if (nthreads == 1) {
    worker(&jobs[0]);
  } else {
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
      if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) break;
      ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    if (started < nthreads) status = OR_NOMEM;
  }
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status && !status) status = jobs[t].status;
  free(jobs);
  free(th);
  return status;
}

/* ------------------------------------------------------------------ dense paged decode */

typedef struct {
  kv_pool pool;
  const uint16_t* q;
  const int32_t* block_table;
  const int32_t* seqlens;
  int batch, s_q, h_q, max_pages;
  double scale;
  int causal;
  double* out;
  double* lse;
  /* split mode: keys restricted to [j0, j1) per request (NULL = whole range) */
  const int32_t* split_lo;
  const int32_t* split_hi;
} dense_ctx;

/* Number of keys query token i of a request with `seqlen` cached tokens may see. */
static int64_t visible_keys(int64_t seqlen, int s_q, int i, int causal) {
  if (!causal) return seqlen;
  int64_t n = seqlen - s_q + i + 1;
  if (n < 0) n = 0;
  if (n > seqlen) n = seqlen;
  return n;
}

static int dense_row(const job* jb, int64_t row, int64_t* key_buf, double* score_buf) {
  const dense_ctx* c = (const dense_ctx*)jb->ctx;
  int h = (int)(row % c->h_q);
  int i = (int)((row / c->h_q) % c->s_q);
  int r = (int)(row / ((int64_t)c->h_q * c->s_q));
  int64_t seqlen = c->seqlens[r];
  if (seqlen < 0 || seqlen > (int64_t)c->max_pages * PAGE) return OR_BAD_ARG;
  int64_t n = visible_keys(seqlen, c->s_q, i, c->causal);
  int64_t j0 = 0, j1 = n;
  if (c->split_lo) {
    j0 = c->split_lo[r];
    j1 = c->split_hi[r];
    if (j0 < 0) j0 = 0;
    if (j1 > n) j1 = n;
    if (j1 < j0) j1 = j0;
  }
  const int h_kv = c->pool.h_kv > 1 ? c->pool.h_kv : 1;
  const int kvh = h / (c->h_q / h_kv);  /* KV head of query head h */
  for (int64_t j = j0; j < j1; ++j) {
    int64_t page = c->block_table[(int64_t)r * c->max_pages + j / PAGE];
    if (page < 0 || page >= c->pool.num_pages) return OR_BAD_PAGE;
    key_buf[j - j0] = (page * PAGE + j % PAGE) * h_kv + kvh;
  }
  double q[D_QK];
  const uint16_t* qr = c->q + row * D_QK;
  for (int d = 0; d < D_QK; ++d) q[d] = half_bits_to_f64(&c->pool, qr[d]);
  return attend(&c->pool, q, key_buf, j1 - j0, c->scale, score_buf, c->out + row * D_V, c->lse + row);
}

/* Dense decode.  q bf16 bits [batch][s_q][h_q][576]; kcache bf16 bits
 * [num_pages][64][1][576]; block_table int32 [batch][max_pages]; seqlens int32
 * [batch].  out fp64 [batch][s_q][h_q][512]; lse fp64 [batch][s_q][h_q]. */
int oracle_mla_decode(const uint16_t* q, const uint16_t* kcache, int64_t num_pages, const int32_t* block_table,
                      int max_pages, const int32_t* seqlens, int batch, int s_q, int h_q, double scale, int causal,
                      double* out, double* lse, int nthreads) {
  if (!q || !kcache || !block_table || !seqlens || !out || !lse) return OR_BAD_ARG;
  if (batch < 0 || s_q < 1 || h_q < 1 || max_pages < 0 || num_pages < 0) return OR_BAD_ARG;
  dense_ctx c = {{0, kcache, NULL, num_pages, 0, 1}, q, block_table, seqlens, batch, s_q, h_q, max_pages,
                 scale, causal, out, lse, NULL, NULL};
  return run_rows(dense_row, &c, (int64_t)batch * s_q * h_q, (int64_t)max_pages * PAGE, nthreads);
}

/* Same, with q and kcache as IEEE binary16 bit patterns. */
int oracle_mla_decode_f16(const uint16_t* q, const uint16_t* kcache, int64_t num_pages, const int32_t* block_table,
                          int max_pages, const int32_t* seqlens, int batch, int s_q, int h_q, double scale,
                          int causal, double* out, double* lse, int nthreads) {
  if (!q || !kcache || !block_table || !seqlens || !out || !lse) return OR_BAD_ARG;
  if (batch < 0 || s_q < 1 || h_q < 1 || max_pages < 0 || num_pages < 0) return OR_BAD_ARG;
  dense_ctx c = {{0, kcache, NULL, num_pages, 1, 1}, q, block_table, seqlens, batch, s_q, h_q, max_pages,
                 scale, causal, out, lse, NULL, NULL};
  return run_rows(dense_row, &c, (int64_t)batch * s_q * h_q, (int64_t)max_pages * PAGE, nthreads);
}

/* Dense decode with h_kv KV heads: kcache [num_pages][64][h_kv][576] (bf16, or
 * binary16 if f16), query head h reads KV head h / (h_q / h_kv); h_kv divides h_q. */
int oracle_mla_decode_hkv(const uint16_t* q, const uint16_t* kcache, int64_t num_pages, const int32_t* block_table,
                          int max_pages, const int32_t* seqlens, int batch, int s_q, int h_q, int h_kv, int f16,
                          double scale, int causal, double* out, double* lse, int nthreads) {
  if (!q || !kcache || !block_table || !seqlens || !out || !lse) return OR_BAD_ARG;
  if (batch < 0 || s_q < 1 || h_q < 1 || max_pages < 0 || num_pages < 0) return OR_BAD_ARG;
  if (h_kv < 1 || h_q % h_kv != 0) return OR_BAD_ARG;
  dense_ctx c = {{0, kcache, NULL, num_pages, f16 ? 1 : 0, h_kv}, q, block_table, seqlens, batch, s_q, h_q,
                 max_pages, scale, causal, out, lse, NULL, NULL};
  return run_rows(dense_row, &c, (int64_t)batch * s_q * h_q, (int64_t)max_pages * PAGE, nthreads);
}

/* Split partial of the dense decode: for each request r only keys j in
 * [split_lo[r], split_hi[r]) (intersected with the visible range) take part.
 * The result is the normalised partial output and its lse. */
int oracle_mla_decode_partial(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                              const int32_t* block_table, int max_pages, const int32_t* seqlens, int batch, int s_q,
                              int h_q, double scale, int causal, const int32_t* split_lo, const int32_t* split_hi,
                              double* out, double* lse, int nthreads) {
  if (!q || !kcache || !block_table || !seqlens || !out || !lse || !split_lo || !split_hi) return OR_BAD_ARG;
  if (batch < 0 || s_q < 1 || h_q < 1 || max_pages < 0 || num_pages < 0) return OR_BAD_ARG;
  dense_ctx c = {{0, kcache, NULL, num_pages, 0, 1}, q, block_table, seqlens, batch, s_q, h_q, max_pages,
                 scale, causal, out, lse, split_lo, split_hi};
  return run_rows(dense_row, &c, (int64_t)batch * s_q * h_q, (int64_t)max_pages * PAGE, nthreads);
}

/* Merge `nsplit` partials of one row: o [nsplit][512], lse [nsplit]. */
int oracle_lse_combine(int nsplit, const double* o, const double* lse, double* out, double* lse_out) {
  if (nsplit < 0 || (nsplit > 0 && (!o || !lse)) || !out || !lse_out) return OR_BAD_ARG;
  double m = -INFINITY;
  for (int s = 0; s < nsplit; ++s)
    if (lse[s] > m) m = lse[s];
  for (int v = 0; v < D_V; ++v) out[v] = 0.0;
  if (m == -INFINITY) {
    *lse_out = -INFINITY;
    return OR_OK;
  }
  double total = 0.0;
  for (int s = 0; s < nsplit; ++s) total += exp(lse[s] - m);
  double L = m + log(total);
  for (int s = 0; s < nsplit; ++s) {
    double w = exp(lse[s] - L);
    for (int v = 0; v < D_V; ++v) out[v] += w * o[(int64_t)s * D_V + v];
  }
  *lse_out = L;
  return OR_OK;
}

/* ------------------------------------------------------------------ sparse FP8 decode */

typedef struct {
  kv_pool pool;
  const uint16_t* q;
  const int32_t* indices;     /* [batch][s_q][cap] physical token ids */
  const int32_t* topk_length; /* [batch] */
  int batch, s_q, h_q, cap;
  double scale;
  double* out;
  double* lse;
} sparse_ctx;

static int sparse_row(const job* jb, int64_t row, int64_t* key_buf, double* score_buf) {
  const sparse_ctx* c = (const sparse_ctx*)jb->ctx;
  int i = (int)((row / c->h_q) % c->s_q);
  int r = (int)(row / ((int64_t)c->h_q * c->s_q));
  int64_t n = c->topk_length[r];
  if (n < 0 || n > c->cap) return OR_BAD_ARG;
  const int32_t* idx = c->indices + ((int64_t)r * c->s_q + i) * c->cap;
  for (int64_t k = 0; k < n; ++k) key_buf[k] = idx[k];
  double q[D_QK];
  const uint16_t* qr = c->q + row * D_QK;
  for (int d = 0; d < D_QK; ++d) q[d] = bf16_bits_to_f64(qr[d]);
  return attend(&c->pool, q, key_buf, n, c->scale, score_buf, c->out + row * D_V, c->lse + row);
}

/* Sparse decode over top-k FP8 records.  kcache_rec u8 [num_pages][64][1][656];
 * indices int32 [batch][s_q][cap]; topk_length int32 [batch]. */
int oracle_mla_sparse_decode(const uint16_t* q, const uint8_t* kcache_rec, int64_t num_pages, const int32_t* indices,
                             const int32_t* topk_length, int batch, int s_q, int h_q, int cap, double scale,
                             double* out, double* lse, int nthreads) {
  if (!q || !kcache_rec || !indices || !topk_length || !out || !lse) return OR_BAD_ARG;
  if (batch < 0 || s_q < 1 || h_q < 1 || cap < 0 || num_pages < 0) return OR_BAD_ARG;
  sparse_ctx c = {{1, NULL, kcache_rec, num_pages, 0, 0}, q, indices, topk_length, batch, s_q, h_q, cap, scale, out, lse};
  return run_rows(sparse_row, &c, (int64_t)batch * s_q * h_q, cap, nthreads);
}

/* Dequantise the record at physical token id `phys` into k[0:576] (for tests). */
int oracle_decode_record(const uint8_t* kcache_rec, int64_t num_pages, int64_t phys, double* k) {
  kv_pool p = {1, NULL, kcache_rec, num_pages, 0, 0};
  return load_key(&p, phys, k);
}

/* ------------------------------------------------------------------ pack */

/* workspace u8 [batch*s_q][cap/64][64][656].  Rows are (request, token). */
int oracle_pack_selected_kv(const uint8_t* kcache_rec, int64_t num_pages, const int32_t* indices,
                            const int32_t* topk_length, int batch, int s_q, int cap, uint8_t* workspace) {
  if (!kcache_rec || !indices || !topk_length || !workspace) return OR_BAD_ARG;
  if (batch < 0 || s_q < 1 || cap < 0 || cap % PAGE != 0) return OR_BAD_ARG;
  for (int r = 0; r < batch; ++r) {
    int64_t n = topk_length[r];
    if (n < 0 || n > cap) return OR_BAD_ARG;
    for (int i = 0; i < s_q; ++i) {
      int64_t row = (int64_t)r * s_q + i;
      const int32_t* idx = indices + row * cap;
      uint8_t* dst_row = workspace + row * (int64_t)cap * REC_BYTES;
      for (int64_t k = 0; k < cap; ++k) {
        /* tile k/64, slot k%64: with 64 records per tile this is record k of the row */
        uint8_t* dst = dst_row + ((k / PAGE) * PAGE + (k % PAGE)) * REC_BYTES;
        if (k < n) {
          int64_t phys = idx[k];
          if (phys < 0 || phys >= num_pages * PAGE) return OR_BAD_INDEX;
          memcpy(dst, kcache_rec + phys * REC_BYTES, REC_BYTES);
        } else {
          memset(dst, 0, REC_BYTES);
        }
      }
    }
  }
  return OR_OK;
}
