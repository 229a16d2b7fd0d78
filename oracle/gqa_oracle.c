/*
 * gqa_oracle.c -- plain, slow, fp64 CPU oracle for Gemma-4-31B decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test-suite, the smoke check and the
 * benchmark's cpu_baseline leg use it.  It shares no code, header, table or
 * constant with the HIP library; it is the definition written out, nothing more.
 *
 * What it computes (the attn.core rows of the "Compute-graph nodes" table on
 * the gemma-4-31B Model Spec page, docs.theformalera.com):
 *
 *   slidingDecodeGQA : o[b,h] = sum_s softmax_s(1 * <q[b,h], k[b,s,h/2]>) * v[b,s,h/2]
 *                      over the last 1024 positions below seq_lens[b]
 *   decodeGQA        : the same with k/v head h/8 and every position s < seq_lens[b]
 *
 * Tensor shapes follow the "Tensors of the main nodes" table of the same page:
 * q [B,32,D], k/v [B,S,kv,D], seq_lens [B], o [B,32,D].  The paged form uses the
 * page size 16 named in the "At a glance" table ("Shape domain" row).
 *
 * Readings where the pages leave a step open (each is also listed with the
 * design notes):
 *   - window: the query is the newest token, already appended to the cache
 *     (compact forward pass of "Gemma 4 31B-it Text Architecture", which
 *     appends K/V before attention and masks keys t-1024 < s <= t), so with
 *     t = L-1 the window is [max(0, L-W), L);
 *   - h/G is floor division (repeat_kv gives query heads G*j .. G*j+G-1 the
 *     kv head j);
 *   - scale is exactly 1 and no logit soft-cap applies to attention;
 *   - L <= 0 yields a zero row (outside the shape domain S >= 1);
 *   - paged pool layout [num_pages, 16, kv, D], logical position s lives in
 *     physical page block_table[b][s/16], slot s%16;
 *   - a cache capped at R positions (the retrofit page's per-layer caches
 *     "capped at its window size") is a ring: position s lives in slot s % R
 *     of [B, R, kv, D], which holds the last R positions written.
 *
 * Arithmetic: every input element is widened exactly to double (bf16 by
 * placing its 16 bits in the top half of an IEEE single), the dot products,
 * the max, the exponentials, the normaliser and the weighted sum are all
 * formed in double, in position order, with no blocking or reordering.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_HEADS 32
#define ORC_PAGE 16

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum {
  ORC_OK = 0,
  ORC_ERR_ARG = -1,
  ORC_ERR_SEQLEN = -2,
  ORC_ERR_PAGE = -3,
  ORC_ERR_NOMEM = -4
};

typedef struct {
  int dtype;
  const void *q, *k, *v;
  const int32_t *seq_lens;
  const int32_t *block_table; /* NULL: contiguous cache */
  int32_t B, cap, max_pages, num_pages, KV, D, window;
  int32_t ring;        /* > 0: contiguous ring of `ring` slots, position s in slot s % ring */
  const void *w_k;     /* non-NULL: keys rebuilt from values (global layers) */
  const int32_t *rows; /* (b, h) pairs -- prefill: (token row, h) -- or NULL for every row */
  int32_t n_rows;
  const int32_t *cu_q; /* non-NULL: prefill, query rows cu_q[b] .. cu_q[b+1]-1 of sequence b */
  int32_t N;           /* prefill: query rows */
  double *out;
  /* shared work counter and first error */
  int32_t next;
  int32_t err;
  pthread_mutex_t mu;
} orc_job;

/* Exact widening of one stored element to double. */
static double orc_elem(const void *base, int dtype, size_t idx) {
  if (dtype == ORC_F32) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Element offset of row (b, position s, kv head g) in k or v; -1 if the
 * block table names a page outside the pool. */
static int64_t orc_row_offset(const orc_job *j, int b, int64_t s, int g) {
  if (j->ring > 0) return (((int64_t)b * j->ring + s % j->ring) * j->KV + g) * (int64_t)j->D;
  if (j->block_table == NULL)
    return (((int64_t)b * j->cap + s) * j->KV + g) * (int64_t)j->D;
  int32_t page = j->block_table[(int64_t)b * j->max_pages + s / ORC_PAGE];
  if (page < 0 || page >= j->num_pages) return -1;
  return (((int64_t)page * ORC_PAGE + s % ORC_PAGE) * j->KV + g) * (int64_t)j->D;
}

static void orc_rope(double *y, int D, long pos, double theta, int active);

/* Key row of position s when keys are rebuilt from values (decodeGQA layers
 * store values only, keys = values on those layers): k = rope(w_k * v, s). */
static void orc_key_from_value(const orc_job *j, int64_t off, int64_t s, double *k) {
  for (int d = 0; d < j->D; ++d)
    k[d] = orc_elem(j->w_k, j->dtype, (size_t)d) * orc_elem(j->v, j->dtype, (size_t)off + d);
  orc_rope(k, j->D, (long)s, 1e6, 64);
}

/* One output row o[b,h,:] written to out[0:D]. */
static int orc_one_row(const orc_job *j, int b, int h, double *out) {
  const int D = j->D;
  const int G = ORC_HEADS / j->KV; /* query heads per kv head */
  const int g = h / G;             /* kv head of query head h */
  const int64_t L = j->seq_lens[b];
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (j->ring == 0 && L > j->cap) return ORC_ERR_SEQLEN;
  if (L <= 0) return ORC_OK;
  const int64_t lo = (j->window > 0 && L > j->window) ? L - j->window : 0;
  const int64_t n = L - lo;

  double *z = (double *)malloc(((size_t)n + (size_t)D) * sizeof(double));
  if (!z) return ORC_ERR_NOMEM;
  const size_t qoff = ((size_t)b * ORC_HEADS + h) * (size_t)D;

  /* logits z_s = 1 * <q[b,h], k[b,s,g]> */
  for (int64_t s = lo; s < L; ++s) {
    int64_t off = orc_row_offset(j, b, s, g);
    if (off < 0) { free(z); return ORC_ERR_PAGE; }
    double acc = 0.0;
    if (j->w_k) {
      double *krow = z + n; /* scratch after the logits */
      orc_key_from_value(j, off, s, krow);
      for (int d = 0; d < D; ++d) acc += orc_elem(j->q, j->dtype, qoff + d) * krow[d];
    } else {
      for (int d = 0; d < D; ++d)
        acc += orc_elem(j->q, j->dtype, qoff + d) * orc_elem(j->k, j->dtype, (size_t)off + d);
    }
    z[s - lo] = acc;
  }
  /* softmax over the window */
  double m = -INFINITY;
  for (int64_t i = 0; i < n; ++i)
    if (z[i] > m) m = z[i];
  double l = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    z[i] = exp(z[i] - m);
    l += z[i];
  }
  /* weighted sum of the value rows */
  for (int64_t s = lo; s < L; ++s) {
    int64_t off = orc_row_offset(j, b, s, g);
    const double p = z[s - lo];
    for (int d = 0; d < D; ++d) out[d] += p * orc_elem(j->v, j->dtype, (size_t)off + d);
  }
  for (int d = 0; d < D; ++d) out[d] /= l;
  free(z);
  return ORC_OK;
}

/* Prefill: output row o[n,h,:] of query row n (a token of a chunk appended to
 * the cache just before attention; "Prefill, Cache, and Long Context" and
 * the compact forward pass of the architecture page).  Token t of the T_b
 * tokens of sequence b sits at position p = seq_lens[b] - T_b + t
 * (positions = past_seen_tokens + arange(T_current), past_seen = L - T) and
 * attends to the keys the masks keep: full mask s <= p, sliding mask
 * p - W < s <= p.  The rest is the decode definition above. */
static int orc_prefill_row(const orc_job *j, int n, int h, double *out) {
  const int D = j->D;
  const int kvh = h / (ORC_HEADS / j->KV); /* kv head of query head h */
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  int b = 0; /* the sequence owning query row n */
  while (b < j->B && j->cu_q[b + 1] <= n) ++b;
  if (b >= j->B) return ORC_ERR_ARG;
  const int64_t T_b = j->cu_q[b + 1] - j->cu_q[b];
  const int64_t Lb = j->seq_lens[b];
  if (Lb > j->cap) return ORC_ERR_SEQLEN;
  const int64_t pos = Lb - T_b + (n - j->cu_q[b]);
  if (pos < 0) return ORC_OK; /* chunk longer than the sequence: outside the domain */
  /* keys kept by the mask: full s <= pos; sliding pos - W < s <= pos */
  const int64_t first = (j->window > 0 && pos - j->window + 1 > 0) ? pos - j->window + 1 : 0;
  const int64_t count = pos - first + 1;

  double *score = (double *)malloc((size_t)count * sizeof(double));
  if (!score) return ORC_ERR_NOMEM;
  const size_t q_at = ((size_t)n * ORC_HEADS + h) * (size_t)D;
  for (int64_t s = first; s <= pos; ++s) {
    const int64_t at = orc_row_offset(j, b, s, kvh);
    if (at < 0) { free(score); return ORC_ERR_PAGE; }
    double dot = 0.0;
    for (int d = 0; d < D; ++d)
      dot += orc_elem(j->q, j->dtype, q_at + d) * orc_elem(j->k, j->dtype, (size_t)at + d);
    score[s - first] = dot; /* scale 1 */
  }
  double top = -INFINITY;
  for (int64_t i = 0; i < count; ++i) top = score[i] > top ? score[i] : top;
  double total = 0.0;
  for (int64_t i = 0; i < count; ++i) {
    score[i] = exp(score[i] - top);
    total += score[i];
  }
  for (int64_t s = first; s <= pos; ++s) {
    const int64_t at = orc_row_offset(j, b, s, kvh);
    for (int d = 0; d < D; ++d)
      out[d] += score[s - first] * orc_elem(j->v, j->dtype, (size_t)at + d);
  }
  for (int d = 0; d < D; ++d) out[d] = out[d] / total;
  free(score);
  return ORC_OK;
}

static void *orc_worker(void *arg) {
  orc_job *j = (orc_job *)arg;
  for (;;) {
    pthread_mutex_lock(&j->mu);
    int32_t r = j->next++;
    int32_t bad = j->err;
    pthread_mutex_unlock(&j->mu);
    if (r >= j->n_rows || bad) break;
    int b, h;
    if (j->rows) {
      b = j->rows[2 * r];
      h = j->rows[2 * r + 1];
    } else {
      b = r / ORC_HEADS;
      h = r % ORC_HEADS;
    }
    int rc;
    if (j->cu_q) /* (b, h) is (query row, head) */
      rc = (b < 0 || b >= j->N || h < 0 || h >= ORC_HEADS)
               ? ORC_ERR_ARG
               : orc_prefill_row(j, b, h, j->out + (size_t)r * j->D);
    else
      rc = (b < 0 || b >= j->B || h < 0 || h >= ORC_HEADS)
               ? ORC_ERR_ARG
               : orc_one_row(j, b, h, j->out + (size_t)r * j->D);
    if (rc) {
      pthread_mutex_lock(&j->mu);
      if (!j->err) j->err = rc;
      pthread_mutex_unlock(&j->mu);
    }
  }
  return NULL;
}

/*
 * oracle_gqa_decode
 *   dtype        ORC_F32 or ORC_BF16 (q, k, v share it)
 *   q            [B, 32, D]
 *   k, v         contiguous: [B, cap, KV, D]; paged: [num_pages, 16, KV, D]
 *   seq_lens     [B] int32
 *   block_table  NULL (contiguous) or [B, max_pages] int32 (paged; cap must
 *                then equal max_pages*16)
 *   KV, D        16/256 for slidingDecodeGQA, 4/512 for decodeGQA
 *   window       1024 for slidingDecodeGQA, <= 0 for no window
 *   rows         n_rows (b, h) pairs, or NULL for all B*32 rows in order
 *   out          [n_rows, D] doubles
 *   nthreads     worker threads (>= 1)
 * Returns 0 or a negative ORC_ERR_* code.
 */
static int orc_run(int dtype, const void *q, const void *k, const void *v, const void *w_k,
                   const int32_t *cu_q, int32_t N, const int32_t *seq_lens,
                   const int32_t *block_table, int32_t B, int32_t cap, int32_t ring,
                   int32_t max_pages, int32_t num_pages, int32_t KV, int32_t D,
                   int32_t window, const int32_t *rows, int32_t n_rows, double *out,
                   int32_t nthreads) {
  if (!q || !(k || w_k) || !v || !seq_lens || !out) return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_ARG;
  if (B < 1 || cap < 1 || KV < 1 || ORC_HEADS % KV != 0 || D < 1) return ORC_ERR_ARG;
  if (w_k && !(KV == 4 && D == 512)) return ORC_ERR_ARG;
  if (block_table && (max_pages < 1 || num_pages < 1 || cap != max_pages * ORC_PAGE))
    return ORC_ERR_ARG;
  /* a ring holds the window: every attended position still has its slot */
  if (ring < 0 || (ring > 0 && (block_table || cu_q || window < 1 || window > ring)))
    return ORC_ERR_ARG;
  if (cu_q) {
    if (N < 0 || cu_q[0] != 0 || cu_q[B] != N) return ORC_ERR_ARG;
    for (int b = 0; b < B; ++b)
      if (cu_q[b + 1] < cu_q[b]) return ORC_ERR_ARG;
  }
  if (!rows) n_rows = (cu_q ? N : B) * ORC_HEADS;
  if (n_rows < 0) return ORC_ERR_ARG;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;

  orc_job j;
  memset(&j, 0, sizeof j);
  j.dtype = dtype; j.q = q; j.k = k; j.v = v; j.w_k = w_k;
  j.seq_lens = seq_lens; j.block_table = block_table;
  j.B = B; j.cap = cap; j.ring = ring; j.max_pages = max_pages; j.num_pages = num_pages;
  j.KV = KV; j.D = D; j.window = window;
  j.rows = rows; j.n_rows = n_rows; j.out = out;
  j.cu_q = cu_q; j.N = N;
  pthread_mutex_init(&j.mu, NULL);

  pthread_t th[256];
  int started = 0;
  for (int t = 1; t < nthreads; ++t)
    if (pthread_create(&th[started], NULL, orc_worker, &j) == 0) ++started;
  orc_worker(&j);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&j.mu);
  return j.err;
}

/*
 * oracle_gqa_decode
 *   dtype        ORC_F32 or ORC_BF16 (q, k, v share it)
 *   q            [B, 32, D]
 *   k, v         contiguous: [B, cap, KV, D]; paged: [num_pages, 16, KV, D]
 *   seq_lens     [B] int32
 *   block_table  NULL (contiguous) or [B, max_pages] int32 (paged; cap must
 *                then equal max_pages*16)
 *   KV, D        16/256 for slidingDecodeGQA, 4/512 for decodeGQA
 *   window       1024 for slidingDecodeGQA, <= 0 for no window
 *   rows         n_rows (b, h) pairs, or NULL for all B*32 rows in order
 *   out          [n_rows, D] doubles
 *   nthreads     worker threads (>= 1)
 * Returns 0 or a negative ORC_ERR_* code.
 */
int oracle_gqa_decode(int dtype, const void *q, const void *k, const void *v,
                      const int32_t *seq_lens, const int32_t *block_table, int32_t B,
                      int32_t cap, int32_t max_pages, int32_t num_pages, int32_t KV,
                      int32_t D, int32_t window, const int32_t *rows, int32_t n_rows,
                      double *out, int32_t nthreads) {
  return orc_run(dtype, q, k, v, NULL, NULL, 0, seq_lens, block_table, B, cap, 0, max_pages,
                 num_pages, KV, D, window, rows, n_rows, out, nthreads);
}

/*
 * oracle_gqa_decode_k_from_v -- decodeGQA over a cache that stores values
 * only.  On the global layers values are keys (Model Spec page, "What to
 * watch for": values = keys; its attn.qk_norm / attn.v_norm / attn.rope rows:
 * v = v_norm(x), k = rope(qk_norm(x) with weight w_k)), so the key of cached
 * position s is k_s = rope(w_k * v_s, s) with theta 1e6 over the first 64 of
 * the 256 pairs (i, i+256).  Arguments as oracle_gqa_decode with KV = 4,
 * D = 512, the value cache in v and the weight w_k [512] (same dtype).
 */
int oracle_gqa_decode_k_from_v(int dtype, const void *q, const void *v, const void *w_k,
                               const int32_t *seq_lens, const int32_t *block_table, int32_t B,
                               int32_t cap, int32_t max_pages, int32_t num_pages,
                               const int32_t *rows, int32_t n_rows, double *out,
                               int32_t nthreads) {
  if (!w_k) return ORC_ERR_ARG;
  return orc_run(dtype, q, NULL, v, w_k, NULL, 0, seq_lens, block_table, B, cap, 0, max_pages,
                 num_pages, 4, 512, 0, rows, n_rows, out, nthreads);
}

/*
 * oracle_gqa_decode_ring -- slidingDecodeGQA over a cache capped at `ring`
 * positions.  The retrofit page ("Progressive Window Assignment") gives each
 * sliding layer its own KV cache capped at its window size; read as a ring,
 * position s lives in slot s % ring of k, v [B, ring, KV, D], so the slots
 * hold the last `ring` positions and the window [max(0, L-W), L) needs
 * window <= ring.  Otherwise as oracle_gqa_decode (contiguous; seq_lens may
 * exceed ring).
 */
int oracle_gqa_decode_ring(int dtype, const void *q, const void *k, const void *v,
                           const int32_t *seq_lens, int32_t B, int32_t ring, int32_t KV,
                           int32_t D, int32_t window, const int32_t *rows, int32_t n_rows,
                           double *out, int32_t nthreads) {
  if (ring < 1) return ORC_ERR_ARG;
  return orc_run(dtype, q, k, v, NULL, NULL, 0, seq_lens, NULL, B, ring, ring, 0, 0, KV, D,
                 window, rows, n_rows, out, nthreads);
}

/*
 * oracle_gqa_prefill -- attention of a chunk of new tokens per sequence
 * (prefill / chunked prefill: "Prefill, Cache, and Long Context" on the
 * architecture page; the masks of its compact forward pass).  The chunk's K/V
 * rows are already in the cache: sequence b holds seq_lens[b] positions, the
 * last T_b = cu_q[b+1] - cu_q[b] of which are its query tokens.
 *   q        [N, 32, D], query rows of sequence b at cu_q[b] .. cu_q[b+1]-1
 *   cu_q     [B+1] int32, cu_q[0] = 0, non-decreasing, cu_q[B] = N
 *   k, v, seq_lens, block_table, cap, max_pages, num_pages, KV, D, window:
 *            as oracle_gqa_decode (window <= 0: full causal mask)
 *   rows     n_rows (query row, head) pairs, or NULL for all N*32 rows
 *   out      [n_rows, D] doubles
 * A token whose position would be negative (T_b > seq_lens[b]) gets a zero row.
 */
int oracle_gqa_prefill(int dtype, const void *q, const void *k, const void *v,
                       const int32_t *cu_q, const int32_t *seq_lens,
                       const int32_t *block_table, int32_t B, int32_t N, int32_t cap,
                       int32_t max_pages, int32_t num_pages, int32_t KV, int32_t D,
                       int32_t window, const int32_t *rows, int32_t n_rows, double *out,
                       int32_t nthreads) {
  if (!cu_q || !k) return ORC_ERR_ARG;
  return orc_run(dtype, q, k, v, NULL, cu_q, N, seq_lens, block_table, B, cap, 0, max_pages,
                 num_pages, KV, D, window, rows, n_rows, out, nthreads);
}

/*
 * ---- KV append with the per-head norms and RoPE of the new token ----------
 *
 * The nodes between the projections and attn.core on the gemma-4-31B Model
 * Spec page ("Compute-graph nodes" table), applied to one new token per
 * sequence whose position is pos = seq_lens[b] - 1 (the cache already counts
 * it, as the architecture page's compact forward pass appends before
 * attending):
 *   attn.qk_norm  per head: y_i = x_i / sqrt(sum_j x_j^2 / D + eps) * w_i
 *                 (one weight vector of length D for q, one for k)
 *   attn.v_norm   per head: y_i = x_i / sqrt(sum_j x_j^2 / D + eps)
 *   attn.rope     rotate pairs (i, i + D/2) by pos * theta^(-2i/D) for
 *                 i < active, other coordinates unchanged:
 *                 (a, b) -> (a cos - b sin, a sin + b cos)
 *                 sliding: D = 256, theta = 1e4, active = 128
 *                 global:  D = 512, theta = 1e6, active = 64
 *   values = keys on global layers: v_raw is k_raw.
 * Outputs (double): q_out [B,32,D] = rope(qk_norm(q_raw, w_q)),
 * k_row [B,KV,D] = rope(qk_norm(k_raw, w_k)), v_row [B,KV,D] = v_norm(v_raw);
 * pos_out[b] = seq_lens[b] - 1.  Sequences with seq_lens[b] < 1 get zero rows
 * and pos_out = -1 (nothing to append).
 */

#define ORC_EPS 1e-6

static void orc_rms(const double* x, int D, const double* w, double* y) {
  double ss = 0.0;
  for (int d = 0; d < D; ++d) ss += x[d] * x[d];
  const double inv = 1.0 / sqrt(ss / D + ORC_EPS);
  for (int d = 0; d < D; ++d) y[d] = x[d] * inv * (w ? w[d] : 1.0);
}

static void orc_rope(double* y, int D, long pos, double theta, int active) {
  const int h = D / 2;
  for (int i = 0; i < active; ++i) {
    const double ang = (double)pos * pow(theta, -2.0 * i / D);
    const double c = cos(ang), s = sin(ang);
    const double a = y[i], b = y[i + h];
    y[i] = a * c - b * s;
    y[i + h] = a * s + b * c;
  }
}

/*
 * oracle_gqa_append_rows
 *   dtype      ORC_F32 or ORC_BF16 for q_raw, k_raw, v_raw, w_q, w_k
 *   q_raw      [B, 32, D];  k_raw, v_raw [B, KV, D] (v_raw unused when KV = 4)
 *   w_q, w_k   [D]
 *   KV, D      16/256 (sliding) or 4/512 (global)
 * Returns 0 or ORC_ERR_ARG.
 */
int oracle_gqa_append_rows(int dtype, const void* q_raw, const void* k_raw, const void* v_raw,
                           const void* w_q, const void* w_k, const int32_t* seq_lens, int32_t B,
                           int32_t KV, int32_t D, double* q_out, double* k_row, double* v_row,
                           int32_t* pos_out) {
  if (!q_raw || !k_raw || !w_q || !w_k || !seq_lens || !q_out || !k_row || !v_row || !pos_out)
    return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_ARG;
  const int global = KV == 4;
  if (!(KV == 16 && D == 256) && !(KV == 4 && D == 512)) return ORC_ERR_ARG;
  if (!global && !v_raw) return ORC_ERR_ARG;
  const double theta = global ? 1e6 : 1e4;
  const int active = global ? 64 : 128;
  double* wq = (double*)malloc(sizeof(double) * D);
  double* wk = (double*)malloc(sizeof(double) * D);
  double* x = (double*)malloc(sizeof(double) * D);
  if (!wq || !wk || !x) { free(wq); free(wk); free(x); return ORC_ERR_NOMEM; }
  for (int d = 0; d < D; ++d) {
    wq[d] = orc_elem(w_q, dtype, d);
    wk[d] = orc_elem(w_k, dtype, d);
  }
  for (int b = 0; b < B; ++b) {
    const long pos = (long)seq_lens[b] - 1;
    pos_out[b] = pos >= 0 ? (int32_t)pos : -1;
    for (int h = 0; h < ORC_HEADS; ++h) {
      double* y = q_out + ((size_t)b * ORC_HEADS + h) * D;
      if (pos < 0) { for (int d = 0; d < D; ++d) y[d] = 0.0; continue; }
      for (int d = 0; d < D; ++d) x[d] = orc_elem(q_raw, dtype, ((size_t)b * ORC_HEADS + h) * D + d);
      orc_rms(x, D, wq, y);
      orc_rope(y, D, pos, theta, active);
    }
    for (int g = 0; g < KV; ++g) {
      double* yk = k_row + ((size_t)b * KV + g) * D;
      double* yv = v_row + ((size_t)b * KV + g) * D;
      if (pos < 0) { for (int d = 0; d < D; ++d) yk[d] = yv[d] = 0.0; continue; }
      for (int d = 0; d < D; ++d) x[d] = orc_elem(k_raw, dtype, ((size_t)b * KV + g) * D + d);
      orc_rms(x, D, wk, yk);
      orc_rope(yk, D, pos, theta, active);
      if (!global)
        for (int d = 0; d < D; ++d) x[d] = orc_elem(v_raw, dtype, ((size_t)b * KV + g) * D + d);
      orc_rms(x, D, NULL, yv);  /* global: values are the raw keys, unit-normalised */
    }
  }
  free(wq); free(wk); free(x);
  return ORC_OK;
}
