/*
 * Host-only driver that runs every entry point of the fp64 C oracle
 * (oracle/gqa_oracle.c) on small ragged, paged, windowed, ring and varlen
 * inputs held in exact-size heap buffers, plus the argument checks.  It is
 * built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitized.py, so any read or write outside a buffer, or
 * any undefined arithmetic, in the oracle ends the run with a report.
 * Test infrastructure only; the numbers it computes are not checked here
 * (the oracle's pins do that), only that every call returns the expected
 * status and every output element is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gqa_decode(int dtype, const void *q, const void *k, const void *v,
                      const int32_t *seq_lens, const int32_t *block_table, int32_t B,
                      int32_t cap, int32_t max_pages, int32_t num_pages, int32_t KV,
                      int32_t D, int32_t window, const int32_t *rows, int32_t n_rows,
                      double *out, int32_t nthreads);
int oracle_gqa_decode_k_from_v(int dtype, const void *q, const void *v, const void *w_k,
                               const int32_t *seq_lens, const int32_t *block_table, int32_t B,
                               int32_t cap, int32_t max_pages, int32_t num_pages,
                               const int32_t *rows, int32_t n_rows, double *out,
                               int32_t nthreads);
int oracle_gqa_decode_ring(int dtype, const void *q, const void *k, const void *v,
                           const int32_t *seq_lens, int32_t B, int32_t ring, int32_t KV,
                           int32_t D, int32_t window, const int32_t *rows, int32_t n_rows,
                           double *out, int32_t nthreads);
int oracle_gqa_prefill(int dtype, const void *q, const void *k, const void *v,
                       const int32_t *cu_q, const int32_t *seq_lens,
                       const int32_t *block_table, int32_t B, int32_t N, int32_t cap,
                       int32_t max_pages, int32_t num_pages, int32_t KV, int32_t D,
                       int32_t window, const int32_t *rows, int32_t n_rows, double *out,
                       int32_t nthreads);
int oracle_gqa_append_rows(int dtype, const void *q_raw, const void *k_raw, const void *v_raw,
                           const void *w_q, const void *w_k, const int32_t *seq_lens, int32_t B,
                           int32_t KV, int32_t D, double *q_out, double *k_row, double *v_row,
                           int32_t *pos_out);

enum { F32 = 0, BF16 = 1, HEADS = 32, PAGE = 16 };

static int failures = 0;
static uint64_t rng = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* xorshift64*, in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* n elements of the dtype, each a value in [-1, 1); bf16 keeps the top half of
 * the float's bits */
static void *fill(int dtype, size_t n) {
  if (n == 0) n = 1;
  if (dtype == F32) {
    float *p = malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = (float)uniform();
    return p;
  }
  uint16_t *p = malloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i) {
    const float f = (float)uniform();
    uint32_t u;
    memcpy(&u, &f, 4);
    p[i] = (uint16_t)(u >> 16);
  }
  return p;
}

static void expect(const char *what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static void expect_finite(const char *what, const double *x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) {
      fprintf(stderr, "FAIL %s: element %zu is not finite\n", what, i);
      ++failures;
      return;
    }
}

/* a block table [B, max_pages] over a pool of B*max_pages pages, in a
 * scrambled order; entries past a sequence's pages stay valid too */
static int32_t *block_table(int B, int max_pages) {
  const int n = B * max_pages;
  int32_t *t = malloc((size_t)n * sizeof *t);
  for (int i = 0; i < n; ++i) t[i] = (int32_t)((i * 7 + 3) % n);
  return t;
}

static void decode_case(int dtype, int KV, int D, int window, int paged, int threads) {
  const int B = 3;
  const int32_t lens[3] = {1, 17, 70};
  const int max_pages = 5, cap = paged ? max_pages * PAGE : 70;
  const int num_pages = B * max_pages;
  const size_t kv_elems = paged ? (size_t)num_pages * PAGE * KV * D : (size_t)B * cap * KV * D;
  void *q = fill(dtype, (size_t)B * HEADS * D);
  void *k = fill(dtype, kv_elems);
  void *v = fill(dtype, kv_elems);
  int32_t *bt = paged ? block_table(B, max_pages) : NULL;
  double *out = malloc((size_t)B * HEADS * D * sizeof *out);
  char what[96];
  snprintf(what, sizeof what, "decode dtype %d KV %d window %d paged %d", dtype, KV, window,
           paged);
  expect(what, oracle_gqa_decode(dtype, q, k, v, lens, bt, B, cap, paged ? max_pages : 0,
                                 paged ? num_pages : 0, KV, D, window, NULL, 0, out, threads),
         0);
  expect_finite(what, out, (size_t)B * HEADS * D);
  /* a subset of (b, h) rows */
  const int32_t rows[6] = {2, 31, 0, 0, 1, 7};
  expect(what, oracle_gqa_decode(dtype, q, k, v, lens, bt, B, cap, paged ? max_pages : 0,
                                 paged ? num_pages : 0, KV, D, window, rows, 3, out, threads),
         0);
  expect_finite(what, out, (size_t)3 * D);
  free(q); free(k); free(v); free(bt); free(out);
}

static void k_from_v_case(int dtype) {
  const int B = 2, KV = 4, D = 512, max_pages = 3, num_pages = 6, cap = max_pages * PAGE;
  const int32_t lens[2] = {5, 40};
  void *q = fill(dtype, (size_t)B * HEADS * D);
  void *v = fill(dtype, (size_t)num_pages * PAGE * KV * D);
  void *w = fill(dtype, D);
  int32_t *bt = block_table(B, max_pages);
  double *out = malloc((size_t)B * HEADS * D * sizeof *out);
  expect("k_from_v paged", oracle_gqa_decode_k_from_v(dtype, q, v, w, lens, bt, B, cap, max_pages,
                                                       num_pages, NULL, 0, out, 2), 0);
  expect_finite("k_from_v paged", out, (size_t)B * HEADS * D);
  void *vc = fill(dtype, (size_t)B * 40 * KV * D);
  expect("k_from_v contiguous", oracle_gqa_decode_k_from_v(dtype, q, vc, w, lens, NULL, B, 40, 0,
                                                            0, NULL, 0, out, 1), 0);
  expect_finite("k_from_v contiguous", out, (size_t)B * HEADS * D);
  expect("k_from_v without weight",
         oracle_gqa_decode_k_from_v(dtype, q, vc, NULL, lens, NULL, B, 40, 0, 0, NULL, 0, out, 1),
         -1);
  free(q); free(v); free(w); free(bt); free(out); free(vc);
}

static void ring_case(int dtype) {
  const int B = 2, KV = 16, D = 256, ring = 48, window = 17;
  const int32_t lens[2] = {10, 100};
  void *q = fill(dtype, (size_t)B * HEADS * D);
  void *k = fill(dtype, (size_t)B * ring * KV * D);
  void *v = fill(dtype, (size_t)B * ring * KV * D);
  double *out = malloc((size_t)B * HEADS * D * sizeof *out);
  expect("ring", oracle_gqa_decode_ring(dtype, q, k, v, lens, B, ring, KV, D, window, NULL, 0, out,
                                        2), 0);
  expect_finite("ring", out, (size_t)B * HEADS * D);
  expect("ring window above the ring",
         oracle_gqa_decode_ring(dtype, q, k, v, lens, B, ring, KV, D, ring + 1, NULL, 0, out, 1),
         -1);
  free(q); free(k); free(v); free(out);
}

static void prefill_case(int dtype, int KV, int D, int window, int paged) {
  const int B = 3;
  const int32_t cu_q[4] = {0, 1, 5, 5}; /* one token, four tokens, an empty chunk */
  const int N = 5;
  const int32_t lens[3] = {1, 30, 20};
  const int max_pages = 2, cap = paged ? max_pages * PAGE : 30, num_pages = B * max_pages;
  const size_t kv_elems = paged ? (size_t)num_pages * PAGE * KV * D : (size_t)B * cap * KV * D;
  void *q = fill(dtype, (size_t)N * HEADS * D);
  void *k = fill(dtype, kv_elems);
  void *v = fill(dtype, kv_elems);
  int32_t *bt = paged ? block_table(B, max_pages) : NULL;
  double *out = malloc((size_t)N * HEADS * D * sizeof *out);
  char what[96];
  snprintf(what, sizeof what, "prefill dtype %d KV %d window %d paged %d", dtype, KV, window,
           paged);
  expect(what, oracle_gqa_prefill(dtype, q, k, v, cu_q, lens, bt, B, N, cap, paged ? max_pages : 0,
                                  paged ? num_pages : 0, KV, D, window, NULL, 0, out, 3), 0);
  expect_finite(what, out, (size_t)N * HEADS * D);
  const int32_t bad_cu[4] = {0, 1, 5, 4};
  expect("prefill with cu_q[B] != N",
         oracle_gqa_prefill(dtype, q, k, v, bad_cu, lens, bt, B, N, cap, paged ? max_pages : 0,
                            paged ? num_pages : 0, KV, D, window, NULL, 0, out, 1), -1);
  free(q); free(k); free(v); free(bt); free(out);
}

static void append_case(int dtype, int KV, int D) {
  const int B = 2;
  const int32_t lens[2] = {1, 9};
  void *qr = fill(dtype, (size_t)B * HEADS * D);
  void *kr = fill(dtype, (size_t)B * KV * D);
  void *vr = fill(dtype, (size_t)B * KV * D);
  void *wq = fill(dtype, D);
  void *wk = fill(dtype, D);
  double *qo = malloc((size_t)B * HEADS * D * sizeof *qo);
  double *ko = malloc((size_t)B * KV * D * sizeof *ko);
  double *vo = malloc((size_t)B * KV * D * sizeof *vo);
  int32_t pos[2];
  expect("append", oracle_gqa_append_rows(dtype, qr, kr, vr, wq, wk, lens, B, KV, D, qo, ko, vo,
                                          pos), 0);
  expect_finite("append q", qo, (size_t)B * HEADS * D);
  expect_finite("append k", ko, (size_t)B * KV * D);
  expect("append with an unknown geometry",
         oracle_gqa_append_rows(dtype, qr, kr, vr, wq, wk, lens, B, 8, 128, qo, ko, vo, pos), -1);
  free(qr); free(kr); free(vr); free(wq); free(wk); free(qo); free(ko); free(vo);
}

int main(void) {
  for (int dtype = F32; dtype <= BF16; ++dtype) {
    for (int paged = 0; paged <= 1; ++paged) {
      decode_case(dtype, 16, 256, 1024, paged, 2);
      decode_case(dtype, 16, 256, 17, paged, 1);
      decode_case(dtype, 4, 512, 0, paged, 3);
      prefill_case(dtype, 16, 256, 1024, paged);
      prefill_case(dtype, 16, 256, 5, paged);
      prefill_case(dtype, 4, 512, 0, paged);
    }
    k_from_v_case(dtype);
    ring_case(dtype);
    append_case(dtype, 16, 256);
    append_case(dtype, 4, 512);
  }
  /* argument checks: an unknown dtype, a paged cap that is not max_pages*16 */
  {
    const int32_t lens[1] = {4};
    void *q = fill(F32, HEADS * 256), *k = fill(F32, 4 * 16 * 256), *v = fill(F32, 4 * 16 * 256);
    int32_t bt[1] = {0};
    double *out = malloc((size_t)HEADS * 256 * sizeof *out);
    expect("unknown dtype",
           oracle_gqa_decode(7, q, k, v, lens, NULL, 1, 4, 0, 0, 16, 256, 1024, NULL, 0, out, 1),
           -1);
    expect("paged cap mismatch",
           oracle_gqa_decode(F32, q, k, v, lens, bt, 1, 17, 1, 1, 16, 256, 1024, NULL, 0, out, 1),
           -1);
    free(q); free(k); free(v); free(out);
  }
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver: all calls clean\n");
  return 0;
}
