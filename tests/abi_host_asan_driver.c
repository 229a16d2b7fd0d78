/*
 * Host-only driver for the host side of libgqadecode: the launch planner, the
 * workspace sizes, the constants, the status strings and the argument checks
 * of the entry points.  tests/test_abi_host_sanitized.py builds it together
 * with the library's sources, the host code instrumented with
 * AddressSanitizer and UndefinedBehaviorSanitizer, so an overflow in the plan
 * or size arithmetic (B up to 256, capacities and windows up to 262144 and
 * beyond) or an access outside a host array ends the run with a report.
 * Every entry point is called only with arguments its checks reject, so no
 * kernel is ever launched and no GPU is needed.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gqa_decode.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static const int32_t kBatches[] = {INT_MIN, -1, 0, 1, 2, 7, 32, 255, 256, 257, INT_MAX};
static const int32_t kCaps[] = {INT_MIN, -1, 0, 1, 15, 16, 17, 1023, 1024, 1025, 8192,
                                131072, 262143, 262144, 262145, INT_MAX};
static const int32_t kWindows[] = {INT_MIN, -5, 0, 1, 17, 1024, 2032, 4096, 8192, 262144,
                                   262145, INT_MAX};

static void plans(void) {
  for (int variant = -1; variant <= 2; ++variant)
    for (size_t i = 0; i < sizeof kBatches / sizeof *kBatches; ++i)
      for (size_t c = 0; c < sizeof kCaps / sizeof *kCaps; ++c) {
        const int32_t B = kBatches[i], cap = kCaps[c];
        int32_t mode = -7, waves = -7, slots = -7;
        const int st = gqa_decode_plan(variant, B, cap, &mode, &waves, &slots);
        const size_t ws = gqa_decode_workspace_bytes(variant, B, cap);
        const int valid = (variant == GQA_SLIDING || variant == GQA_GLOBAL) && B >= 1 &&
                          B <= 256 && cap >= 1 && cap <= 262144;
        if (valid) {
          expect("plan of a valid shape", st, GQA_OK);
          if (mode != GQA_MODE_UNIT && mode != GQA_MODE_STREAM && mode != GQA_MODE_GROUP) {
            fprintf(stderr, "FAIL plan mode %d (variant %d B %d cap %d)\n", mode, variant, B, cap);
            ++failures;
          }
          if (waves < 1 || slots < 0 || (mode != GQA_MODE_UNIT && ws == 0)) {
            fprintf(stderr, "FAIL plan waves %d slots %d ws %zu (variant %d B %d cap %d)\n", waves,
                    slots, ws, variant, B, cap);
            ++failures;
          }
        } else {
          if (st == GQA_OK) {
            fprintf(stderr, "FAIL plan accepted variant %d B %d cap %d\n", variant, B, cap);
            ++failures;
          }
          if (ws != 0) {
            fprintf(stderr, "FAIL workspace %zu for variant %d B %d cap %d\n", ws, variant, B, cap);
            ++failures;
          }
        }
        for (size_t w = 0; w < sizeof kWindows / sizeof *kWindows; ++w) {
          const int32_t W = kWindows[w];
          const int stw = gqa_decode_sliding_window_plan(B, cap, W, &mode, &waves, &slots);
          const size_t wsw = gqa_decode_sliding_window_workspace_bytes(B, cap, W);
          const size_t wsr = gqa_decode_sliding_ring_workspace_bytes(B, cap, W);
          const int wvalid = B >= 1 && B <= 256 && cap >= 1 && cap <= 262144 && W >= 1 &&
                             W <= 262144;
          if (!wvalid && (stw == GQA_OK || wsw != 0)) {
            fprintf(stderr, "FAIL window plan accepted B %d cap %d window %d\n", B, cap, W);
            ++failures;
          }
          if (wvalid && stw != GQA_OK) {
            fprintf(stderr, "FAIL window plan rejected B %d cap %d window %d\n", B, cap, W);
            ++failures;
          }
          (void)wsr;
        }
      }
}

static void constants_and_strings(void) {
  for (int variant = -2; variant <= 3; ++variant) {
    int32_t h = 0, kv = 0, d = 0, w = 0, p = 0;
    const int st = gqa_decode_constants(variant, &h, &kv, &d, &w, &p);
    expect("constants", st, variant == GQA_SLIDING || variant == GQA_GLOBAL ? GQA_OK
                                                                             : GQA_ERR_DTYPE);
  }
  for (int s = -20; s <= 5; ++s) {
    const char* str = gqa_status_str(s);
    if (!str || strlen(str) == 0) {
      fprintf(stderr, "FAIL empty status string for %d\n", s);
      ++failures;
    }
  }
}

/* aligned host stand-ins: the entry points only look at the pointer values
 * before they reject the call */
static _Alignas(64) unsigned char buf[256];

static void rejections(void) {
  void* ok = buf;
  void* mis = buf + 4;
  const int32_t* lens = (const int32_t*)buf;
  int32_t ws_cap = 0;
  (void)ws_cap;
  expect("sliding NULL q",
         gqa_decode_sliding(NULL, ok, ok, lens, ok, 4, 2048, GQA_BF16, NULL, 0, NULL),
         GQA_ERR_NULL);
  expect("sliding B=257", gqa_decode_sliding(ok, ok, ok, lens, ok, 257, 2048, GQA_BF16, NULL, 0,
                                             NULL), GQA_ERR_SHAPE);
  expect("sliding S_max above the maximum",
         gqa_decode_sliding(ok, ok, ok, lens, ok, 4, 262145, GQA_BF16, NULL, 0, NULL),
         GQA_ERR_SHAPE);
  expect("sliding bad dtype",
         gqa_decode_sliding(ok, ok, ok, lens, ok, 4, 2048, 9, NULL, 0, NULL), GQA_ERR_DTYPE);
  expect("sliding misaligned k",
         gqa_decode_sliding(ok, mis, ok, lens, ok, 4, 2048, GQA_BF16, NULL, 0, NULL),
         GQA_ERR_ALIGN);
  expect("global without its workspace",
         gqa_decode_global(ok, ok, ok, lens, ok, 32, 131072, GQA_BF16, NULL, 0, NULL),
         GQA_ERR_WORKSPACE);
  expect("global paged num_pages 0",
         gqa_decode_global_paged(ok, ok, ok, lens, 8192, lens, ok, 32, 0, GQA_BF16, ok, 1 << 30,
                                 NULL), GQA_ERR_SHAPE);
  expect("window 0", gqa_decode_sliding_window(ok, ok, ok, lens, ok, 4, 2048, 0, GQA_BF16, NULL,
                                               0, NULL), GQA_ERR_SHAPE);
  expect("ring window above the ring",
         gqa_decode_sliding_ring(ok, ok, ok, lens, ok, 4, 1024, 1025, GQA_BF16, ok, 1 << 30, NULL),
         GQA_ERR_SHAPE);
  expect("prefill N negative",
         gqa_prefill_sliding(ok, ok, ok, lens, lens, ok, 2, -1, 2048, GQA_BF16, NULL),
         GQA_ERR_SHAPE);
  expect("prefill NULL cu_q",
         gqa_prefill_global(ok, ok, ok, NULL, lens, ok, 2, 8, 2048, GQA_BF16, NULL),
         GQA_ERR_NULL);
  expect("prefill window 0",
         gqa_prefill_sliding_window(ok, ok, ok, lens, lens, ok, 2, 8, 2048, 0, GQA_BF16, NULL),
         GQA_ERR_SHAPE);
  expect("keys-from-values NULL w_k",
         gqa_decode_global_k_eq_v(ok, ok, NULL, lens, ok, 4, 2048, GQA_BF16, ok, 1 << 30, NULL),
         GQA_ERR_NULL);
}

int main(void) {
  plans();
  constants_and_strings();
  rejections();
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("library host side: all calls clean\n");
  return 0;
}
