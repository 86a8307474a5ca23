/*
 * Host-side argument checks of every entry point, for a build of the library
 * with AddressSanitizer and UndefinedBehaviorSanitizer on its host code (see
 * tests/test_host_sanitizers.py). Every call here must fail in the checks
 * that run before any HIP call, so the tensor "pointers" are fake aligned
 * addresses that nothing dereferences; the split-count and workspace-size
 * rules are pure host arithmetic when the CU count is given. Exit status 0
 * when every call returned what it should (a sanitizer report aborts first).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gqa_decode.h"

#define P(i) ((void*)(uintptr_t)(0x10000u * (i)))
static const void *Q = P(1), *K = P(2), *V = P(3), *O = P(5), *W = P(6);
static const int32_t* L = (const int32_t*)P(4);

static int failures;

static void expect(const char* what, long got, long want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %ld, want %ld (%s)\n", what, got, want, gqa_last_error());
    ++failures;
  } else if (want < 0 && gqa_last_error()[0] == '\0') {
    fprintf(stderr, "FAIL %s: no message\n", what);
    ++failures;
  }
}

static int ex(const void* q, const void* out, int B, int h_q, int h_kv, int d, float scale, int ns,
              int in_dt, int out_dt, int64_t hint, void* ws, size_t ws_bytes, int flags) {
  return gqa_decode_attn_ex(q, K, V, L, NULL, (void*)out, B, h_q, h_kv, d, scale, ns, in_dt, out_dt, hint,
                            ws, ws_bytes, NULL, flags);
}

int main(void) {
  expect("null q", ex(NULL, O, 1, 64, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("null out", ex(Q, NULL, 1, 64, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("B = 0", ex(Q, O, 0, 64, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("B too large", ex(Q, O, 70000, 64, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("h_q % h_kv", ex(Q, O, 1, 60, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("n_rep 3", ex(Q, O, 1, 24, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_UNSUPPORTED);
  expect("n_rep 32", ex(Q, O, 1, 256, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_UNSUPPORTED);
  expect("d 96", ex(Q, O, 1, 64, 8, 96, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_UNSUPPORTED);
  expect("scale inf", ex(Q, O, 1, 64, 8, 128, INFINITY, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("scale nan", ex(Q, O, 1, 64, 8, 128, NAN, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("in dtype", ex(Q, O, 1, 64, 8, 128, 0.088f, 0, 2, 0, 0, NULL, 0, 0), GQA_ERR_UNSUPPORTED);
  expect("out dtype", ex(Q, O, 1, 64, 8, 128, 0.088f, 0, 1, 7, 0, NULL, 0, 0), GQA_ERR_UNSUPPORTED);
  expect("flags", ex(Q, O, 1, 64, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 4), GQA_ERR_INVALID_ARG);
  expect("n_splits", ex(Q, O, 1, 64, 8, 128, 0.088f, 4097, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("hint", ex(Q, O, 1, 64, 8, 128, 0.088f, 0, 1, 0, -1, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("misaligned q", ex((const char*)Q + 8, O, 1, 64, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0),
         GQA_ERR_INVALID_ARG);
  expect("out aliases q", ex(Q, Q, 1, 64, 8, 128, 0.088f, 0, 1, 0, 0, NULL, 0, 0), GQA_ERR_INVALID_ARG);
  expect("workspace alignment", ex(Q, O, 1, 64, 8, 128, 0.088f, 0, 1, 0, 0, (char*)W + 64, 1 << 20, 0),
         GQA_ERR_INVALID_ARG);
  expect("workspace too small", ex(Q, O, 1, 64, 8, 128, 0.088f, 8, 1, 0, 0, (void*)W, 16, 0), GQA_ERR_WORKSPACE);
  expect("base entry d", gqa_decode_attn(Q, K, V, L, (void*)O, 1, 64, 8, 80, 0.088f, 0), GQA_ERR_UNSUPPORTED);

  expect("multi S_q 0", gqa_decode_attn_multi(Q, K, V, L, NULL, (void*)O, 2, 0, 64, 8, 128, 0.088f, 0, 0, 0,
                                              NULL, 0, NULL), GQA_ERR_INVALID_ARG);
  expect("multi S_q 65", gqa_decode_attn_multi(Q, K, V, L, NULL, (void*)O, 2, 65, 64, 8, 128, 0.088f, 0, 0, 0,
                                               NULL, 0, NULL), GQA_ERR_INVALID_ARG);
  expect("partial without workspace", gqa_decode_partial(Q, K, V, L, NULL, 1, 64, 8, 128, 0.088f, 0, 1, 0,
                                                         NULL, 0, NULL, 0), GQA_ERR_INVALID_ARG);
  expect("merge small workspace", gqa_decode_merge(L, W, 16, (void*)O, 1, 64, 8, 128, 8, 0, 0, NULL),
         GQA_ERR_WORKSPACE);
  expect("triplet d", gqa_decode_attn_triplet(Q, K, V, L, NULL, (float*)W, (float*)((char*)W + 4096), 1, 64, 8, 96,
                                              0.088f, 0, 1, 0, NULL, 0, NULL, 0), GQA_ERR_UNSUPPORTED);
  expect("merge triplets parts", gqa_merge_triplets((const float*)W, (const float*)((char*)W + 65536), 0, 64, 128,
                                                    (void*)O, 0, NULL), GQA_ERR_INVALID_ARG);
  expect("append n_new", gqa_kv_append(Q, V, (void*)K, (void*)O, NULL, L, NULL, 2, 0, 8, 128, 1, 100, NULL),
         GQA_ERR_INVALID_ARG);
  expect("append lens overlap", gqa_kv_append(Q, V, (void*)K, (void*)O, NULL, L, (int32_t*)L, 2, 1, 8, 128, 1,
                                              100, NULL), GQA_ERR_INVALID_ARG);
  expect("step lens out", gqa_decode_step(Q, W, (char*)W + 0x4000, (void*)K, (void*)V, L, NULL, NULL, (void*)O, 2,
                                          64, 8, 128, 0.088f, 0, 1, 0, 100, NULL, 0, NULL), GQA_ERR_INVALID_ARG);
  expect("step fp32", gqa_decode_step(Q, W, (char*)W + 0x4000, (void*)K, (void*)V, L, (int32_t*)((char*)W + 0x8000),
                                      NULL, (void*)O, 2, 64, 8, 128, 0.088f, 0, 0, 0, 100, NULL, 0, NULL),
         GQA_ERR_UNSUPPORTED);
  expect("events", gqa_decode_set_split_events((hipEvent_t)P(7), NULL), GQA_ERR_INVALID_ARG);
  expect("events off", gqa_decode_set_split_events(NULL, NULL), GQA_OK);

  /* split-count rules and workspace sizes: host arithmetic */
  expect("pick 8k", gqa_decode_pick_splits(1, 8, 8192, 256), 32);
  expect("pick 8191", gqa_decode_pick_splits(1, 8, 8191, 256), 64);
  expect("pick 40000 (8-wave round)", gqa_decode_pick_splits(1, 8, 40000, 256), 32);
  expect("pick 65537", gqa_decode_pick_splits(1, 8, 65537, 256), 128);
  expect("pick no hint (8-wave round)", gqa_decode_pick_splits(1, 8, 0, 256), 32);
  expect("pick 1M", gqa_decode_pick_splits(1, 8, 1 << 20, 256), 256);
  expect("pick d64 8k", gqa_decode_pick_splits_d(1, 8, 64, 8192, 256), 64);
  expect("pick d96", gqa_decode_pick_splits_d(1, 8, 96, 8192, 256), GQA_ERR_UNSUPPORTED);
  expect("pick ragged", gqa_decode_pick_splits(8, 8, 32768, 256), 32);
  expect("pick huge", gqa_decode_pick_splits(1, 1, (int64_t)1 << 40, 256), GQA_MAX_SPLITS);
  expect("multi S_q 4 (two tiles, one per pass)", gqa_decode_multi_splits(1, 4, 64, 8, 8192, 256), 16);
  expect("multi S_q 4, 16k (two tiles per pass)", gqa_decode_multi_splits(1, 4, 64, 8, 16384, 256), 32);
  expect("multi S_q 16, 16k (one tile per wave, one workgroup per CU)", gqa_decode_multi_splits(1, 16, 64, 8, 16384, 256), 32);
  expect("multi S_q 16, 8k (one sequence of 8 tiles from 4096 tokens: one tile per wave)", gqa_decode_multi_splits(1, 16, 64, 8, 8192, 256), 32);
  expect("multi S_q 16, 64k (one tile per wave, two workgroups per CU)", gqa_decode_multi_splits(1, 16, 64, 8, 65536, 256), 64);
  expect("multi bad h_kv", gqa_decode_multi_splits(1, 4, 64, 0, 8192, 256), GQA_ERR_INVALID_ARG);
  expect("multi S_q 2, d 128 (8-wave round)", gqa_decode_multi_splits_d(1, 2, 64, 8, 128, 8192, 256), 32);
  expect("multi S_q 2, d 64", gqa_decode_multi_splits_d(1, 2, 64, 8, 64, 8192, 256), 64);
  expect("multi bad d_head", gqa_decode_multi_splits_d(1, 2, 64, 8, 96, 8192, 256), GQA_ERR_UNSUPPORTED);
  expect("workspace bytes", (long)gqa_decode_workspace_bytes(8, 64, 128, 37),
         (long)(512 * 8 + ((8L * 64 * 37 * 128 * 4 + 255) / 256) * 256 + ((8L * 64 * 37 * 8 + 255) / 256) * 256 +
                256));
  expect("workspace bytes 0", (long)gqa_decode_workspace_bytes(0, 64, 128, 4), 0);
  for (int s = 0; s >= -5; --s)
    if (!gqa_status_string(s) || !gqa_status_string(s)[0]) {
      fprintf(stderr, "FAIL status string %d\n", s);
      ++failures;
    }
  printf("host checks: %d failure(s)\n", failures);
  return failures ? 1 : 0;
}
