/* A plain C caller of the library's ABI (no Python, no torch): argument
 * checks and host-side queries only, so it runs without a GPU. Every call
 * below returns before any GPU work (a size query, or an argument check that
 * fails on the host). Exits 0 when every check holds, else prints the failed
 * one and exits 1. Also built with AddressSanitizer and UndefinedBehavior-
 * Sanitizer on the host code of the library (see test_abi.py). */
#include <stdio.h>
#include <string.h>

#include "lce.h"

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

static lce_dims dims(int64_t n, int64_t h, int64_t v, int32_t p, int32_t flags) {
  lce_dims d;
  memset(&d, 0, sizeof d);
  d.n_tokens = n;
  d.hidden = h;
  d.vocab = v;
  d.n_shards = p;
  d.ignore_index = -100;
  d.reduction = LCE_REDUCTION_MEAN;
  d.flags = flags;
  return d;
}

int main(void) {
  lce_dims d = dims(4096, 2048, 32000, 8, 0);

  CHECK((lce_version() >> 16) == 1);
  const size_t ws = lce_workspace_bytes(&d);
  CHECK(ws > 0);
  CHECK(lce_state_bytes(&d) > 0 && lce_state_bytes(&d) <= ws);
  size_t wb = 0, xb = 0;
  CHECK(lce_ring_payload(&d, &wb, &xb) == LCE_PAYLOAD_WEIGHTS);
  CHECK(wb == (size_t)(32000 / 8) * 2048 * 8);
  CHECK(lce_ring_payload(&d, NULL, NULL) == LCE_PAYLOAD_WEIGHTS);

  /* the five workloads' sizes: every flag combination has a workspace, the
     bf16 one is larger, keeping ignored rows needs less */
  const int64_t shapes[5][4] = {{256, 128, 1024, 4},
                                {4096, 2048, 32000, 8},
                                {16384, 4096, 128256, 8},
                                {65536, 7168, 129280, 8},
                                {131071, 4096, 151936, 16}};
  for (int i = 0; i < 5; ++i) {
    for (int f = 0; f < 16; ++f) {
      lce_dims w = dims(shapes[i][0], shapes[i][1], shapes[i][2], (int32_t)shapes[i][3], f);
      CHECK(lce_workspace_bytes(&w) > 0);
      CHECK(lce_state_bytes(&w) <= lce_workspace_bytes(&w));
    }
    lce_dims plain = dims(shapes[i][0], shapes[i][1], shapes[i][2], (int32_t)shapes[i][3], 0);
    lce_dims b16 = plain, keep = plain;
    b16.flags = LCE_FLAG_BF16_GRADS;
    keep.flags = LCE_FLAG_KEEP_IGNORED_ROWS;
    CHECK(lce_workspace_bytes(&b16) > lce_workspace_bytes(&plain));
    CHECK(lce_workspace_bytes(&keep) < lce_workspace_bytes(&plain));
  }

  /* errors come back before any GPU work, with a message */
  lce_dims bad = d;
  bad.vocab = 32001;
  CHECK(lce_workspace_bytes(&bad) == 0);
  CHECK(lce_state_bytes(&bad) == 0);
  CHECK(lce_ring_payload(&bad, &wb, &xb) == LCE_ERR_INVALID_ARG);
  const void* shards[8];
  void* grads[8];
  for (int s = 0; s < 8; ++s) {
    shards[s] = (const void*)(size_t)0x10000;
    grads[s] = (void*)(size_t)0x10000;
  }
  void* fake = (void*)(size_t)0x10000;
  int st = lce_forward(&bad, fake, shards, NULL, (const int32_t*)fake, (float*)fake, (float*)fake, NULL, fake,
                       ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  CHECK(strstr(lce_last_error(), "divisible") != NULL);
  CHECK(strcmp(lce_status_string(LCE_ERR_INVALID_ARG), "") != 0);
  CHECK(strcmp(lce_status_string(12345), "unknown status") == 0);
  st = lce_forward(NULL, fake, shards, NULL, (const int32_t*)fake, (float*)fake, (float*)fake, NULL, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  lce_dims odd = d;
  odd.hidden = 100;
  st = lce_forward(&odd, fake, shards, NULL, (const int32_t*)fake, (float*)fake, (float*)fake, NULL, fake, ws, NULL);
  CHECK(st == LCE_ERR_UNSUPPORTED);
  lce_dims flag = d;
  flag.flags = 1 << 7;
  st = lce_forward(&flag, fake, shards, NULL, (const int32_t*)fake, (float*)fake, (float*)fake, NULL, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  /* the forward checks its own part of the workspace, the backward all of it */
  st = lce_forward(&d, fake, shards, NULL, (const int32_t*)fake, (float*)fake, (float*)fake, NULL, fake,
                   lce_state_bytes(&d) - 1, NULL);
  CHECK(st == LCE_ERR_WORKSPACE);
  st = lce_backward(&d, fake, shards, NULL, (const int32_t*)fake, (const float*)fake, (const float*)fake, fake,
                    (void* const*)grads, fake, ws - 1, NULL);
  CHECK(st == LCE_ERR_WORKSPACE);
  int32_t order[8] = {0, 1, 2, 3, 4, 5, 6, 6};
  st = lce_backward(&d, fake, shards, order, (const int32_t*)fake, (const float*)fake, (const float*)fake, fake,
                    (void* const*)grads, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  CHECK(strstr(lce_last_error(), "permutation") != NULL);
  grads[3] = NULL;
  st = lce_backward(&d, fake, shards, NULL, (const int32_t*)fake, (const float*)fake, (const float*)fake, fake,
                    (void* const*)grads, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  grads[3] = fake;
  st = lce_fwd_round(&d, 8, 0, fake, fake, (const int32_t*)fake, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  st = lce_fwd_round(&d, 0, -1, fake, fake, (const int32_t*)fake, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  st = lce_fwd_finish(&d, (const int32_t*)fake, NULL, (float*)fake, NULL, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  st = lce_bwd_round(&d, 0, 0, fake, (const char*)fake + 2, (const int32_t*)fake, (const float*)fake,
                     (const float*)fake, fake, fake, 0, fake, ws, NULL);
  CHECK(st == LCE_ERR_UNSUPPORTED);
  /* the forward without a workspace refuses a batch beyond its scratch */
  lce_dims big = dims(1 << 19, 64, 16 * 2048, 16, 0);
  const void* shards16[16];
  for (int s = 0; s < 16; ++s) shards16[s] = fake;
  CHECK(lce_forward_noalloc_max_bytes() == ((size_t)32 << 20));
  st = lce_forward_noalloc(&big, fake, shards16, NULL, (const int32_t*)fake, (float*)fake, (float*)fake, NULL, NULL);
  CHECK(st == LCE_ERR_WORKSPACE);
  CHECK(strstr(lce_last_error(), "scratch") != NULL);
  /* an empty trace collects nothing */
  CHECK(lce_trace_enable(0) == LCE_OK);
  lce_trace_entry entries[4];
  CHECK(lce_trace_collect(entries, 4) == 0);
  CHECK(lce_trace_collect(NULL, 1) == LCE_ERR_INVALID_ARG);
  CHECK(lce_trace_enable(-1) == LCE_ERR_INVALID_ARG);
  printf("c abi ok: workspace %zu bytes, state %zu bytes\n", ws, lce_state_bytes(&d));
  return 0;
}
