/* A plain C caller of the library's ABI (no Python, no torch): argument
 * checks and host-side queries only, so it runs without a GPU. Exits 0 when
 * every check holds, else prints the failed one and exits 1. */
#include <stdio.h>
#include <string.h>

#include "lce.h"

#define CHECK(cond)                                            \
  do {                                                         \
    if (!(cond)) {                                             \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                \
    }                                                          \
  } while (0)

int main(void) {
  lce_dims d;
  memset(&d, 0, sizeof d);
  d.n_tokens = 4096;
  d.hidden = 2048;
  d.vocab = 32000;
  d.n_shards = 8;
  d.ignore_index = -100;
  d.reduction = LCE_REDUCTION_MEAN;
  d.flags = 0;

  CHECK((lce_version() >> 16) == 1);
  const size_t ws = lce_workspace_bytes(&d);
  CHECK(ws > 0);
  CHECK(lce_state_bytes(&d) > 0 && lce_state_bytes(&d) <= ws);
  size_t wb = 0, xb = 0;
  CHECK(lce_ring_payload(&d, &wb, &xb) == LCE_PAYLOAD_WEIGHTS);
  CHECK(wb == (size_t)(32000 / 8) * 2048 * 8);

  /* errors come back before any GPU work, with a message */
  lce_dims bad = d;
  bad.vocab = 32001;
  CHECK(lce_workspace_bytes(&bad) == 0);
  const void* shards[8];
  float* grads[8];
  for (int s = 0; s < 8; ++s) {
    shards[s] = (const void*)(size_t)0x10000;
    grads[s] = (float*)(size_t)0x10000;
  }
  void* fake = (void*)(size_t)0x10000;
  int st = lce_forward(&bad, fake, shards, NULL, (const int32_t*)fake, (float*)fake, (float*)fake, NULL, fake,
                       ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  CHECK(strstr(lce_last_error(), "divisible") != NULL);
  CHECK(strcmp(lce_status_string(LCE_ERR_INVALID_ARG), "") != 0);
  st = lce_forward(&d, fake, shards, NULL, (const int32_t*)fake, (float*)fake, (float*)fake, NULL, fake, ws - 1,
                   NULL);
  CHECK(st == LCE_ERR_WORKSPACE);
  int32_t order[8] = {0, 1, 2, 3, 4, 5, 6, 6};
  st = lce_backward(&d, fake, shards, order, (const int32_t*)fake, (const float*)fake, (const float*)fake, fake,
                    (void* const*)grads, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  st = lce_fwd_round(&d, 8, 0, fake, fake, (const int32_t*)fake, fake, ws, NULL);
  CHECK(st == LCE_ERR_INVALID_ARG);
  st = lce_bwd_round(&d, 0, 0, fake, (const char*)fake + 2, (const int32_t*)fake, (const float*)fake,
                     (const float*)fake, fake, fake, 0, fake, ws, NULL);
  CHECK(st == LCE_ERR_UNSUPPORTED);
  printf("c abi ok: workspace %zu bytes, state %zu bytes\n", ws, lce_state_bytes(&d));
  return 0;
}
