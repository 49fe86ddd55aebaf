/* Plain C (C99) use of the library's host-side entry points, compiled and run by
 * tests/test_c_abi.py: the headers must compile as C and the exported symbols must
 * link from C.  Nothing here touches the GPU.
 *
 * Scenario: a block manager with 64 blocks of 16 tokens prefills two prompts that
 * share their first 16 tokens (the second finds that full block cached), both
 * decode one token, and the host metadata builders turn the resulting tables into
 * slots that must agree with the manager's own. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nvpaged.h"
#include "nvpaged_blocks.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  enum { BS = 16, NB = 64, W = 8 };
  CHECK(strcmp(nv_status_string(NV_OK), "ok") == 0);
#ifndef NV_HOST_ONLY
  CHECK(nv_set_check_mode(0) >= 0); /* lives in the GPU part of the library */
#endif

  /* XXH64 of the empty input with seed 0: the algorithm's published value. */
  CHECK(nv_bm_xxh64("", 0, 0) == 0xEF46DB3751D8E999ull);

  nv_block_manager* bm = NULL;
  CHECK(nv_bm_create(NB, BS, &bm) == NV_OK && bm != NULL);

  /* prompts: 20 and 37 tokens, the first 16 equal */
  int32_t tokens[57];
  for (int i = 0; i < 20; ++i) tokens[i] = 100 + i;
  for (int i = 0; i < 37; ++i) tokens[20 + i] = i < 16 ? 100 + i : 500 + i;
  const int32_t cu_tokens[3] = {0, 20, 57};
  const int64_t ids[2] = {7, 9};
  int32_t tables[2 * W], cached[2];
  CHECK(nv_bm_prefill_step(bm, ids, cu_tokens, tokens, 2, tables, W, cached) == NV_OK);
  CHECK(cached[0] == 0 && cached[1] == BS);
  CHECK(tables[0] == tables[W]); /* the shared first block */
  int32_t ref = 0, has_hash = 0;
  uint64_t h = 0;
  CHECK(nv_bm_get_block(bm, tables[0], &ref, &has_hash, &h) == NV_OK && ref == 2 && has_hash);

  /* prefill metadata for the uncached tokens */
  const int32_t num_new[2] = {20 - cached[0], 37 - cached[1]};
  int32_t cu_q[3], cu_k[3], max_q = 0, max_k = 0, slots[64], nslots = 0;
  CHECK(nv_prepare_prefill(tables, W, cached, num_new, 2, BS, NB, 16, cu_q, cu_k, &max_q, &max_k,
                           slots, 64, &nslots, 0, NULL, 0, NULL) == NV_OK);
  CHECK(cu_q[2] == 20 + 21 && cu_k[2] == 57 && max_q == 21 && max_k == 37 && nslots == 48);
  CHECK(slots[0] == tables[0] * BS && slots[41] == -1);

  /* one decode step each */
  const int32_t next[2] = {1, 2};
  int32_t dtables[2 * W], lens[2], dslots[2];
  CHECK(nv_bm_decode_step(bm, ids, next, 2, dtables, W, lens, dslots) == NV_OK);
  CHECK(lens[0] == 21 && lens[1] == 38);
  int32_t pslots[2], sched[2], maxlen = 0;
  CHECK(nv_prepare_decode(dtables, W, lens, 2, BS, NB, pslots, sched, &maxlen) == NV_OK);
  CHECK(pslots[0] == dslots[0] && pslots[1] == dslots[1] && maxlen == 38);
  CHECK(sched[0] == 1 && sched[1] == 0); /* longest first */
  CHECK(pslots[0] == dtables[20 / BS] * BS + 20 % BS);

  CHECK(nv_bm_deallocate(bm, 7) == NV_OK && nv_bm_deallocate(bm, 9) == NV_OK);
  CHECK(nv_bm_num_free_blocks(bm) == NB);
  nv_bm_destroy(bm);

  /* Stress: rounds of prompts drawn from a small vocabulary (so prefixes repeat and
   * blocks are shared), decode steps that open new blocks, and releases, until the
   * pool is exhausted and refilled many times; every block must come back. */
  CHECK(nv_bm_create(NB, BS, &bm) == NV_OK);
  uint32_t rng = 12345u;
  int32_t prompt[6 * BS];
  int64_t live[8];
  int nlive = 0;
  for (int round = 0; round < 400; ++round) {
    rng = rng * 1664525u + 1013904223u;
    if (nlive < 8 && (rng >> 28) < 10) {
      const int32_t len = 1 + (int32_t)((rng >> 8) % (6 * BS - 1));
      for (int i = 0; i < len; ++i)
        prompt[i] = (int32_t)((i < 2 * BS) ? (uint32_t)(i % 7) : (rng >> (i % 16)) % 5u);
      int32_t ok = 0;
      CHECK(nv_bm_can_allocate(bm, len, &ok) == NV_OK);
      if (ok) {
        int32_t nc = -1;
        CHECK(nv_bm_allocate(bm, 1000 + round, prompt, len, &nc) == NV_OK);
        CHECK(nc >= 0 && nc < len && nc % BS == 0);
        live[nlive++] = 1000 + round;
      } else {
        CHECK(nv_bm_allocate(bm, 1000 + round, prompt, len, NULL) != NV_OK ||
              nv_bm_deallocate(bm, 1000 + round) == NV_OK);
      }
    } else if (nlive > 0 && (rng >> 29) < 6) {
      for (int j = 0; j < nlive; ++j) {
        int32_t ok = 0;
        CHECK(nv_bm_can_append(bm, live[j], &ok) == NV_OK);
        if (ok) CHECK(nv_bm_append_token(bm, live[j], (int32_t)(rng % 5)) == NV_OK);
      }
    } else if (nlive > 0) {
      const int j = (int)((rng >> 4) % (uint32_t)nlive);
      CHECK(nv_bm_deallocate(bm, live[j]) == NV_OK);
      live[j] = live[--nlive];
    }
  }
  while (nlive > 0) CHECK(nv_bm_deallocate(bm, live[--nlive]) == NV_OK);
  CHECK(nv_bm_num_free_blocks(bm) == NB);
  nv_bm_destroy(bm);
  printf("c abi ok\n");
  return 0;
}
