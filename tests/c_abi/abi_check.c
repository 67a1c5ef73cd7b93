/* A C program against include/cpa.h and libcpa.so: the header is plain C and
 * the host-side calls work without a GPU.  The step follows the token-budget
 * example of "Chunked Prefill" (deepconcepts.dev), opening sections: with 32
 * running users and a budget of 512, an 8192-token prompt gets a 480-token
 * chunk.  A budget of 16 cannot give each of the 32 users its one token, which
 * the library reports as CPA_ERR_BUDGET.  Prints "ok" and exits 0, or names
 * the failed check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cpa.h"

#define CHECK(c)                                                 \
  do {                                                           \
    if (!(c)) {                                                  \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                  \
    }                                                            \
  } while (0)

enum { kUsers = 32, kReqs = kUsers + 1, kPlanWords = 1 << 16 };

int main(void) {
  cpa_req_t reqs[kReqs];
  for (int i = 0; i < kUsers; ++i) {
    reqs[i].id = i;
    reqs[i].num_computed = 1000 + 37 * i;
    reqs[i].target_len = 0;
    reqs[i].is_decode = 1;
  }
  reqs[kUsers].id = kUsers;
  reqs[kUsers].num_computed = 0;
  reqs[kUsers].target_len = 8192;
  reqs[kUsers].is_decode = 0;

  cpa_build_params_t p;
  memset(&p, 0, sizeof p);
  p.token_budget = 512;
  p.block_size = CPA_BLOCK_SIZE;
  p.num_q_heads = 32;
  p.num_kv_heads = 8;
  p.head_dim = 128;
  p.policy = CPA_POLICY_TRUNCATE;

  static int32_t order[kReqs], nsch[kReqs], qsl[kReqs + 1], seq[kReqs], ctx[kReqs], newb[kReqs];
  static int32_t plan[kPlanWords];
  cpa_meta_t m;
  memset(&m, 0, sizeof m);
  m.max_seqs = kReqs;
  m.order = order;
  m.num_scheduled = nsch;
  m.query_start_loc = qsl;
  m.seq_lens = seq;
  m.context_lens = ctx;
  m.new_blocks = newb;
  m.plan_capacity = kPlanWords;
  m.plan = plan;

  CHECK(cpa_build_metadata(reqs, kReqs, &p, NULL, 0, 0, &m) == CPA_OK);
  CHECK(m.num_seqs == kReqs && m.num_decodes == kUsers && m.num_tokens == 512);
  CHECK(nsch[kUsers] == 480 && qsl[kReqs] == 512 && ctx[kUsers] == 0 && seq[kUsers] == 480);
  for (int i = 0; i < kUsers; ++i) CHECK(nsch[i] == 1 && seq[i] == ctx[i] + 1);
  CHECK(newb[kUsers] == 30); /* 480 / 16 pages */
  CHECK(m.counts.num_decode_splits > 0 && m.counts.num_chunk_tiles > 0);
  CHECK(m.plan_words == m.counts.num_decode_splits * CPA_DECODE_SPLIT_WORDS +
                            m.counts.num_chunk_tiles * CPA_CHUNK_TILE_WORDS +
                            m.counts.num_decode_merges * CPA_DECODE_MERGE_WORDS +
                            m.counts.num_chunk_merges * CPA_CHUNK_MERGE_WORDS);
  const size_t ws = cpa_workspace_size(&m.counts, p.num_q_heads, p.num_kv_heads, p.head_dim);
  CHECK(ws > 0 && ws % 256 == 0);

  p.token_budget = 16; /* fewer tokens than running users */
  CHECK(cpa_build_metadata(reqs, kReqs, &p, NULL, 0, 0, &m) == CPA_ERR_BUDGET);
  CHECK(strstr(cpa_status_string(CPA_ERR_BUDGET), "BUDGET") != NULL);
  CHECK(cpa_status_string(CPA_OK) != NULL);
  printf("ok\n");
  return 0;
}
