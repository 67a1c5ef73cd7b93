/*
 * cpa.h -- C ABI of the chunked-prefill mixed-batch attention library (libcpa.so)
 *
 * One continuous-batching step packs decode rows (one query each) and prefill
 * chunks (C query tokens each) into a single token batch.  Each chunk token
 * attends to every earlier chunk's K/V already in the paged cache plus a
 * causal mask inside its own chunk; the step's own K/V is appended first.
 *
 * Sources, by page title and section:
 *   [P1] "Chunked Prefill" (deepconcepts.dev): the token budget; decodes take
 *        one token each and the prompt gets the rest ("Why a chunk can be nearly
 *        free"); a budget below the running count can never finish a prompt
 *        ("The budget points in two directions").
 *   [P2] "05. Chunked Prefill" (vLLM learning book): section 3, a chunk's
 *        queries see all cached earlier chunks plus a causal mask inside the
 *        chunk; section 4, all rows are packed into one 1-D token tensor told
 *        apart by query_start_loc / seq_lens; section 5, decode-first hybrid
 *        split of the budget; section 8, attention reads the cache including
 *        the K/V the current chunk just wrote.
 *   [P4] tbr8.org chunked-prefill deep dive: 3.1, decode tokens first and the
 *        remaining budget to prefill; 3.3, a chunk carries the length of the
 *        prefix already cached; 4.1, a chunk never sees later chunks; 4.2,
 *        16-token KV pages and per-chunk page allocation.
 *   [P5] "How Chunked Prefill Stops Decode Starvation": "The fix", a prefill
 *        that does not fit the remaining budget is chunked.
 *
 * Conventions shared by every call
 *   - All sizes are int32 unless stated.  bf16 tensors are passed as void*
 *     holding IEEE bfloat16 bit patterns.
 *   - Every buffer is allocated and owned by the caller.  The library
 *     allocates no memory, keeps no pointer after a call returns and has no
 *     global mutable state; calls are re-entrant.
 *   - Device calls are asynchronous on the given HIP stream and are ordered
 *     only by that stream.  Device-side integer inputs are trusted: validation
 *     happens on the host in cpa_build_metadata.
 *   - Status: CPA_OK (0) or a negative CPA_ERR_*; the library never aborts and
 *     never throws across the ABI.  CPA_ERR_DEVICE carries a launch failure
 *     reported by hipGetLastError.
 *   - Supported shapes: head_dim in {64, 128}; num_q_heads a multiple of
 *     num_kv_heads, with G = num_q_heads / num_kv_heads from 1 to one chunk
 *     tile's rows R (256 at head_dim 128, 128 at 64); num_kv_heads at most
 *     256; block_size 16; bf16 only.  G = 1, 2, 4 and 8 run kernels compiled
 *     for them, any other G the same kernels with G read at run time; a
 *     decode piece takes one wave per 32 query heads of its group.
 *
 * KV cache layout (one tensor each for K and V; the same page id in both)
 *   k_cache [num_blocks][num_kv_heads][head_dim/8][16][8]
 *       a page's keys in 8-value pieces: element d of slot s sits at
 *       [d/8][s][d%8], so each 1 KB run holds 4 pieces of all 16 keys
 *   v_cache [num_blocks][num_kv_heads][head_dim][16]   transposed in a page
 *   Position p of a row lives in page block_table[row][p / 16], slot p % 16.
 *
 * Packed tensors
 *   q     [num_tokens][num_q_heads][head_dim]   bf16
 *   k_new [num_tokens][num_kv_heads][head_dim]  bf16
 *   v_new [num_tokens][num_kv_heads][head_dim]  bf16
 *   out   [num_tokens][num_q_heads][head_dim]   bf16
 *   lse   [num_tokens][num_q_heads]             fp32, natural log (optional)
 *   Row s owns packed tokens [query_start_loc[s], query_start_loc[s+1]).
 *   Rows [0, num_decodes) are decode rows (one token each); the rest are
 *   prefill chunks.  Query head h reads KV head h / (num_q_heads/num_kv_heads).
 */
#ifndef CPA_H
#define CPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPA_OK 0
#define CPA_ERR_INVALID (-1)     /* malformed input (lengths, ordering, block ids, slots) */
#define CPA_ERR_BUDGET (-2)      /* more running decodes than budget tokens [P1] */
#define CPA_ERR_CAPACITY (-3)    /* a caller-provided array or workspace is too small */
#define CPA_ERR_UNSUPPORTED (-4) /* head_dim, head ratio or block size not supported */
#define CPA_ERR_DEVICE (-5)      /* a kernel launch failed */

#define CPA_BLOCK_SIZE 16

/* Plan entry sizes in int32 words (see cpa_plan_counts_t).  q_* are chunk-local
 * token indices; kv_* are key positions of the row. */
#define CPA_DECODE_SPLIT_WORDS 4 /* {row, kv_begin, kv_end, decode partial slot or -1} */
#define CPA_DECODE_MERGE_WORDS 4 /* {row, first decode slot, num slots, 0} */
#define CPA_CHUNK_TILE_WORDS 8   /* {row, q_begin, q_end, kv_begin, kv_end, chunk slot or -1, 0, 0} */
#define CPA_CHUNK_MERGE_WORDS 8  /* {row, q_begin, q_end, first chunk slot, num slots, 0, 0, 0} */

/* One queued request, in queue order: running decodes, then prefills first
 * come first served (a continued chunked prompt precedes newer prompts). */
typedef struct {
  int32_t id;           /* caller's tag; copied nowhere, for the caller's use */
  int32_t num_computed; /* tokens already in the KV cache ([P4] 3.3 cached_prefix_len) */
  int32_t target_len;   /* prompt length of a prefill; ignored for a decode */
  int32_t is_decode;    /* nonzero: wants exactly one token this step */
} cpa_req_t;

typedef struct {
  int32_t token_budget;        /* max tokens this step, decodes included [P1][P2 5] */
  int32_t long_prefill_cap;    /* per-request cap on a prefill's share, 0 = none
                                  ([P1] "Checking it on a real system") */
  int32_t block_size;          /* must be 16 [P4 4.2] */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t decode_split_tokens; /* keys per decode split, multiple of 16, at most 1024;
                                  0 = chosen by size */
  int32_t chunk_split_tokens;  /* prefix keys per chunk-tile split, multiple of 64;
                                  0 = chosen by size; a value above every context = no split */
  int32_t policy;              /* CPA_POLICY_* below, optionally | the flags
                                  CPA_POLICY_ADAPTIVE_CHUNK, CPA_POLICY_BLOCK_ALIGNED */
  int32_t max_prefill_tokens;  /* prefill quota of CPA_POLICY_QUOTA (> 0, at most
                                  INT32_MAX - token_budget); else ignored */
} cpa_build_params_t;

/* How the budget left after the decodes goes to prefills (tbr8.org deep dive
 * section 3; every policy schedules all decodes first, one token each):
 *   CPA_POLICY_TRUNCATE  prefills in queue order, each min(remaining prompt,
 *                        long_prefill_cap, remaining budget) tokens: a prompt
 *                        that does not fit is chunked to what remains ([P1],
 *                        [P2] 5, [P5] "The fix").  The default.
 *   CPA_POLICY_DEFER     3.1 as printed: a prefill's chunk is min(remaining
 *                        prompt, long_prefill_cap); it is scheduled only if the
 *                        remaining budget holds all of it, and the first one
 *                        that does not fit ends the scan.
 *   CPA_POLICY_QUOTA     3.2: prefills share max_prefill_tokens of their own
 *                        (the step may then exceed token_budget), cut to
 *                        token_budget - decodes when the decodes take more than
 *                        70% of token_budget; within it as TRUNCATE.
 *   CPA_POLICY_ADAPTIVE_CHUNK (flag) 7.1: the per-request cap is
 *                        long_prefill_cap x4 with no decode, x2 under 10
 *                        decodes, x1 under 50, /2 (at least 1) beyond; needs
 *                        long_prefill_cap > 0.
 *   CPA_POLICY_BLOCK_ALIGNED (flag): a chunk that stops before the end of
 *                        its prompt stops on a page boundary instead
 *                        (context + n rounded down to a multiple of 16) when
 *                        that leaves it at least one token; the tokens given
 *                        back stay in the budget for the prompts behind it.
 *                        Every page such a chunk writes is complete, so a
 *                        prefix cache can reuse it ([P1] closing notes: a
 *                        chunked prefill reuses only cached pages on page
 *                        boundaries; [P4] 6.1). */
#define CPA_POLICY_TRUNCATE 0
#define CPA_POLICY_DEFER 1
#define CPA_POLICY_QUOTA 2
#define CPA_POLICY_ADAPTIVE_CHUNK 0x100
#define CPA_POLICY_BLOCK_ALIGNED 0x200

/* Counts of the device work plan built by cpa_build_metadata.  The plan is one
 * int32 array of four sections, in this order: num_decode_splits entries of
 * CPA_DECODE_SPLIT_WORDS, num_chunk_tiles of CPA_CHUNK_TILE_WORDS,
 * num_decode_merges of CPA_DECODE_MERGE_WORDS, num_chunk_merges of
 * CPA_CHUNK_MERGE_WORDS (the two merge sections run as one launch).  A chunk tile covers R
 * (token, query head) rows of one KV head, R = 256 at head_dim 128 and 128 at
 * head_dim 64: floor(R / G) tokens, G = num_q_heads / num_kv_heads (when G does
 * not divide R, a tile's last R mod G rows hold no query). */
typedef struct {
  int32_t num_decode_splits;   /* one wave per (split, KV head, 32 query heads of the group) */
  int32_t num_decode_merges;   /* decode rows whose keys were split in several pieces */
  int32_t num_chunk_tiles;     /* one workgroup per (tile, KV head) */
  int32_t num_chunk_merges;    /* chunk tiles whose prefix keys were split in several pieces */
  int32_t num_decode_partials; /* decode partial slots: num_q_heads x (head_dim + 2) fp32 each */
  int32_t num_chunk_partials;  /* chunk partial slots: num_kv_heads x R x (head_dim bf16 + 2 fp32) */
} cpa_plan_counts_t;

/* Host arrays filled by cpa_build_metadata; the caller provides them with the
 * stated capacities.  Unused optional outputs may be NULL. */
typedef struct {
  int32_t max_seqs;         /* capacity of the per-row arrays */
  int32_t* order;           /* [max_seqs]  request index (into reqs) of each row */
  int32_t* num_scheduled;   /* [max_seqs]  tokens of each row this step */
  int32_t* query_start_loc; /* [max_seqs+1] prefix sums of num_scheduled */
  int32_t* seq_lens;        /* [max_seqs]  context_len + num_scheduled */
  int32_t* context_lens;    /* [max_seqs]  tokens cached before this step */
  int32_t* new_blocks;      /* [max_seqs]  pages the row newly reaches (nullable) */
  int32_t max_tokens;       /* capacity of slot_mapping */
  int64_t* slot_mapping;    /* [max_tokens] page*16+slot per packed token (nullable;
                               needs a host block table) */
  int32_t plan_capacity;    /* capacity of plan in int32 words */
  int32_t* plan;            /* [plan_capacity] device work plan (nullable: then only
                               the counts are produced) */
  /* outputs */
  int32_t num_seqs;
  int32_t num_decodes;
  int32_t num_tokens;
  int32_t plan_words;       /* int32 words written to plan */
  cpa_plan_counts_t counts;
} cpa_meta_t;

/*
 * cpa_build_metadata -- host-side decode-first budget split and work plan.
 *
 * Every decode request gets one token; by default the remaining budget goes
 * to prefill requests in queue order, each taking min(remaining prompt,
 * long_prefill_cap, remaining budget) tokens, so a prompt that does not fit is
 * chunked ([P1] second section: budget 512 with 32 users gives 480-token
 * chunks; [P2] section 5; [P4] 3.1; [P5] "The fix").  params->policy selects
 * the variants described at CPA_POLICY_TRUNCATE.  Rows are emitted decodes first
 * (queue order) then prefills (queue order); a request given no token is left
 * out.  new_blocks = ceil(seq_len/16) - ceil(context_len/16) ([P4] 4.2, for
 * chunks that start mid-page too).
 *
 * If host_block_table is given ([n_reqs][bt_stride] int32, rows indexed by
 * request, not by output row) the call also checks that every row's pages
 * cover seq_len, that ids are in [0, num_blocks), that no two scheduled tokens
 * share a slot, and fills slot_mapping.
 *
 * Synchronous, pure, host only (no HIP call).  Returns CPA_OK,
 * CPA_ERR_BUDGET (decodes > token_budget), CPA_ERR_INVALID (negative lengths,
 * target_len < num_computed, bad block ids, duplicate slots, split sizes that
 * are not whole pages / KV tiles, an unknown policy, a quota without
 * max_prefill_tokens, adaptive chunking without a cap), CPA_ERR_CAPACITY (an
 * output array too small) or
 * CPA_ERR_UNSUPPORTED (shape outside the supported set).  On error the
 * outputs are unspecified.
 */
int cpa_build_metadata(const cpa_req_t* reqs, int n_reqs, const cpa_build_params_t* params,
                       const int32_t* host_block_table, int bt_stride, int num_blocks,
                       cpa_meta_t* out);

/*
 * cpa_append_kv -- write the step's K/V into the paged cache ([P2] section 8:
 * the chunk's own K/V is in the cache when attention runs; [P4] 4.2).
 *
 * For packed token t of row s at position p = context_lens[s] + t -
 * query_start_loc[s]:  k_cache page block_table[s][p/16], slot p%16 <- k_new[t]
 * and the same for V (transposed layout).  Exactly num_tokens*num_kv_heads
 * slots of each cache are written; nothing else is touched.  Enqueue it
 * before cpa_attention of the same step on the same stream.
 *
 * d_* pointers are device int32 arrays: query_start_loc [num_seqs+1],
 * context_lens [num_seqs], block_table [num_seqs][bt_stride] (rows in output
 * row order).  num_tokens = 0 returns CPA_OK without a launch.  Returns
 * CPA_OK, CPA_ERR_UNSUPPORTED (head_dim, block size), CPA_ERR_INVALID
 * (negative sizes, bt_stride <= 0, or a NULL pointer when num_tokens > 0) or
 * CPA_ERR_DEVICE.  Device-side inputs are trusted: row starts, contexts and
 * page ids must be those cpa_build_metadata accepted.
 */
int cpa_append_kv(const void* k_new, const void* v_new, const int32_t* d_query_start_loc,
                  const int32_t* d_context_lens, const int32_t* d_block_table, int bt_stride,
                  int num_seqs, int num_tokens, int num_kv_heads, int head_dim, int block_size,
                  void* k_cache, void* v_cache, void* stream);

/*
 * cpa_workspace_size -- bytes of device workspace cpa_attention needs for a
 * plan with these counts: the partial results of every split piece, with its
 * running max and sum in fp32.  A decode piece keeps its unnormalised fp32
 * output, a chunk piece its output divided by its own sum in bf16:
 * num_decode_partials * num_q_heads * (head_dim + 2) * 4 bytes plus
 * num_chunk_partials * num_kv_heads * R * (head_dim * 2 + 2 * 4) bytes (R,
 * the rows of a chunk tile: 256 at head_dim 128, 128 at 64), each of the six
 * regions rounded up to 256 bytes.  0 when nothing is split.
 */
size_t cpa_workspace_size(const cpa_plan_counts_t* counts, int num_q_heads, int num_kv_heads,
                          int head_dim);

/*
 * cpa_attention -- attention of every packed query over the paged cache.
 *
 * Query j of row s (position context_lens[s] + j) attends to keys
 * k <= context_lens[s] + j of its row: all earlier chunks plus causal inside
 * its own chunk ([P2] section 3; [P4] 4.1; [P5] "The fix").  Decode rows are
 * the one-query case.  out[t][h] = sum_k softmax(scale * <q[t][h], K[k]>) V[k]
 * with bf16 inputs, fp32 accumulation and a bf16 result (round to nearest
 * even); lse[t][h] = log(sum_k exp(scale * <q, K[k]>)) if lse is non-NULL.
 *
 * d_plan is the plan from cpa_build_metadata copied to the device, with its
 * counts in *counts (host pointer).  A contiguous run of the plan's sections
 * may be run alone by passing counts with the other sections set to 0 and
 * d_plan pointing at the first section run.  The decode and the chunk
 * sections are independent (they touch different output rows), so after this
 * step's append they may run concurrently on two streams; a merge section must
 * run after the split or tile section it merges, on the same stream or after
 * an event.  Both merge sections present in one call run as one launch.  workspace must hold
 * cpa_workspace_size(counts, ...) bytes (may be NULL when nothing is split);
 * its contents need no initialisation.  The append of this step must already
 * be enqueued on the same stream.  d_seq_lens is not read (the plan carries
 * the key ranges) and may be NULL.  Returns CPA_OK, CPA_ERR_UNSUPPORTED,
 * CPA_ERR_CAPACITY (workspace too small), CPA_ERR_INVALID or CPA_ERR_DEVICE.
 */
int cpa_attention(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* d_block_table, int bt_stride, const int32_t* d_query_start_loc,
                  const int32_t* d_seq_lens, const int32_t* d_context_lens, const int32_t* d_plan,
                  const cpa_plan_counts_t* counts, int num_seqs, int num_decodes, int num_tokens,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  float softmax_scale, void* out, float* lse, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * cpa_attention_noalloc -- cpa_attention for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, meaning and results as cpa_attention, without workspace /
 * workspace_bytes: the partial results of split pieces live in a
 * file-scope device array of CPA_NOALLOC_SCRATCH_BYTES (64 MiB) inside the
 * library, one copy per GPU, held until the process ends.  The call itself
 * allocates nothing (no hipMalloc, no hipFree); the first call on a device
 * looks the array's device address up once (hipGetSymbolAddress) on the
 * current device, which must be the device of `stream`.  Its contents need no
 * initialisation (every partial is written before it is read).  All calls on
 * one GPU share the array: two calls whose launches may overlap on one GPU
 * (different streams, or a graph replayed while another call runs) race on it
 * and must be ordered by the caller.  Returns CPA_ERR_CAPACITY, with nothing
 * launched, when cpa_workspace_size(counts, ...) exceeds
 * CPA_NOALLOC_SCRATCH_BYTES; CPA_ERR_DEVICE if the current device cannot be
 * read; otherwise as cpa_attention.
 */
#define CPA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int cpa_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* d_block_table, int bt_stride,
                          const int32_t* d_query_start_loc, const int32_t* d_seq_lens,
                          const int32_t* d_context_lens, const int32_t* d_plan,
                          const cpa_plan_counts_t* counts, int num_seqs, int num_decodes,
                          int num_tokens, int num_q_heads, int num_kv_heads, int head_dim,
                          int block_size, float softmax_scale, void* out, float* lse,
                          void* stream);

/* cpa_status_string -- static, human-readable name of a status code. */
const char* cpa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CPA_H */
