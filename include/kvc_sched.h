/*
 * kvc_sched.h - iteration-level scheduler and step builder for the paged KV
 * cache: decides, step by step, which requests decode a token and which
 * prompt chunks prefill, and builds the kernels' batch descriptors for that
 * step (block tables, context lengths, chunk offsets).
 *
 * Policies (restated from aiwithghost.com "KV cache and continuous batching:
 * 1,000 people ask AI", sections "How does continuous batching share the
 * server?" and "What our lab measured", and gouthm.com "The KV cache is not
 * your bottleneck", section "The fix that mattered"):
 *   KVC_SCHED_PREFILL_FIRST  continuous batching: at the start of every step
 *       free slots take the next queued requests in queue order; while any
 *       admitted prompt still has tokens to prefill, the step prefills only
 *       (decode pauses), chunks taken in admission order up to the token
 *       budget; otherwise every admitted request decodes one token.
 *   KVC_SCHED_DECODE_FIRST   continuous batching with decode given strict
 *       priority: every request that has its first token decodes at every
 *       step, and prompt chunks (admission order) fill the token budget of the
 *       same step, so a long prompt is split over several steps and delays
 *       decode by at most one chunk (budget 2,048 on the gouthm page).
 *   KVC_SCHED_STATIC         static batching: groups of `slots` requests in
 *       queue order; a group prefills all its prompts in its first step
 *       (budget not applied) and decodes until its longest answer is done;
 *       finished requests idle in their slots; the next group starts after.
 * A prompt's last prefill chunk yields the answer's first token; each later
 * token takes one decode step. A request leaves after the step that makes its
 * answer_len-th token. A decode row of a request with prompt length p and g
 * tokens generated so far writes its newest token's K/V at position p + g - 1
 * and attends over p + g positions (context_lens as kvc_decode_append_attention
 * takes them).
 *
 * Cache blocks: the scheduler owns a pool of num_blocks block ids (the first
 * dimension of every layer's kvc_cache pool). Before a step, each of its rows
 * (decode rows first, then prefill chunks, in the order listed) takes the
 * lowest-numbered free ids until it holds ceil(tokens / 16) blocks, counting
 * the tokens the step writes; a request that leaves returns all of its blocks
 * after its last step. Admission does not reserve memory: a step that the pool
 * cannot cover fails with KVC_ERR_NO_BLOCKS and changes nothing (pre-emption
 * is not done; a pool of slots * max_blocks_per_seq blocks never runs out).
 *
 * Host memory only: no call touches the GPU. An object is not thread-safe.
 * Errors return a negative kvc status (kvc.h) and leave the object unchanged.
 */
#ifndef KVC_SCHED_H
#define KVC_SCHED_H

#include <stdint.h>

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVC_SCHED_PREFILL_FIRST = 0,
  KVC_SCHED_DECODE_FIRST = 1,
  KVC_SCHED_STATIC = 2,
};

typedef struct kvc_sched kvc_sched;

/* A scheduler with `slots` concurrent requests, a prefill budget of
 * token_budget prompt tokens per step (continuous policies), a pool of
 * num_blocks 16-token cache blocks and block tables of max_blocks_per_seq
 * columns. Returns NULL for an unknown policy, slots < 1, token_budget < 1,
 * num_blocks < 0, max_blocks_per_seq < 1 or when memory runs out. */
kvc_sched* kvc_sched_create(int32_t policy, int32_t slots, int32_t token_budget,
                            int32_t num_blocks, int32_t max_blocks_per_seq);

/* Frees the scheduler (NULL is ignored). */
void kvc_sched_destroy(kvc_sched* s);

/* Queues a request with a prompt of prompt_len tokens whose answer has
 * answer_len tokens. Returns its id (0, 1, 2, ... in submission order), or
 * KVC_ERR_SHAPE when a length is < 1 or prompt_len + answer_len - 1 tokens do
 * not fit max_blocks_per_seq blocks. */
int32_t kvc_sched_submit(kvc_sched* s, int32_t prompt_len, int32_t answer_len);

/* Requests queued or running. */
int32_t kvc_sched_unfinished(const kvc_sched* s);

/* One step's plan and batch descriptors, written into caller-owned host
 * arrays. Each id / length array has room for `slots` rows, prefill_cu_chunk_lens
 * for slots + 1, each block table for slots * max_blocks_per_seq entries
 * (row-major, one row per listed request, unused columns -1). */
typedef struct kvc_step {
  /* decode rows, in admission order */
  int32_t n_decode;
  int32_t* decode_ids;
  int32_t* decode_context_lens;  /* p + g: positions attended, the newest included */
  int32_t* decode_block_table;
  int32_t decode_max_context;    /* max of decode_context_lens, 0 with no rows */
  /* prefill chunks, in admission order */
  int32_t n_prefill;
  int32_t* prefill_ids;
  int32_t* prefill_prefix_lens;   /* first prompt position of the chunk */
  int32_t* prefill_cu_chunk_lens; /* n_prefill + 1 offsets into the packed chunk rows */
  int32_t* prefill_block_table;
  int32_t prefill_total_tokens;
  int32_t prefill_max_chunk;
  int32_t prefill_max_context;   /* max of prefix + chunk, 0 with no chunks */
  /* requests whose first token this step makes, and those leaving after it */
  int32_t n_first;
  int32_t* first_token_ids;
  int32_t n_finished;
  int32_t* finished_ids;
} kvc_step;

/* Builds the next step into *step and advances the scheduler past it (the
 * step's tokens count as made). Returns 1 when a step was built, 0 when no
 * request is queued or running (*step then holds empty counts), or a negative
 * status: KVC_ERR_NULL for a NULL pointer, KVC_ERR_NO_BLOCKS when the pool
 * cannot cover the step (nothing changes). */
int32_t kvc_sched_next_step(kvc_sched* s, kvc_step* step);

#ifdef __cplusplus
}
#endif

#endif /* KVC_SCHED_H */
