/*
 * ha_scheduler.h -- token-budget step generator for chunked prefill (host C ABI
 * of libhybridattn.so).
 *
 * Turns a stream of requests (prompt length, number of tokens to generate)
 * into a sequence of mixed steps and writes, for each step, exactly the
 * metadata paged_kv_append and hybrid_attn_fwd take: cu_seqlens_q,
 * seqlens_k, block_table and slot_mapping, with pages handed out from a pool
 * of num_blocks 16-token pages.
 *
 * Policy (wangyu.me, "大语言模型推理优化（二）：Chunked Prefill", section on the
 * vLLM implementation: the per-step token budget max_num_batched_tokens and
 * the scheduler that serves running requests first and fills the rest from
 * the waiting queue):
 *   - every step has a budget of max_num_batched_tokens tokens;
 *   - first, running requests in admission order: each takes its remaining
 *     tokens (all known tokens not yet through the model: 1 for a request that
 *     is decoding, the rest of the prompt for one still in prefill), capped by
 *     long_prefill_token_threshold when that is > 0, and by what is left of the
 *     budget;
 *   - then waiting requests in arrival order are admitted while budget is
 *     left, each with min(prompt, threshold if > 0, budget left) tokens;
 *   - so a prompt is cut into chunks of size min(remaining, budget left) --
 *     there is no fixed chunk size.
 *   After a step, a request that has caught up with its known tokens (its last
 *   prompt chunk, or a decode token) samples one new token; a request that has
 *   sampled max_new_tokens tokens is finished and its pages return to the pool
 *   (the last sampled token is never fed back).
 * Readings where the page is silent: the threshold applies to new requests too
 * (its stated purpose is to bound a long prompt's first chunk); a request is
 * admitted or extended only as far as free pages allow (no preemption): its
 * chunk shrinks to the tokens that fit, and a request that gets no token waits.
 *
 * Segments of a step are packed in the order above.  seqlens_k[b] = tokens of
 * the request already through the model + this step's tokens; the query rows
 * of segment b are the request's token positions first_pos[b] ..
 * first_pos[b] + Lq_b - 1; slot_mapping holds their cache slots
 * (page * 16 + position % 16) in the same order.
 *
 * Host memory only; the scheduler allocates with new/malloc and is not
 * thread-safe (one owner).  No GPU call is made.
 */
#ifndef HA_SCHEDULER_H
#define HA_SCHEDULER_H

#include <stdint.h>

#include "hybrid_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ha_sched ha_sched;

typedef struct {
  int32_t num_seqs;      /* segments in the step (0 when nothing is left to run) */
  int32_t total_q;       /* query rows = tokens through the model this step */
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int32_t num_decodes;   /* segments with one query row taken by a decoding request */
  int32_t num_sampling;  /* segments that sample a token after this step */
} ha_step_shape;

/*
 * ha_sched_create -- a scheduler with a per-step token budget, an optional
 * long-prefill threshold (0 = none), a pool of num_blocks pages of 16 tokens
 * and block-table rows of max_blocks_per_seq entries.  NULL on invalid
 * arguments (budget < 1, threshold < 0, num_blocks < 1, max_blocks_per_seq < 1)
 * or when out of host memory.
 */
ha_sched* ha_sched_create(int32_t max_num_batched_tokens, int32_t long_prefill_token_threshold,
                          int32_t num_blocks, int32_t max_blocks_per_seq);

/* ha_sched_destroy -- frees the scheduler (NULL is ignored). */
void ha_sched_destroy(ha_sched* s);

/*
 * ha_sched_add_request -- queues a request at the end of the waiting queue.
 * HA_ERR_INVALID_ARGUMENT for prompt_len < 1, max_new_tokens < 1, a request
 * whose prompt + max_new_tokens - 1 tokens need more than max_blocks_per_seq
 * pages, a duplicate live request_id, or a call between next_step and
 * complete_step.
 */
ha_status ha_sched_add_request(ha_sched* s, int64_t request_id, int32_t prompt_len,
                               int32_t max_new_tokens);

/*
 * ha_sched_next_step -- plans the next step and writes its metadata into
 * caller-owned host arrays:
 *   cu_seqlens_q  [max_seqs + 1]
 *   seqlens_k, request_ids, first_pos  [max_seqs]
 *   block_table   [max_seqs, max_blocks_per_seq] (entries past a segment's
 *                 pages are -1)
 *   slot_mapping  [max_tokens]
 * A step has at most max_seqs segments (requests beyond them wait, as with a
 * max_num_seqs limit).  HA_ERR_INVALID_ARGUMENT for null pointers,
 * max_seqs < 1, max_tokens smaller than the budget, or a step already planned
 * and not completed; HA_ERR_UNSUPPORTED when requests are left but no token can
 * be scheduled (pool exhausted).  A step with num_seqs = 0 means nothing is left.
 */
ha_status ha_sched_next_step(ha_sched* s, ha_step_shape* shape, int32_t* cu_seqlens_q,
                             int32_t* seqlens_k, int32_t* block_table, int32_t* slot_mapping,
                             int64_t* request_ids, int32_t* first_pos, int32_t max_seqs,
                             int32_t max_tokens);

/*
 * ha_sched_complete_step -- marks the planned step as run: advances every
 * scheduled request, samples, finishes requests and frees their pages.
 * finished_ids (may be NULL) receives up to max_finished ids of the requests
 * that finished; *num_finished (may be NULL) their count.
 * HA_ERR_INVALID_ARGUMENT when no step is planned.
 */
ha_status ha_sched_complete_step(ha_sched* s, int64_t* finished_ids, int32_t max_finished,
                                 int32_t* num_finished);

/* ha_sched_num_unfinished -- requests waiting or running (-1 for NULL). */
int32_t ha_sched_num_unfinished(const ha_sched* s);

/* ha_sched_free_blocks -- pages currently in the free pool (-1 for NULL). */
int32_t ha_sched_free_blocks(const ha_sched* s);

#ifdef __cplusplus
}
#endif

#endif /* HA_SCHEDULER_H */
