/*
 * pagedattn_kvm.h - host-side KV block manager and step scheduler for the
 * paged-attention library (C ABI, host memory only, no GPU calls).
 *
 * Sources, by page and passage:
 *   [MR] "Pure-Rust engines as a comparison" (mistral.rs).  The
 *        paged-attention section gives a vLLM-v1-style KV cache manager
 *        (get_computed_blocks, allocate_slots, free, cache_blocks) over a
 *        flat block pool with an LRU free list and content-addressed block
 *        hashing: full blocks are registered and a lookup follows the hash
 *        chain to the longest hit.  The scheduling section gives
 *        alternating steps (all prompt or all completion, a 4096-token
 *        budget, 512-token chunks, at most 8 decode steps in a row).
 *   [TS] TensorSharp, Mistral 3 page, section 11: blocks shared across
 *        sequences by block-hash prefix caching, with reuse counters.
 *
 * Everything here runs on the host.  A manager owns host memory (its
 * tables); the caller owns the device KV pool, whose block ids the manager
 * hands out.  Functions are not thread-safe on the same object.
 * Return values are pa_status codes (pagedattn.h) plus PA_ERR_NO_BLOCKS;
 * failures set pa_last_error_message().
 */
#ifndef PAGEDATTN_KVM_H
#define PAGEDATTN_KVM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_ERR_NO_BLOCKS = -11,  /* the pool cannot hold the request (nothing changed) */
  PA_ERR_REQUEST = -12     /* unknown or duplicate request id, or bad state     */
};

typedef struct pa_kvm pa_kvm; /* opaque */

typedef struct pa_kvm_stats {
  int64_t num_blocks;
  int64_t block_size;
  int64_t free_blocks;        /* blocks on the free list (cached ones included)   */
  int64_t cached_blocks;      /* blocks registered under a content hash           */
  int64_t active_requests;
  int64_t prefix_queries;     /* get_computed_blocks calls                        */
  int64_t prefix_hit_blocks;  /* blocks reused from the cache (cumulative)        */
  int64_t prefix_hit_tokens;  /* tokens reused from the cache (cumulative)        */
  int64_t evictions;          /* cached blocks recycled by an allocation          */
} pa_kvm_stats;

/* A manager for a pool of num_blocks blocks of block_size tokens
 * (block_size in {8, 16, 32}, as the attention kernels require).
 * enable_prefix_cache = 0 disables hashing and lookups.  NULL on error. */
pa_kvm *pa_kvm_create(int32_t num_blocks, int32_t block_size, int32_t enable_prefix_cache);
void pa_kvm_destroy(pa_kvm *m);

/* Register a request and its prompt token ids.  The manager keeps the
 * token ids (they are what blocks are hashed on). */
int pa_kvm_add_request(pa_kvm *m, int64_t request_id, const int32_t *token_ids, int32_t num_tokens);

/* Append token ids (sampled tokens) to a request's sequence. */
int pa_kvm_append_tokens(pa_kvm *m, int64_t request_id, const int32_t *token_ids, int32_t num_tokens);

/* For a request with no blocks yet: attach the longest chain of cached full
 * blocks that matches its leading tokens, and count them as computed.  At
 * least one token is always left to compute.  *num_computed_tokens
 * receives the number of tokens covered (a multiple of block_size). */
int pa_kvm_get_computed_blocks(pa_kvm *m, int64_t request_id, int32_t *num_computed_tokens);

/* Make room for num_new_tokens more tokens after the computed ones:
 * allocate blocks from the free list (recycling least-recently-freed
 * cached blocks first).  All or nothing: PA_ERR_NO_BLOCKS leaves the state
 * unchanged. */
int pa_kvm_allocate_slots(pa_kvm *m, int64_t request_id, int32_t num_new_tokens);

/* Mark num_tokens more tokens as computed (their K/V are in the pool) and
 * register every block that became full under its content hash. */
int pa_kvm_commit(pa_kvm *m, int64_t request_id, int32_t num_tokens);

/* Release a finished or preempted request.  Blocks whose reference count
 * drops to zero return to the free list, the request's last block first,
 * so the shared prefix blocks stay cached the longest. */
int pa_kvm_free(pa_kvm *m, int64_t request_id);

/* The request's block table (physical block ids in logical order).
 * *num_blocks receives the count; at most max_blocks are written. */
int pa_kvm_block_table(const pa_kvm *m, int64_t request_id, int32_t *table, int32_t max_blocks,
                       int32_t *num_blocks);

/* Slots (block_id * block_size + offset) of logical positions
 * first_pos .. first_pos + count - 1, which must be covered by allocated
 * blocks. */
int pa_kvm_slot_mapping(const pa_kvm *m, int64_t request_id, int32_t first_pos, int32_t count,
                        int64_t *slots);

/* Tokens of the request so far, and how many of them are computed. */
int pa_kvm_request_info(const pa_kvm *m, int64_t request_id, int32_t *num_tokens,
                        int32_t *num_computed_tokens, int32_t *num_blocks);

int pa_kvm_get_stats(const pa_kvm *m, pa_kvm_stats *stats);

/* Grow the pool to new_num_blocks (>= the current count), after the caller
 * has moved the device pool into an allocation of that size (e.g. with
 * pa_kv_cache_copy_blocks; [TS] section 11, the grow path of the paged
 * buffers).  Block ids already handed out keep their meaning; the new ids
 * go to the front of the free list, so they are used before any cached
 * block is recycled. */
int pa_kvm_grow(pa_kvm *m, int32_t new_num_blocks);

/* ------------------------------------------------------------------------
 * Step scheduler: alternates all-prompt and all-completion steps ([MR]
 * scheduling section).
 *
 * Reading of the policy used here (the page gives the rule and the limits
 * but not every tie-break):
 *  - Prompt work is a partly computed prompt or a waiting request.  A step
 *    is a prompt step when there is prompt work and either no sequence is
 *    decoding or at least min_decode_steps decode steps ran since the last
 *    prompt step (max_decode_steps caps the run of decode steps when
 *    min_decode_steps is set higher).  Otherwise it is a decode step; a
 *    prompt step that can place nothing falls back to a decode step.
 *  - A prompt step continues partly computed prompts in admission order,
 *    then admits waiting requests first come, first served (after attaching
 *    their cached prefix blocks).  Each sequence contributes at most
 *    max_chunk_tokens of its remaining tokens, the step at most
 *    max_batched_tokens (and cap_tokens) tokens and max_seqs sequences.  A
 *    waiting request whose blocks cannot be allocated stops admission.
 *  - A decode step gives every decoding sequence one token, in admission
 *    order.
 *  - When an admitted request needs a block and the pool is empty, the most
 *    recently admitted request after it (not already in the step) is
 *    preempted: its blocks are released and it returns to the front of the
 *    waiting queue with all its tokens, which it later recomputes (its
 *    full blocks usually still hit the prefix cache).  With nobody to
 *    preempt the request waits for a later step.
 *  - A request's block table must fit a step row (cap_blocks), and the
 *    oldest request must fit the pool; otherwise next_step fails with
 *    PA_ERR_SHAPE or PA_ERR_NO_BLOCKS.
 *
 * Mixed policy (config.mixed != 0; the one-batch variant of the same
 * limits): every step first gives each decoding sequence one token, in
 * admission order, then fills the rest of max_batched_tokens with prompt
 * chunks as a prompt step does.  Decode tokens count against the budget.
 * A step holding both kinds is kind 3 and runs as one pa_prefill_chunk
 * over all its rows (a decode row is a chunk of one token); a step with
 * one kind only is kind 1 or 2 as above.
 * ------------------------------------------------------------------------ */
typedef struct pa_sched pa_sched; /* opaque */

typedef struct pa_sched_config {
  int32_t max_batched_tokens;   /* 4096 */
  int32_t max_chunk_tokens;     /* 512  */
  int32_t max_decode_steps;     /* 8    */
  int32_t min_decode_steps;     /* 1    */
  int32_t max_seqs;             /* sequences per step */
  int32_t mixed;                /* 0: alternate; else one mixed batch per step */
} pa_sched_config;

/* One step's inputs for the attention kernels, written into caller-owned
 * host arrays of the given capacities.  kind: 0 = none (idle), 1 = prompt
 * (use pa_prefill_chunk), 2 = decode (use pa_decode), 3 = mixed (decode rows
 * first, then prompt chunks; use pa_prefill_chunk over all rows). */
typedef struct pa_step {
  int32_t kind;
  int32_t num_seqs;
  int32_t num_tokens;           /* new tokens this step (rows of q)           */
  int32_t max_query_len;
  int32_t max_context_len;
  int32_t max_blocks_per_seq;   /* row stride of block_tables                 */
  int64_t *request_ids;         /* [cap_seqs]                                 */
  int32_t *query_start_loc;     /* [cap_seqs + 1]                             */
  int32_t *context_lens;        /* [cap_seqs]  computed + new tokens          */
  int32_t *block_tables;        /* [cap_seqs * cap_blocks]                    */
  int64_t *slot_mapping;        /* [cap_tokens]                               */
  int32_t cap_seqs, cap_tokens, cap_blocks;
} pa_step;

pa_sched *pa_sched_create(pa_kvm *kvm, const pa_sched_config *cfg);
void pa_sched_destroy(pa_sched *s);
int pa_sched_add_request(pa_sched *s, int64_t request_id, const int32_t *prompt, int32_t prompt_len,
                         int32_t max_new_tokens);
/* Plan the next step into *step. */
int pa_sched_next_step(pa_sched *s, pa_step *step);
/* After the step ran: commit its tokens.  Every sequence whose tokens are
 * now all computed (a decode step, or the prompt step that finished its
 * prompt) either finishes, when it already produced max_new_tokens tokens
 * (its blocks are freed), or appends sampled[i] (step order; token id 0 when
 * sampled is NULL).  *num_finished receives how many finished. */
int pa_sched_complete_step(pa_sched *s, const pa_step *step, const int32_t *sampled, int32_t *num_finished);
/* Requests not admitted (new or preempted), admitted (prefilling or
 * decoding), and finished so far. */
int pa_sched_counts(const pa_sched *s, int32_t *waiting, int32_t *running, int32_t *finished);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_KVM_H */
