/*
 * pagedattn_serve.h - a native serving step over the paged-attention
 * library (MI355X, gfx950): the step scheduler of pagedattn_kvm.h plans a
 * step straight into pinned host memory, the step's block tables, context
 * lengths, query offsets and slot mapping travel to the device in one
 * asynchronous copy, and the step's K/V write and attention launches are
 * enqueued from here, so a serving loop spends one call per step on the
 * host side of the kernels.
 *
 * A step has three calls, in the order a model runs them:
 *   pa_serve_plan     the scheduler plans the step (the alternating or mixed
 *                     policy of pagedattn_kvm.h) and its arrays are copied to
 *                     the device on `stream`; the caller reads which
 *                     requests and positions the step holds and computes
 *                     their q, k and v rows;
 *   pa_serve_attend   writes the step's new K/V rows into the pool through
 *                     its slot mapping (pa_kv_cache_write) and runs
 *                     pa_prefill_chunk (prompt steps) or pa_decode (decode
 *                     steps) on `stream`; a mixed step runs all its rows
 *                     through pa_prefill_chunk (a decode row is a chunk of
 *                     one token), or, when one of its decode rows has a
 *                     context of mixed_split_context tokens or more and
 *                     longer than every chunk's context, its leading
 *                     one-token rows through split-K pa_decode and the
 *                     prompt chunks after them through pa_prefill_chunk;
 *   pa_serve_complete commits the step with the tokens sampled from it.
 *
 * Two pinned staging buffers alternate: a plan waits (on the host) for the
 * copy out of the buffer it reuses, issued two plans earlier, so the
 * arrays a plan returns stay valid until the plan after the next.  The
 * object is not thread-safe; calls on one object must come from one thread
 * in plan / attend / complete order.
 */
#ifndef PAGEDATTN_SERVE_H
#define PAGEDATTN_SERVE_H

#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"
#include "pagedattn_kvm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_serve pa_serve; /* opaque */

/* Bytes of the caller-owned device buffer that receives a step's arrays
 * (slot mapping, query offsets, context lengths, block tables) for steps of
 * at most max_seqs sequences, max_tokens new tokens and max_blocks_per_seq
 * table entries per sequence; 0 if a size is not positive. */
size_t pa_serve_meta_bytes(int32_t max_seqs, int32_t max_blocks_per_seq, int32_t max_tokens);

/* A serving object over the scheduler `sched` (which it does not own and
 * which must outlive it).  The capacities bound every step (the scheduler's
 * max_seqs, its max_batched_tokens or more, and the longest block table);
 * num_heads is the query heads of q, scale multiplies every q.k and
 * partition_size is the split-K partition of decode steps (0: one pass per
 * sequence).  mixed_split_context (0: never) is the decode-row context at
 * which a mixed step's decode rows go through split-K decode instead of the
 * prefill kernel, which gives each of them one work-group per kv head: a
 * long context then spreads over many work-groups (only when that row is
 * also longer than every chunk's context in the step).  `dev_meta` is a device
 * buffer of at least
 * pa_serve_meta_bytes(...) bytes, owned by the caller and used by every
 * step.  The object allocates its two pinned staging buffers and two HIP
 * events on the current device.  Returns NULL on a bad argument or a failed
 * allocation (message in pa_last_error_message). */
pa_serve *pa_serve_create(pa_sched *sched, int32_t num_heads, float scale, int32_t partition_size,
                          int32_t mixed_split_context, int32_t max_seqs, int32_t max_blocks_per_seq,
                          int32_t max_tokens, void *dev_meta, size_t dev_meta_bytes);
void pa_serve_destroy(pa_serve *s);

/* Plans the next step into *step (its arrays point into the pinned staging
 * buffer) and enqueues the copy of its arrays to dev_meta on `stream`.
 * step->kind 0 means nothing to run (no copy is enqueued).  Returns PA_OK
 * or the scheduler's error (e.g. PA_ERR_NO_BLOCKS), PA_ERR_HIP if the copy
 * cannot be enqueued, PA_ERR_SHAPE if a plan is still waiting for its
 * complete call. */
int pa_serve_plan(pa_serve *s, pa_step *step, void *stream);

/* Enqueues the planned step's K/V write and attention on `stream` (the
 * stream of its plan, so that they follow the copy): new_key
 * and new_value are the step's new rows [num_tokens, num_kv_heads, head_dim
 * (v_head_dim)], q [num_tokens, num_heads, head_dim] and out [num_tokens,
 * num_heads, v_head_dim], device pointers in step order; the pool is
 * `cache`.  The split-K partials of a decode step, or of a mixed step's
 * decode rows, go to `workspace` (at least pa_decode_workspace_bytes(
 * num_seqs, num_heads, v_head_dim, max_context_len, partition_size) bytes;
 * may be NULL when the partition size is 0).  Returns PA_OK, PA_ERR_SHAPE when no step is planned, or the
 * status of the write or attention call. */
int pa_serve_attend(pa_serve *s, const pa_kv_cache *cache, const void *new_key, const void *new_value,
                    const void *q, void *out, void *workspace, size_t workspace_bytes, void *stream);

/* Commits the planned step (pa_sched_complete_step with its arrays):
 * sampled[i] is the token sampled for sequence i of the step (NULL: token
 * id 0).  *num_finished receives how many requests finished. */
int pa_serve_complete(pa_serve *s, const int32_t *sampled, int32_t *num_finished);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_SERVE_H */
