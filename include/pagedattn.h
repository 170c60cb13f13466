/*
 * pagedattn.h - C ABI of a paged-attention library for AMD Instinct MI355X
 * (gfx950): paged attention over a block-table KV cache.
 *
 * The KV cache is a pool of fixed-size blocks.  Each sequence owns an
 * ordered list of block ids (its block table), and blocks may be shared
 * between sequences with a common prefix.  New tokens are scattered into
 * the pool through a slot mapping.  Decode and chunked-prefill attention
 * read the pool in place, block by block, through the tables.
 *
 * Sources, by page and passage:
 *   [TS]  TensorSharp, "Mistral 3" model page.  Section 3 "Forward graph"
 *         scales Q by 1/sqrt(headDim), appends K/V to the cache, then runs
 *         standard causal GQA attention.  Section 11 "Batched / paged
 *         forward" gives the per-layer paged buffer
 *         [numBlocks * blockSize * numKvHeads * headDim], the slotMapping
 *         scatter to blockId * blockSize + offset, and the online-softmax
 *         paged attention loop parallel over (sequence, head).
 *   [MR]  "Pure-Rust engines as a comparison" (mistral.rs), section on
 *         paged attention: blocks of 8, 16 or 32 tokens, default 32, and
 *         an explicit unsupported setting is an error rather than a silent
 *         fallback.  The scheduling section gives chunked prefill of up to
 *         512 tokens under a 4096-token budget.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer named *device* is HIP device memory.  The caller
 *    allocates and owns every buffer.  The library never allocates, never
 *    frees and never synchronises.  It keeps no per-call state, so calls
 *    are reentrant and may run on any number of streams at once.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *    Every call only enqueues work on it.  Results are visible after the
 *    caller synchronises with that stream.
 *  - Layouts are row-major and contiguous:
 *      k_cache          : [num_blocks, block_size, num_kv_heads, head_dim]
 *      v_cache          : [num_blocks, block_size, num_kv_heads, v_head_dim]
 *    where v_head_dim (the value head dim) is head_dim unless the cache
 *    descriptor sets it ([TS] section 4.1: separate key and value lengths,
 *    each defaulting to the head dim).
 *      block_tables     : [num_seqs, max_blocks_per_seq] int32
 *      context_lens     : [num_seqs] int32 (tokens already in the cache,
 *                         including the tokens this step wrote)
 *    A token at logical position p of sequence i sits in physical block
 *    block_tables[i][p / block_size] at offset p % block_size.  Its slot is
 *    block_id * block_size + offset.
 *  - Query head h reads kv head h / (num_heads / num_kv_heads).
 *  - `scale` multiplies every q.k dot product.  It is normally
 *    1/sqrt(head_dim); any finite value is accepted, zero and negative
 *    included, and every entry point applies it to the fp32 dot product
 *    before the softmax takes its max (a non-finite scale returns
 *    PA_ERR_SHAPE).
 *  - Element types: q, k_cache, v_cache and out share one dtype (fp32 or
 *    bf16).  Arithmetic is fp32 in either case.  bf16 outputs are rounded
 *    to nearest even.
 *  - Supported shapes: block_size in {8, 16, 32}, head_dim and v_head_dim
 *    each in {64, 128}, num_heads / num_kv_heads in {1, 2, 4, 8}.  Queries
 *    have head_dim elements per head, outputs v_head_dim.
 *
 * Errors
 * ------
 *  Every entry point checks its arguments on the host before it enqueues
 *  anything.  On failure it returns a negative pa_status and records a
 *  message naming what was expected and what it got; read the message
 *  with pa_last_error_message() (thread-local).  Nothing aborts.  A
 *  launch failure reported by the HIP runtime returns PA_ERR_HIP.  Faults
 *  during execution surface at the caller's next synchronisation.
 *
 *  Contracts on the *contents* of device buffers are the caller's, and the
 *  host cannot check them without reading device memory:
 *    - block ids lie in [0, num_blocks);
 *    - context_lens[i] <= max_context_len and
 *      context_lens[i] <= max_blocks_per_seq * block_size;
 *    - slots are distinct.
 *  The kernels still never touch memory outside the buffers the sizes
 *  describe.  A block id outside [0, num_blocks) drops that block's tokens
 *  from the softmax.  A context length above either bound is cut to the
 *  bound.  A slot outside [0, num_blocks * block_size) is skipped.  A
 *  result computed under a broken contract is unspecified.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_BF16 = 1
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                     */
  PA_ERR_DTYPE = -2,       /* dtype is not a pa_dtype value                  */
  PA_ERR_SHAPE = -3,       /* a size is out of range, or sizes disagree      */
  PA_ERR_BLOCK_SIZE = -4,  /* block_size not in {8, 16, 32}                  */
  PA_ERR_HEAD_DIM = -5,    /* head_dim not in {64, 128}                      */
  PA_ERR_GQA = -6,         /* num_heads / num_kv_heads not in {1, 2, 4, 8}   */
  PA_ERR_WORKSPACE = -7,   /* split-K workspace missing or too small         */
  PA_ERR_UNSUPPORTED = -8, /* a valid request this build does not implement  */
  PA_ERR_HIP = -9,         /* the HIP runtime reported an error              */
  PA_ERR_PARTITION = -10   /* partition_size not 0 or a positive multiple
                              of block_size                                  */
} pa_status;

/* One layer's paged KV pool.  The pointers are device memory owned by the
 * caller, contiguous, K laid out [num_blocks, block_size, num_kv_heads,
 * head_dim] and V [num_blocks, block_size, num_kv_heads, v_head_dim].
 * [TS] section 11 (layout), section 4.1 (separate key and value lengths). */
typedef struct pa_kv_cache {
  void *k_cache;
  void *v_cache;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;   /* key (and query) head dim */
  int32_t dtype;      /* pa_dtype */
  int32_t v_head_dim; /* value (and output) head dim; 0 means head_dim */
} pa_kv_cache;

/* ---------------------------------------------------------------------
 * pa_kv_cache_write - scatter new tokens' K and V into the paged pool.
 * [TS] section 11: the slotMapping scatter.  [TS] section 3: K/V are
 * appended before attention, so the tokens a step writes are attended by
 * that same step.
 *
 *   key, value   : device, [num_tokens, num_kv_heads, head_dim] and
 *                  [num_tokens, num_kv_heads, v_head_dim], cache dtype.
 *   slot_mapping : device, [num_tokens] int64.  Token t is copied to slot
 *                  slot_mapping[t], i.e. to block slot/block_size at offset
 *                  slot%block_size, for every kv head.  A negative slot
 *                  skips its token (padding).  A slot at or past
 *                  num_blocks*block_size is skipped as well.
 *   num_tokens   : >= 0.  0 enqueues nothing.
 *
 * The copy is bit-exact.  Slots must be distinct: if two tokens name the
 * same slot, which one lands there is unspecified.  Only num_kv_heads *
 * head_dim * element_size % 16 == 0 (and the same of v_head_dim) is
 * required of the shape; block_size and the head dims need not be in the
 * attention-supported sets.
 * --------------------------------------------------------------------- */
int pa_kv_cache_write(const pa_kv_cache *cache, const void *key, const void *value,
                      const int64_t *slot_mapping, int32_t num_tokens, void *stream);

/* ---------------------------------------------------------------------
 * pa_kv_cache_copy_blocks - copy whole blocks (K and V, every kv head)
 * from one pool to another, or inside one pool.  [TS] section 11: a pool
 * grown into a larger allocation keeps the K/V already written; with an id
 * map the same call copies a shared block into a sequence's own block.
 *
 *   src, dst         : pools with the same dtype, block_size, num_kv_heads,
 *                      head_dim and v_head_dim (num_blocks may differ; they
 *                      may be the same pool).
 *   src_ids, dst_ids : device, [num_copies] int32, copy i moves block
 *                      src_ids[i] of src to block dst_ids[i] of dst; or both
 *                      NULL to copy blocks 0 .. num_copies-1 to the same ids
 *                      (then num_copies must fit both pools).  A copy whose
 *                      id is outside its pool is skipped.  Destination ids
 *                      must be distinct, and no destination block may also
 *                      be a source block of the same call.
 *   num_copies       : >= 0.  0 enqueues nothing.
 * The copy is bit-exact.
 * --------------------------------------------------------------------- */
int pa_kv_cache_copy_blocks(const pa_kv_cache *src, const pa_kv_cache *dst, const int32_t *src_ids,
                            const int32_t *dst_ids, int32_t num_copies, void *stream);

/* ---------------------------------------------------------------------
 * pa_decode_workspace_bytes - bytes of fp32 workspace that split-K decode
 * needs: the per-partition running max m, sum l and unnormalised output
 * o[head_dim] for every (sequence, query head, partition), where there are
 * ceil(max_context_len / partition_size) partitions.  head_dim is the
 * width of the output rows: the cache's v_head_dim.  Returns 0 when
 * partition_size <= 0 (single pass) or when there is at most one
 * partition.  Negative sizes also give 0.
 * --------------------------------------------------------------------- */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size);

/* ---------------------------------------------------------------------
 * pa_decode - attention of one new query token per sequence over its whole
 * context in the paged cache.  [TS] section 3 (scaled causal GQA over the
 * cache, the new token included once written), section 11 (paged buffers
 * and the online-softmax loop over (sequence, head)).
 *
 *   out            : device, [num_seqs, num_heads, v_head_dim], cache dtype.
 *   q              : device, [num_seqs, num_heads, head_dim], cache dtype.
 *   block_tables   : device, [num_seqs, max_blocks_per_seq] int32.  Entries
 *                    past a sequence's last block are never read.
 *   context_lens   : device, [num_seqs] int32.  The query token is the
 *                    last of its sequence's context_lens[i] tokens and sees
 *                    all of them.  A context of 0 gives a zero output.
 *   max_context_len: host int, an upper bound of context_lens.  It sizes
 *                    the grid and the workspace, so no device read is
 *                    needed.
 *   scale          : multiplies q.k.
 *   partition_size : 0 for a single pass, with one work-group per
 *                    (sequence, kv head) walking the whole context.
 *                    Otherwise it is split-K flash-decoding: a positive
 *                    multiple of block_size that sets the tokens per
 *                    partition.  Each partition yields (m, l, o), and a
 *                    reduce kernel merges them with the same rescaling rule
 *                    the online softmax applies between tiles.  A sequence
 *                    that fits in one partition is written directly.
 *   workspace      : device, >= pa_decode_workspace_bytes(...) bytes when
 *                    partition_size > 0 and max_context_len > partition_size;
 *                    otherwise it may be NULL.  It is only scratch:
 *                    contents before and after the call carry no meaning.
 *
 * pa_decode enqueues pa_decode_partition and then pa_decode_reduce.
 * --------------------------------------------------------------------- */
int pa_decode(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs,
              int32_t num_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
              const int32_t *context_lens, int32_t max_context_len, float scale,
              int32_t partition_size, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------
 * pa_decode_static - pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and arguments, without the
 * workspace.  The split-K partials go to a static scratch array that the
 * library holds on every GPU it runs on, PA_STATIC_WORKSPACE_BYTES bytes,
 * until the process ends.  The call allocates nothing and frees nothing.
 *
 *   cache ... partition_size, stream : as pa_decode.
 *
 * A request whose partials need more than PA_STATIC_WORKSPACE_BYTES
 * (pa_decode_workspace_bytes of the same sizes) returns PA_ERR_WORKSPACE
 * before anything is enqueued; a larger partition_size or pa_decode with
 * a caller workspace serves it.  The current device must be the device of
 * `stream` (PA_ERR_SHAPE otherwise).  Every call on one GPU shares that
 * GPU's scratch: two calls whose kernels overlap on one GPU (different
 * streams, or graph replays in flight together) race and their results
 * are unspecified; calls ordered on one stream are safe.  The scratch
 * needs no clearing: each call writes every partial it reads.
 * --------------------------------------------------------------------- */
#define PA_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
int pa_decode_static(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs, int32_t num_heads,
                     const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                     int32_t max_context_len, float scale, int32_t partition_size, void *stream);

/* ---------------------------------------------------------------------
 * pa_decode_append - one whole decode step: writes each sequence's newest
 * K and V rows into the cache and attends over the context, as
 * pa_kv_cache_write (with slot = the slot of position context_lens[i] - 1
 * through the block table) followed by pa_decode.  [TS] section 3 appends
 * the new token's K/V to the cache and then attends with it; section 11
 * writes them through the slot mapping.  On bf16 pools the write happens
 * inside the partition kernel: the partition that holds the newest token
 * takes its rows from key / value and stores them into the slot, saving a
 * launch; fp32 pools run a separate write first.  Results equal pa_decode's up
 * to rounding (the newest token's weight is merged last).
 *
 *   cache ... workspace_bytes : as pa_decode.
 *   key, value : device, [num_seqs, num_kv_heads, head_dim] and
 *                [num_seqs, num_kv_heads, v_head_dim], cache dtype: the
 *                rows of position context_lens[i] - 1 of sequence i.  A
 *                sequence with context 0 has no new token (its rows are
 *                not read).  A slot whose block id is outside the pool is
 *                not written and its token is left out, as pa_decode
 *                leaves out a token in an invalid block.
 * --------------------------------------------------------------------- */
int pa_decode_append(const pa_kv_cache *cache, void *out, const void *q, const void *key, const void *value,
                     int32_t num_seqs, int32_t num_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t max_context_len, float scale, int32_t partition_size,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------
 * pa_decode_partition - first stage of pa_decode, same arguments.  It
 * writes the final output of every sequence with at most one partition.
 * For every other sequence it writes (m, l, o) per partition into the
 * workspace.  Call pa_decode_reduce afterwards on the same stream.  A
 * caller may run other work between the two stages.
 * --------------------------------------------------------------------- */
int pa_decode_partition(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs,
                        int32_t num_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                        const int32_t *context_lens, int32_t max_context_len, float scale,
                        int32_t partition_size, void *workspace, size_t workspace_bytes,
                        void *stream);

/* ---------------------------------------------------------------------
 * pa_decode_reduce - second stage of pa_decode.  For every sequence with
 * more than one partition, it merges the partitions' (m, l, o) into
 *   out = sum_p o_p * 2^(m_p - M) / sum_p l_p * 2^(m_p - M),  M = max_p m_p,
 * where m is kept in base-2 units of the scaled scores.  Sequences with
 * at most one partition are left untouched.  head_dim is the output row
 * width (the cache's v_head_dim).  dtype, num_seqs, num_heads,
 * head_dim, context_lens, max_context_len, partition_size and the
 * workspace must match the pa_decode_partition call that filled it.
 * --------------------------------------------------------------------- */
int pa_decode_reduce(void *out, int32_t dtype, int32_t num_seqs, int32_t num_heads,
                     int32_t head_dim, const int32_t *context_lens, int32_t max_context_len,
                     int32_t partition_size, const void *workspace, size_t workspace_bytes,
                     void *stream);

/* ---------------------------------------------------------------------
 * pa_decode_cascade - pa_decode for a batch whose sequences come in groups
 * that share a prefix of whole blocks (the same physical blocks lead their
 * block tables, as the block-hash prefix cache of [MR] produces; [TS]
 * section 11 reuses blocks across sequences the same way).  The shared
 * tokens are read once per group: in the same launch as the members' own
 * tokens (split-K partitions after the shared ones), work-groups compute
 * every member's attention over the shared tokens on MFMA tiles whose
 * columns are the members' query heads (one split-K partial per 512-token
 * chunk), and the reduce merges all of them.  The workspace holds
 * ceil(max_context_len / 512) + ceil(max_context_len / partition_size)
 * partials per (row, head).  The result
 * is pa_decode's up to rounding.
 *
 *   cache ... partition_size : as pa_decode (partition_size > 0 required).
 *   num_groups     : >= 1 when num_seqs > 0.
 *   group_start    : device, [num_groups + 1] int32, ascending, from 0 to
 *                    num_seqs: group g is rows group_start[g] ..
 *                    group_start[g+1]-1 (a sequence sharing nothing is a
 *                    group of one with shared_len 0).
 *   shared_len     : device, [num_groups] int32, tokens the group shares
 *                    (any count, usually a multiple of block_size): every
 *                    row of the group that has a token at position
 *                    p < shared_len keeps it in the same block.  The shared blocks are read through the
 *                    table of the group's longest row; a row whose context
 *                    ends inside the shared part sees only its own tokens.
 *   max_group_size : host int, >= every group's size (sizes the grid).
 *   max_shared_len : host int, >= 0, an upper bound of shared_len that sizes
 *                    the launch's shared chunks (ceil(max_shared_len / 512)
 *                    per group).  A shared_len above it is clamped to
 *                    512 * that many chunks; the tokens past the clamp
 *                    run in the members' own partitions, so the result
 *                    stays correct and only the sharing is lost.
 *   workspace      : device, >= pa_decode_cascade_workspace_bytes(...)
 *                    bytes; scratch.
 * bf16 only (PA_ERR_UNSUPPORTED otherwise).  The workspace size takes the
 * width of the output rows (the cache's v_head_dim) as head_dim, as
 * pa_decode_workspace_bytes does.
 * --------------------------------------------------------------------- */
size_t pa_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size);
int pa_decode_cascade(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs, int32_t num_heads,
                      const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                      int32_t max_context_len, float scale, int32_t partition_size, int32_t num_groups,
                      const int32_t *group_start, const int32_t *shared_len, int32_t max_group_size,
                      int32_t max_shared_len, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------
 * pa_prefill_chunk - causal attention of a packed chunk of new tokens per
 * sequence over that sequence's cached prefix plus the chunk itself.
 * [TS] section 3: scaled causal GQA; the chunk's K/V are written with
 * pa_kv_cache_write first.  [MR] scheduling section: prefill proceeds in
 * chunks of up to 512 tokens under a 4096-token step budget.
 *
 *   out, q          : device, [num_query_tokens, num_heads, v_head_dim] and
 *                     [num_query_tokens, num_heads, head_dim], cache
 *                     dtype.  Sequence i owns rows
 *                     query_start_loc[i] .. query_start_loc[i+1]-1.
 *   query_start_loc : device, [num_seqs + 1] int32, non-decreasing, with
 *                     last entry <= num_query_tokens.  Rows at or past
 *                     num_query_tokens are never touched.
 *   max_query_len   : host int, an upper bound of each sequence's row
 *                     count.  It sizes the grid.
 *   context_lens    : device, [num_seqs] int32: cached prefix plus chunk.
 *                     Chunk row t of sequence i has absolute position
 *                     context_lens[i] - q_len_i + t and sees keys at
 *                     positions 0 .. that position (causal mask aligned to
 *                     the end of the context).
 *   block_tables, max_blocks_per_seq, max_context_len, scale : as for
 *                     pa_decode.
 *
 * bf16 runs on bf16 MFMA tiles with fp32 accumulation; the softmax
 * weights are rounded to bf16 before they multiply V.  fp32 runs every
 * packed row as a single-pass decode of its own (fp32 arithmetic
 * throughout, no tiling across rows), at most 65535 query rows
 * (PA_ERR_UNSUPPORTED above that).
 * --------------------------------------------------------------------- */
int pa_prefill_chunk(const pa_kv_cache *cache, void *out, const void *q,
                     const int32_t *query_start_loc, int32_t num_seqs, int32_t num_heads,
                     int32_t num_query_tokens, int32_t max_query_len,
                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t max_context_len, float scale,
                     void *stream);

/* Short static name of a status code, e.g. "PA_ERR_BLOCK_SIZE". */
const char *pa_status_string(int status);

/* Message of the last failed call on this thread, e.g.
 * "block_size 24 not in {8, 16, 32}".  Empty after a successful call. */
const char *pa_last_error_message(void);

/* Library version as major*10000 + minor*100 + patch. */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
