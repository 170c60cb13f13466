"""CPU oracle for paged attention over a block-table KV cache.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's product
path never imports, calls or links it, and this module imports nothing from
the library.

It is the plain definition, written out slowly:

1. *write*  - scatter each new token's K and V into the paged pool at
   ``slot = block_id * block_size + offset``.  TensorSharp, Mistral 3 page,
   section 11 "Batched / paged forward": K/V scatter via slotMapping into the
   per-layer paged buffer ``[numBlocks * blockSize * numKvHeads * headDim]``.
2. *gather* - copy a sequence's logical K/V out of the pool through its
   block table into a dense ``[n, num_kv_heads, head_dim]`` array, the
   per-sequence cache layout of sections 7 and 10 (heads-first there; the
   axis order does not change any value).  Section 11 describes exactly this
   gather-then-attend structure for the GGML backends.
3. *attend* - scaled dot products, causal mask, max-subtracted softmax and
   the weighted sum of V, per query head, with query head ``h`` reading kv
   head ``h // (num_heads / num_kv_heads)`` (grouped-query attention,
   sections 2, 3 and 4.1).  The 1/sqrt(head_dim) factor of section 3 is the
   ``scale`` argument and multiplies the dot product.

Readings where the pages are silent (each also listed in the design notes):

* causal alignment for a chunk of ``q_len`` new tokens over a context of
  ``n`` tokens (cached prefix + chunk): chunk token ``t`` sits at absolute
  position ``n - q_len + t`` and sees keys ``0 .. n - q_len + t``;
* a decode step is that rule with ``q_len = 1``: the newest token, already
  written, sees the whole context (section 3 appends before attending);
* the softmax is the plain one: no sliding window, sink or soft-cap
  (section 8: full attention only);
* a row with no visible key (``n = 0``) returns zeros;
* arithmetic is float64 unless ``acc_dtype`` says otherwise.

Key and value head dims may differ (section 4.1: separate key and value
lengths, each defaulting to the head dim).  Below, ``D`` is the key (and
query) head dim and ``Dv`` the value head dim, which is also the width of
the outputs; every function works for ``Dv == D`` and ``Dv != D`` alike.

Parity pins live in the CPU test suite; every function here is pinned.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_cache_write",
    "gather_sequence",
    "attention_weights",
    "attention",
    "paged_decode",
    "paged_prefill",
]


def kv_cache_write(k_cache, v_cache, key, value, slot_mapping):
    """Return copies of the caches with token ``t`` stored at slot
    ``slot_mapping[t]`` (TensorSharp Mistral 3, section 11, slotMapping
    scatter).

    ``k_cache``/``v_cache``: ``[num_blocks, block_size, num_kv_heads, D]``
    and ``[..., Dv]`` (any element type: the write is a copy).
    ``key``/``value``: ``[T, num_kv_heads, D]`` and ``[T, num_kv_heads, Dv]``.
    A negative slot skips its token.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    num_blocks, block_size = k.shape[0], k.shape[1]
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        block_id = slot // block_size
        offset = slot % block_size
        if block_id >= num_blocks:
            raise IndexError(f"slot {slot} outside a pool of {num_blocks} x {block_size}")
        k[block_id, offset] = key[t]
        v[block_id, offset] = value[t]
    return k, v


def gather_sequence(cache, table_row, n):
    """Dense ``[n, num_kv_heads, head_dim]`` copy of a sequence's first
    ``n`` logical tokens.  Logical position ``p`` lives in physical block
    ``table_row[p // block_size]`` at offset ``p % block_size``."""
    block_size = cache.shape[1]
    dense = np.empty((n,) + cache.shape[2:], dtype=cache.dtype)
    for j in range(-(-n // block_size)):
        start = j * block_size
        take = min(block_size, n - start)
        dense[start:start + take] = cache[int(table_row[j]), :take]
    return dense


def attention_weights(q_h, k_g, scale, query_pos, acc_dtype=np.float64):
    """Softmax weights ``P[t, p]`` of one query head.

    ``q_h``: ``[Tq, D]``; ``k_g``: ``[n, D]`` keys of the matching kv head;
    ``query_pos``: ``[Tq]`` absolute positions.  Key ``p`` is visible to
    query ``t`` iff ``p <= query_pos[t]``.  Masked entries get weight 0.
    """
    q_h = np.asarray(q_h, dtype=acc_dtype)
    k_g = np.asarray(k_g, dtype=acc_dtype)
    n = k_g.shape[0]
    scores = (q_h @ k_g.T) * acc_dtype(scale)                     # [Tq, n]
    visible = np.arange(n)[None, :] <= np.asarray(query_pos)[:, None]
    scores = np.where(visible, scores, -np.inf)
    weights = np.zeros_like(scores)
    for t in range(scores.shape[0]):
        if not visible[t].any():
            continue                                               # no key: zeros
        m = scores[t].max()
        e = np.where(visible[t], np.exp(scores[t] - m), acc_dtype(0))
        weights[t] = e / e.sum()
    return weights


def attention(q, k, v, scale, query_pos, acc_dtype=np.float64):
    """Grouped-query attention of ``q [Tq, Hq, D]`` over dense
    ``k [n, Hkv, D]``, ``v [n, Hkv, Dv]``; query head ``h`` uses kv head
    ``h // (Hq // Hkv)``.  Returns ``[Tq, Hq, Dv]`` in ``acc_dtype``."""
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError(f"num_heads {Hq} is not a multiple of num_kv_heads {Hkv}")
    group = Hq // Hkv
    out = np.zeros((Tq, Hq, v.shape[2]), dtype=acc_dtype)
    for h in range(Hq):
        g = h // group
        weights = attention_weights(q[:, h, :], k[:, g, :], scale, query_pos, acc_dtype)
        out[:, h, :] = weights @ np.asarray(v[:, g, :], dtype=acc_dtype)
    return out


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale,
                 acc_dtype=np.float64, seqs=None):
    """One query token per sequence over its whole context.

    ``q [S, Hq, D]``; caches ``[NB, BS, Hkv, D]`` and ``[NB, BS, Hkv, Dv]``
    already holding the new tokens; ``block_tables [S, max_blocks]``;
    ``context_lens [S]``.  ``seqs`` restricts the work to some sequences
    (others stay zero).  Returns ``[S, Hq, Dv]`` in ``acc_dtype``.
    """
    S, Hq, D = q.shape
    out = np.zeros((S, Hq, v_cache.shape[3]), dtype=acc_dtype)
    for i in (range(S) if seqs is None else seqs):
        n = int(context_lens[i])
        k = gather_sequence(k_cache, block_tables[i], n)
        v = gather_sequence(v_cache, block_tables[i], n)
        out[i:i + 1] = attention(q[i:i + 1], k, v, scale, np.array([n - 1]), acc_dtype)
    return out


def paged_prefill(q, query_start_loc, k_cache, v_cache, block_tables, context_lens, scale,
                  acc_dtype=np.float64, seqs=None):
    """Causal attention of each sequence's packed chunk over its cached
    prefix plus the chunk itself.

    Sequence ``i`` owns query rows ``query_start_loc[i] .. [i+1]-1`` of
    ``q [Tq, Hq, D]``; ``context_lens[i]`` counts prefix + chunk.  Returns
    ``[Tq, Hq, Dv]`` in ``acc_dtype``.
    """
    Tq, Hq, D = q.shape
    out = np.zeros((Tq, Hq, v_cache.shape[3]), dtype=acc_dtype)
    S = len(context_lens)
    for i in (range(S) if seqs is None else seqs):
        r0, r1 = int(query_start_loc[i]), int(query_start_loc[i + 1])
        q_len = r1 - r0
        n = int(context_lens[i])
        if q_len == 0:
            continue
        k = gather_sequence(k_cache, block_tables[i], n)
        v = gather_sequence(v_cache, block_tables[i], n)
        positions = n - q_len + np.arange(q_len)
        out[r0:r1] = attention(q[r0:r1], k, v, scale, positions, acc_dtype)
    return out
