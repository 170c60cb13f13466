"""Seeded generators for the five synthetic paged-attention workloads.

Everything here is *input construction*: drawing context lengths, laying
sequences out in a block pool, building block tables and slot mappings, and
drawing Q/K/V.  No attention arithmetic happens here.

Recipe (shared by every workload):

* one ``numpy.random.default_rng(seed)`` (PCG64) per case;
* draw order: context lengths -> block placement (one permutation of the
  pool) -> Q -> K pool -> V pool -> boost mask;
* values are standard normal float32; bf16 cases round them to the nearest
  bf16 (ties to even) and both sides consume those rounded values;
* the cache layout is ``[num_blocks, block_size, num_kv_heads, head_dim]``,
  the flat product order of the per-layer paged buffers in the TensorSharp
  Mistral 3 page, section 11 ("Batched / paged forward"); the V pool's last
  dim is the value head dim, which a case may draw apart from the key head
  dim (section 4.1: separate key and value lengths);
* a slot is ``block_id * block_size + offset`` (same section, the
  slotMapping scatter);
* in "poison" mode every slot that no sequence references, including the
  tails of partially filled blocks, holds NaN, and so does every slot that
  the new tokens will be written to, so a kernel that reads outside the
  context or attends before writing produces NaN;
* block-table entries past a sequence's last block are padded with the id of
  an unreferenced (hence NaN-filled in poison mode) block.

The newest token(s) of each sequence are not in the cache when a case is
handed out: ``new_key``/``new_value`` carry them together with their
``slot_mapping``; the caller writes them first and attends afterwards
(the Mistral 3 page, section 3, appends K/V to the cache before attention).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

BF16 = "bf16"
F32 = "f32"

_BF16_QNAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# storage helpers (bit-level representation changes, no arithmetic of the
# method)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  NaN maps to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = _BF16_QNAN
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def storage_to_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Value view of a storage array: bf16 bits or float32 -> float32."""
    if dtype == BF16:
        return bf16_bits_to_f32(arr)
    if dtype == F32:
        return np.asarray(arr, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _nan_value(dtype: str):
    return _BF16_QNAN if dtype == BF16 else np.float32(np.nan)


def _draw_normal(rng: np.random.Generator, shape, dtype: str, chunk_rows: int = 0) -> np.ndarray:
    """Standard-normal draw stored as ``dtype`` (bf16 bits or float32).

    Large pools are drawn in consecutive chunks along axis 0 to bound the
    float32 temporary; the chunking is part of the recipe.
    """
    shape = tuple(int(s) for s in shape)
    out_dt = np.uint16 if dtype == BF16 else np.float32
    out = np.empty(shape, dtype=out_dt)
    n0 = shape[0]
    step = chunk_rows if chunk_rows > 0 else max(n0, 1)
    for s in range(0, n0, step):
        e = min(n0, s + step)
        x = rng.standard_normal(size=(e - s,) + shape[1:], dtype=np.float32)
        out[s:e] = f32_to_bf16_bits(x) if dtype == BF16 else x
    return out


# --------------------------------------------------------------------------
# cases
# --------------------------------------------------------------------------

@dataclasses.dataclass
class _PagedBase:
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    k_cache: np.ndarray          # [NB, BS, Hkv, D] storage, before new tokens
    v_cache: np.ndarray
    new_key: np.ndarray          # [T_new, Hkv, D] storage
    new_value: np.ndarray
    slot_mapping: np.ndarray     # [T_new] int64
    block_tables: np.ndarray     # [S, max_blocks_per_seq] int32
    context_lens: np.ndarray     # [S] int32, including the new tokens
    pad_block: int               # id used to pad block-table rows

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def v_head_dim(self) -> int:
        """Value head dim (the output width); equals head_dim unless the
        case was drawn with a value head dim of its own."""
        return int(self.v_cache.shape[3])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes_logical(self) -> int:
        """K+V bytes a kernel must read: every context token, all kv heads."""
        el = 2 if self.dtype == BF16 else 4
        return (int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads
                * (self.head_dim + self.v_head_dim) * el)

    def unique_blocks(self) -> int:
        used = set()
        bs = self.block_size
        for i, n in enumerate(self.context_lens.tolist()):
            nblk = -(-n // bs)
            used.update(self.block_tables[i, :nblk].tolist())
        return len(used)


@dataclasses.dataclass
class DecodeCase(_PagedBase):
    q: np.ndarray = None         # [S, Hq, D] storage: one query token per sequence


@dataclasses.dataclass
class PrefillCase(_PagedBase):
    q: np.ndarray = None               # [Tq, Hq, D] storage, packed by sequence
    query_start_loc: np.ndarray = None  # [S+1] int32

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        ql = self.query_lens
        return int(ql.max()) if ql.size else 0


# --------------------------------------------------------------------------
# layout: placing sequences in the block pool
# --------------------------------------------------------------------------

def _blocks_for(n: int, bs: int) -> int:
    return -(-int(n) // bs)


def _layout(rng, context_lens, block_size, *, num_blocks=None, pool_factor=1.25,
            shared_blocks=0, group_of=None, extra_table_cols=0):
    """Draw block tables for ``context_lens``.

    ``shared_blocks`` > 0 with ``group_of[i]`` gives every sequence of a group
    the same first ``shared_blocks`` physical blocks (a prefix held once in
    the pool, as a content-hashed prefix cache would share it).  Shared and
    private ids come from one random permutation of the pool, so they
    interleave in id space.

    Returns ``(block_tables, num_blocks, pad_block)``.
    """
    ctx = [int(n) for n in context_lens]
    S = len(ctx)
    need = [_blocks_for(n, block_size) for n in ctx]
    if shared_blocks:
        groups = sorted(set(group_of))
        private = [max(0, need[i] - shared_blocks) for i in range(S)]
        unique = shared_blocks * len(groups) + sum(private)
    else:
        groups = []
        private = need
        unique = sum(need)
    if num_blocks is None:
        # one spare block at least, so a padding id always exists
        num_blocks = max(unique + 1, int(math.ceil(pool_factor * unique)))
    if num_blocks < unique + 1:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {unique} blocks plus a pad block")
    perm = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0
    shared_ids = {}
    for g in groups:
        shared_ids[g] = perm[cursor:cursor + shared_blocks]
        cursor += shared_blocks
    max_blocks = max(need) if need else 1
    max_blocks = max(1, max_blocks) + int(extra_table_cols)
    pad = int(perm[unique])  # never referenced by any sequence
    tables = np.full((S, max_blocks), pad, dtype=np.int32)
    for i in range(S):
        row = []
        if shared_blocks:
            row.extend(shared_ids[group_of[i]][:min(shared_blocks, need[i])].tolist())
        row.extend(perm[cursor:cursor + private[i]].tolist())
        cursor += private[i]
        tables[i, :len(row)] = row
    return tables, int(num_blocks), pad


def _slots_of(table_row, positions, bs):
    positions = np.asarray(positions, dtype=np.int64)
    return table_row[positions // bs].astype(np.int64) * bs + positions % bs


def _finish(rng, *, kind, name, dtype, Hq, Hkv, D, bs, ctx, tables, nb, pad, q_rows,
            new_positions, boost_frac=0.0, boost=8.0, poison=True, chunk_rows=256,
            query_start_loc=None, Dv=None):
    """Draw Q, K, V (in that order), apply the boost mask, split off the new
    tokens and poison what no sequence may read.  ``Dv`` is the value head
    dim (default ``D``)."""
    Dv = D if Dv is None else int(Dv)
    q = _draw_normal(rng, (q_rows, Hq, D), dtype)
    k = _draw_normal(rng, (nb, bs, Hkv, D), dtype, chunk_rows=chunk_rows)
    v = _draw_normal(rng, (nb, bs, Hkv, Dv), dtype, chunk_rows=chunk_rows)
    kflat = k.reshape(nb * bs, Hkv, D)
    vflat = v.reshape(nb * bs, Hkv, Dv)

    if boost_frac > 0.0:
        # iid Bernoulli(boost_frac) per (sequence, position, kv head); the
        # whole D-vector of a chosen key is multiplied by `boost` (a power of
        # two, so exact on bf16 values).  A shared physical row is boosted
        # once however many sequences reference it.
        boosted = np.zeros((nb * bs, Hkv), dtype=bool)
        for i, n in enumerate(ctx):
            m = rng.random((n, Hkv)) < boost_frac
            slots = _slots_of(tables[i], np.arange(n), bs)
            boosted[slots] |= m
        rows, heads = np.nonzero(boosted)
        vals = storage_to_f32(kflat[rows, heads], dtype) * np.float32(boost)
        kflat[rows, heads] = f32_to_bf16_bits(vals) if dtype == BF16 else vals

    # new tokens: their values are the drawn pool values at their slots
    slot_list = []
    for i, pos in enumerate(new_positions):
        slot_list.append(_slots_of(tables[i], pos, bs))
    slot_mapping = np.concatenate(slot_list).astype(np.int64) if slot_list else np.zeros(0, np.int64)
    new_key = kflat[slot_mapping].copy()
    new_value = vflat[slot_mapping].copy()

    if poison:
        referenced = np.zeros(nb * bs, dtype=bool)
        for i, n in enumerate(ctx):
            referenced[_slots_of(tables[i], np.arange(n), bs)] = True
        referenced[slot_mapping] = False  # not valid until written
        nanv = _nan_value(dtype)
        kflat[~referenced] = nanv
        vflat[~referenced] = nanv

    common = dict(name=name, dtype=dtype, num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                  block_size=bs, scale=1.0 / math.sqrt(D), k_cache=k, v_cache=v,
                  new_key=new_key, new_value=new_value, slot_mapping=slot_mapping,
                  block_tables=tables, context_lens=np.asarray(ctx, dtype=np.int32),
                  pad_block=pad, q=q)
    if kind == "decode":
        return DecodeCase(**common)
    return PrefillCase(query_start_loc=query_start_loc, **common)


# --------------------------------------------------------------------------
# generic cases (tests use these at small sizes)
# --------------------------------------------------------------------------

def random_decode(seed: int, context_lens: Sequence[int], *, num_heads=8, num_kv_heads=2,
                  head_dim=64, block_size=16, dtype=F32, num_blocks=None, pool_factor=1.25,
                  shared_blocks=0, group_of=None, boost_frac=0.0, poison=True,
                  extra_table_cols=0, name="decode", v_head_dim=None) -> DecodeCase:
    """One decode token per sequence; ``context_lens`` include that token.
    ``v_head_dim`` (default ``head_dim``) is the value head dim."""
    rng = np.random.default_rng(seed)
    ctx = [int(n) for n in context_lens]
    tables, nb, pad = _layout(rng, ctx, block_size, num_blocks=num_blocks, pool_factor=pool_factor,
                              shared_blocks=shared_blocks, group_of=group_of,
                              extra_table_cols=extra_table_cols)
    new_positions = [np.array([n - 1], dtype=np.int64) if n > 0 else np.zeros(0, np.int64) for n in ctx]
    return _finish(rng, kind="decode", name=name, dtype=dtype, Hq=num_heads, Hkv=num_kv_heads,
                   D=head_dim, bs=block_size, ctx=ctx, tables=tables, nb=nb, pad=pad,
                   q_rows=len(ctx), new_positions=new_positions, boost_frac=boost_frac,
                   poison=poison, Dv=v_head_dim)


def random_prefill(seed: int, prefix_lens: Sequence[int], query_lens: Sequence[int], *,
                   num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, dtype=BF16,
                   num_blocks=None, pool_factor=1.25, poison=True, extra_table_cols=0,
                   name="prefill", v_head_dim=None) -> PrefillCase:
    """A packed chunk of ``query_lens[i]`` new tokens per sequence appended
    after ``prefix_lens[i]`` cached tokens.  ``v_head_dim`` (default
    ``head_dim``) is the value head dim."""
    rng = np.random.default_rng(seed)
    prefix = [int(n) for n in prefix_lens]
    qlen = [int(n) for n in query_lens]
    ctx = [p + t for p, t in zip(prefix, qlen)]
    tables, nb, pad = _layout(rng, ctx, block_size, num_blocks=num_blocks, pool_factor=pool_factor,
                              extra_table_cols=extra_table_cols)
    qsl = np.zeros(len(ctx) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(qlen)
    new_positions = [np.arange(p, p + t, dtype=np.int64) for p, t in zip(prefix, qlen)]
    return _finish(rng, kind="prefill", name=name, dtype=dtype, Hq=num_heads, Hkv=num_kv_heads,
                   D=head_dim, bs=block_size, ctx=ctx, tables=tables, nb=nb, pad=pad,
                   q_rows=int(qsl[-1]), new_positions=new_positions, poison=poison,
                   query_start_loc=qsl, Dv=v_head_dim)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------

def tiny_fp32_decode(seed: int = 1000, poison: bool = True) -> DecodeCase:
    """1 sequence, 8 q / 2 kv heads, head_dim 64, context 100 (99 cached + 1
    new token written through slot_mapping), block_size 16, a pool of 64
    blocks of which the sequence's 7 are a random draw, fp32, scale 1/8."""
    rng = np.random.default_rng(seed)
    ctx = [100]
    tables, nb, pad = _layout(rng, ctx, 16, num_blocks=64)
    return _finish(rng, kind="decode", name="tiny_fp32_decode", dtype=F32, Hq=8, Hkv=2, D=64,
                   bs=16, ctx=ctx, tables=tables, nb=nb, pad=pad, q_rows=1,
                   new_positions=[np.array([99])], poison=poison)


def decode_batch(seed: int = 2000, poison: bool = True, num_seqs: int = 32,
                 ctx_low: int = 512, ctx_high: int = 4096, fixed_ctx: Optional[int] = None,
                 num_heads: int = 32, v_head_dim: Optional[int] = None) -> DecodeCase:
    """32 sequences, 32 q / 8 kv heads, head_dim 128, block_size 32, context
    uniform in [512, 4096], pool 1.25x the blocks in use, bf16.  ``num_heads``
    = 64 gives eight query heads per kv head over the same K/V;
    ``v_head_dim`` a value head dim of its own."""
    rng = np.random.default_rng(seed)
    if fixed_ctx is not None:
        ctx = [int(fixed_ctx)] * num_seqs
    else:
        ctx = rng.integers(ctx_low, ctx_high, size=num_seqs, endpoint=True).tolist()
    tables, nb, pad = _layout(rng, ctx, 32)
    return _finish(rng, kind="decode", name="decode_batch_bs32", dtype=BF16, Hq=num_heads, Hkv=8, D=128,
                   bs=32, ctx=ctx, tables=tables, nb=nb, pad=pad, q_rows=num_seqs,
                   new_positions=[np.array([n - 1]) for n in ctx], poison=poison, Dv=v_head_dim)


def long_context_decode(seed: int = 3000, poison: bool = True, num_seqs: int = 4,
                        ctx_low: int = 32768, ctx_high: int = 131072) -> DecodeCase:
    """4 sequences, 32 q / 8 kv heads, head_dim 128, block_size 32, context
    uniform in [32768, 131072], 1% of keys scaled by 8, bf16."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_low, ctx_high, size=num_seqs, endpoint=True).tolist()
    tables, nb, pad = _layout(rng, ctx, 32)
    return _finish(rng, kind="decode", name="long_context_decode", dtype=BF16, Hq=32, Hkv=8, D=128,
                   bs=32, ctx=ctx, tables=tables, nb=nb, pad=pad, q_rows=num_seqs,
                   new_positions=[np.array([n - 1]) for n in ctx], boost_frac=0.01, poison=poison)


def chunked_prefill(seed: int = 4000, poison: bool = True, num_seqs: int = 8, chunk: int = 512,
                    prefix_high: int = 3584, block_size: int = 32, num_heads: int = 32) -> PrefillCase:
    """8 sequences each appending a 512-token chunk (4096-token budget) onto
    a cached prefix uniform in [0, 3584]; 32 q / 8 kv heads, head_dim 128,
    block_size 32 (8 and 16 as variants), bf16.  The chunk's slot mapping
    follows the randomly drawn block table, continuing the prefix's partial
    last block.  ``num_heads`` = 64 gives eight query heads per kv head."""
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, prefix_high, size=num_seqs, endpoint=True).tolist()
    qlen = [chunk] * num_seqs
    ctx = [p + chunk for p in prefix]
    tables, nb, pad = _layout(rng, ctx, block_size)
    qsl = np.zeros(num_seqs + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(qlen)
    name = "chunked_prefill" if block_size == 32 else f"chunked_prefill_bs{block_size}"
    if num_heads != 32:
        name += f"_{num_heads}q"
    return _finish(rng, kind="prefill", name=name, dtype=BF16, Hq=num_heads, Hkv=8, D=128,
                   bs=block_size, ctx=ctx, tables=tables, nb=nb, pad=pad, q_rows=int(qsl[-1]),
                   new_positions=[np.arange(p, p + chunk) for p in prefix], poison=poison,
                   query_start_loc=qsl)


def prefix_shared_decode(seed: int = 5000, block_size: int = 16, poison: bool = True,
                         groups: int = 4, per_group: int = 16, shared_blocks: int = 64,
                         tail_high: int = 2048) -> DecodeCase:
    """64 sequences in 4 groups of 16; each group shares its first 64
    physical blocks, followed by a private tail uniform in [1, 2048] tokens;
    block_size 8 or 16; 32 q / 8 kv heads, head_dim 128, bf16."""
    rng = np.random.default_rng(seed)
    S = groups * per_group
    tails = rng.integers(1, tail_high, size=S, endpoint=True).tolist()
    ctx = [shared_blocks * block_size + t for t in tails]
    group_of = [i // per_group for i in range(S)]
    tables, nb, pad = _layout(rng, ctx, block_size, shared_blocks=shared_blocks, group_of=group_of)
    return _finish(rng, kind="decode", name=f"prefix_shared_decode_bs{block_size}", dtype=BF16,
                   Hq=32, Hkv=8, D=128, bs=block_size, ctx=ctx, tables=tables, nb=nb, pad=pad,
                   q_rows=S, new_positions=[np.array([n - 1]) for n in ctx], poison=poison)


CONFIG_NAMES = (
    "tiny_fp32_decode",
    "decode_batch_bs32",
    "long_context_decode",
    "chunked_prefill",
    "prefix_shared_decode_bs8",
    "prefix_shared_decode_bs16",
)


def make_config(name: str, seed: Optional[int] = None, poison: bool = True):
    """Build a named workload.  Default seeds are 1000 x the workload number."""
    if name == "tiny_fp32_decode":
        return tiny_fp32_decode(1000 if seed is None else seed, poison=poison)
    if name == "decode_batch_bs32":
        return decode_batch(2000 if seed is None else seed, poison=poison)
    if name == "long_context_decode":
        return long_context_decode(3000 if seed is None else seed, poison=poison)
    if name == "chunked_prefill":
        return chunked_prefill(4000 if seed is None else seed, poison=poison)
    if name == "prefix_shared_decode_bs8":
        return prefix_shared_decode(5000 if seed is None else seed, block_size=8, poison=poison)
    if name == "prefix_shared_decode_bs16":
        return prefix_shared_decode(5000 if seed is None else seed, block_size=16, poison=poison)
    raise KeyError(name)
