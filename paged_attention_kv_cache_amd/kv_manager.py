"""Binding of the host KV block manager and step scheduler
(``include/pagedattn_kvm.h``): argument marshalling over numpy host arrays.

``KvManager`` hands out block ids of a pool the caller allocates on the
device; ``StepScheduler`` plans alternating prompt / decode steps whose
``block_tables``, ``context_lens``, ``query_start_loc`` and
``slot_mapping`` feed ``pa_prefill_chunk`` / ``pa_decode`` /
``pa_kv_cache_write`` directly; ``Server`` (``include/pagedattn_serve.h``)
runs a step's planning, copy and launches inside the library.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from ._binding import PaKvmStats, PaSchedConfig, PaStep, _check, load_library

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _tokens(token_ids: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(token_ids, dtype=np.int32).reshape(-1))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_i32p)


def _p64(a: np.ndarray):
    return a.ctypes.data_as(_i64p)


class KvManager:
    """Block pool with an LRU free list and block-hash prefix caching."""

    def __init__(self, num_blocks: int, block_size: int, enable_prefix_cache: bool = True):
        self._lib = load_library()
        h = self._lib.pa_kvm_create(num_blocks, block_size, 1 if enable_prefix_cache else 0)
        if not h:
            _check("pa_kvm_create", -3 if block_size in (8, 16, 32) else -4)
        self._h = ctypes.c_void_p(h)
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_kvm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def add_request(self, request_id: int, token_ids: Sequence[int]) -> None:
        t = _tokens(token_ids)
        _check("pa_kvm_add_request", self._lib.pa_kvm_add_request(self._h, request_id, _p32(t), t.size))

    def append_tokens(self, request_id: int, token_ids: Sequence[int]) -> None:
        t = _tokens(token_ids)
        _check("pa_kvm_append_tokens", self._lib.pa_kvm_append_tokens(self._h, request_id, _p32(t), t.size))

    def get_computed_blocks(self, request_id: int) -> int:
        n = ctypes.c_int32(0)
        _check("pa_kvm_get_computed_blocks",
               self._lib.pa_kvm_get_computed_blocks(self._h, request_id, ctypes.byref(n)))
        return n.value

    def allocate_slots(self, request_id: int, num_new_tokens: int) -> None:
        _check("pa_kvm_allocate_slots", self._lib.pa_kvm_allocate_slots(self._h, request_id, num_new_tokens))

    def commit(self, request_id: int, num_tokens: int) -> None:
        _check("pa_kvm_commit", self._lib.pa_kvm_commit(self._h, request_id, num_tokens))

    def free(self, request_id: int) -> None:
        _check("pa_kvm_free", self._lib.pa_kvm_free(self._h, request_id))

    def block_table(self, request_id: int) -> np.ndarray:
        n = ctypes.c_int32(0)
        _check("pa_kvm_block_table", self._lib.pa_kvm_block_table(self._h, request_id, None, 0, ctypes.byref(n)))
        out = np.zeros(n.value, dtype=np.int32)
        _check("pa_kvm_block_table",
               self._lib.pa_kvm_block_table(self._h, request_id, _p32(out), out.size, ctypes.byref(n)))
        return out

    def slot_mapping(self, request_id: int, first_pos: int, count: int) -> np.ndarray:
        out = np.zeros(count, dtype=np.int64)
        _check("pa_kvm_slot_mapping",
               self._lib.pa_kvm_slot_mapping(self._h, request_id, first_pos, count, _p64(out)))
        return out

    def request_info(self, request_id: int) -> tuple[int, int, int]:
        """(tokens, computed tokens, blocks) of a request."""
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_kvm_request_info", self._lib.pa_kvm_request_info(
            self._h, request_id, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
        return a.value, b.value, c.value

    def grow(self, new_num_blocks: int) -> None:
        """Extend the pool to new_num_blocks (after the device pool moved)."""
        _check("pa_kvm_grow", self._lib.pa_kvm_grow(self._h, new_num_blocks))
        self.num_blocks = new_num_blocks

    def stats(self) -> dict:
        s = PaKvmStats()
        _check("pa_kvm_get_stats", self._lib.pa_kvm_get_stats(self._h, ctypes.byref(s)))
        return {name: getattr(s, name) for name, _ in PaKvmStats._fields_}


@dataclass
class Step:
    """One planned step (views into the scheduler's host arrays)."""

    kind: int                      # 0 idle, 1 prompt, 2 decode, 3 mixed (decode rows, then prompt chunks)
    request_ids: np.ndarray        # [num_seqs] int64
    query_start_loc: np.ndarray    # [num_seqs + 1] int32
    context_lens: np.ndarray       # [num_seqs] int32
    block_tables: np.ndarray       # [num_seqs, max_blocks_per_seq] int32
    slot_mapping: np.ndarray       # [num_tokens] int64
    max_query_len: int
    max_context_len: int

    @property
    def num_seqs(self) -> int:
        return int(self.request_ids.size)

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.size)


KIND_IDLE, KIND_PROMPT, KIND_DECODE, KIND_MIXED = 0, 1, 2, 3


class StepScheduler:
    """Step planner over a KvManager: alternating all-prompt / all-decode
    steps, or with ``mixed`` one batch per step (every decoding sequence's
    token, then prompt chunks in the rest of the token budget)."""

    def __init__(self, kvm: KvManager, max_batched_tokens: int = 4096, max_chunk_tokens: int = 512,
                 max_decode_steps: int = 8, min_decode_steps: int = 1, max_seqs: int = 256,
                 max_blocks_per_seq: int = 512, mixed: bool = False):
        self._lib = load_library()
        self.kvm = kvm
        cfg = PaSchedConfig(max_batched_tokens, max_chunk_tokens, max_decode_steps, min_decode_steps, max_seqs,
                            1 if mixed else 0)
        h = self._lib.pa_sched_create(kvm.handle, ctypes.byref(cfg))
        if not h:
            _check("pa_sched_create", -3)
        self._h = ctypes.c_void_p(h)
        cap_tokens = max(max_batched_tokens, max_seqs)
        self._ids = np.zeros(max_seqs, dtype=np.int64)
        self._qsl = np.zeros(max_seqs + 1, dtype=np.int32)
        self._ctx = np.zeros(max_seqs, dtype=np.int32)
        self._tab = np.zeros((max_seqs, max_blocks_per_seq), dtype=np.int32)
        self._slots = np.zeros(cap_tokens, dtype=np.int64)
        self._step = PaStep(0, 0, 0, 0, 0, 0, _p64(self._ids), _p32(self._qsl), _p32(self._ctx),
                            _p32(self._tab), _p64(self._slots), max_seqs, cap_tokens, max_blocks_per_seq)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_request(self, request_id: int, prompt: Sequence[int], max_new_tokens: int) -> None:
        t = _tokens(prompt)
        _check("pa_sched_add_request",
               self._lib.pa_sched_add_request(self._h, request_id, _p32(t), t.size, max_new_tokens))

    def next_step(self) -> Step:
        _check("pa_sched_next_step", self._lib.pa_sched_next_step(self._h, ctypes.byref(self._step)))
        st = self._step
        n, t = st.num_seqs, st.num_tokens
        return Step(st.kind, self._ids[:n], self._qsl[:n + 1], self._ctx[:n], self._tab[:n],
                    self._slots[:t], st.max_query_len, st.max_context_len)

    def complete_step(self, sampled: Optional[Sequence[int]] = None) -> int:
        """Commit the last planned step; returns how many requests finished."""
        fin = ctypes.c_int32(0)
        s = None if sampled is None else _tokens(sampled)
        if s is not None and s.size < self._step.num_seqs:
            raise ValueError(f"{s.size} sampled tokens for {self._step.num_seqs} sequences")
        _check("pa_sched_complete_step", self._lib.pa_sched_complete_step(
            self._h, ctypes.byref(self._step), None if s is None else _p32(s), ctypes.byref(fin)))
        return fin.value

    def counts(self) -> tuple[int, int, int]:
        """(waiting, admitted, finished) request counts."""
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_sched_counts", self._lib.pa_sched_counts(self._h, ctypes.byref(a), ctypes.byref(b),
                                                             ctypes.byref(c)))
        return a.value, b.value, c.value


class Server:
    """The native serving step of ``include/pagedattn_serve.h`` over a
    StepScheduler: ``plan`` (the scheduler plans into pinned host memory and
    the step's arrays are copied to the device), ``attend`` (the step's K/V
    write and attention launches) and ``complete`` (commit with sampled
    tokens), each one library call.  The device buffer for the step's arrays
    is allocated here; ``plan`` and ``attend`` of one step take the same
    stream.  With ``mixed_split_context`` > 0 a mixed step whose longest
    decode row reaches that many tokens of context, and is longer than every
    chunk's context, runs its decode rows through split-K decode (0, the
    default: every mixed step in one prefill launch)."""

    def __init__(self, sched: StepScheduler, num_heads: int, scale: float, partition_size: int, max_seqs: int,
                 max_blocks_per_seq: int, max_tokens: int, mixed_split_context: int = 0, device="cuda"):
        import torch
        self._lib = load_library()
        self.sched = sched
        nbytes = int(self._lib.pa_serve_meta_bytes(max_seqs, max_blocks_per_seq, max_tokens))
        if nbytes == 0:
            raise ValueError(f"capacities must be positive: {max_seqs} seqs, {max_blocks_per_seq} blocks, "
                             f"{max_tokens} tokens")
        self._meta = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = self._lib.pa_serve_create(sched._h, num_heads, float(scale), partition_size, mixed_split_context,
                                      max_seqs, max_blocks_per_seq, max_tokens, self._meta.data_ptr(), nbytes)
        if not h:
            _check("pa_serve_create", -3)
        self._h = ctypes.c_void_p(h)
        self._step = PaStep()
        self._caps = (max_seqs, max_blocks_per_seq, max_tokens)
        self._views = {}  # staging buffer (by address of its request ids) -> numpy views over it

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_serve_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _arrays(self, st):
        key = ctypes.cast(st.request_ids, ctypes.c_void_p).value
        v = self._views.get(key)
        if v is None:
            S, B, T = self._caps
            v = (np.ctypeslib.as_array(st.request_ids, shape=(S,)),
                 np.ctypeslib.as_array(st.query_start_loc, shape=(S + 1,)),
                 np.ctypeslib.as_array(st.context_lens, shape=(S,)),
                 np.ctypeslib.as_array(st.block_tables, shape=(S * B,)).reshape(S, B),
                 np.ctypeslib.as_array(st.slot_mapping, shape=(T,)))
            self._views[key] = v
        return v

    def plan(self, stream=None) -> Step:
        """Plan the next step; its arrays are views into pinned staging memory,
        valid until the plan after the next."""
        from ._binding import _stream
        _check("pa_serve_plan", self._lib.pa_serve_plan(self._h, ctypes.byref(self._step), _stream(stream)))
        st = self._step
        n, t = st.num_seqs, st.num_tokens
        if st.kind == KIND_IDLE:
            e = np.zeros(0, np.int64)
            return Step(KIND_IDLE, e, np.zeros(1, np.int32), np.zeros(0, np.int32),
                        np.zeros((0, self._caps[1]), np.int32), e, 0, 0)
        ids, qsl, ctx, tab, slots = self._arrays(st)
        return Step(st.kind, ids[:n], qsl[:n + 1], ctx[:n], tab[:n], slots[:t], st.max_query_len,
                    st.max_context_len)

    def attend(self, k_cache, v_cache, new_key, new_value, q, out, workspace=None, stream=None) -> None:
        """The planned step's K/V write and attention (GPU tensors: the pool,
        the step's new K/V rows, its q rows and the output rows)."""
        from ._binding import _stream, make_cache
        cache = make_cache(k_cache, v_cache)
        ws = 0 if workspace is None else workspace.data_ptr()
        wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check("pa_serve_attend", self._lib.pa_serve_attend(
            self._h, ctypes.byref(cache), new_key.data_ptr(), new_value.data_ptr(), q.data_ptr(), out.data_ptr(),
            ws, wsb, _stream(stream)))

    def complete(self, sampled: Optional[Sequence[int]] = None) -> int:
        """Commit the planned step; returns how many requests finished."""
        fin = ctypes.c_int32(0)
        s = None if sampled is None else _tokens(sampled)
        if s is not None and s.size < self._step.num_seqs:
            raise ValueError(f"{s.size} sampled tokens for {self._step.num_seqs} sequences")
        _check("pa_serve_complete", self._lib.pa_serve_complete(self._h, None if s is None else _p32(s),
                                                                ctypes.byref(fin)))
        return fin.value


def grow_pool(kvm: KvManager, k_cache, v_cache, new_num_blocks: int):
    """Move a device pool (``[num_blocks, block_size, num_kv_heads,
    head_dim]`` K and V tensors) into an allocation of ``new_num_blocks``
    blocks with the library's block copy, and extend the manager to match.
    Returns the new (K, V) tensors."""
    import torch
    from ._binding import pa_kv_cache_copy_blocks
    old = int(k_cache.shape[0])
    if new_num_blocks < old:
        raise ValueError(f"a pool only grows ({old} -> {new_num_blocks})")
    shape = (new_num_blocks,) + tuple(k_cache.shape[1:])
    nk = torch.empty(shape, dtype=k_cache.dtype, device=k_cache.device)
    nv = torch.empty(shape, dtype=v_cache.dtype, device=v_cache.device)
    pa_kv_cache_copy_blocks(k_cache, v_cache, nk, nv, num_copies=old)
    kvm.grow(new_num_blocks)
    return nk, nv
