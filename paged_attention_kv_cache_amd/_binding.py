"""ctypes binding of ``libpagedattn.so`` (the C ABI in ``include/pagedattn.h``
and ``include/pagedattn_kvm.h``).

Argument marshalling only: tensors in, device pointers and sizes out, the
status code checked.  Every step of the computation runs in the library's
HIP kernels.  torch supplies device memory and the current stream.  If the
library has not been built, the first call raises: there is no fallback
path.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpagedattn.so")

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1

STATUS = {
    0: "PA_OK",
    -1: "PA_ERR_NULL",
    -2: "PA_ERR_DTYPE",
    -3: "PA_ERR_SHAPE",
    -4: "PA_ERR_BLOCK_SIZE",
    -5: "PA_ERR_HEAD_DIM",
    -6: "PA_ERR_GQA",
    -7: "PA_ERR_WORKSPACE",
    -8: "PA_ERR_UNSUPPORTED",
    -9: "PA_ERR_HIP",
    -10: "PA_ERR_PARTITION",
    -11: "PA_ERR_NO_BLOCKS",
    -12: "PA_ERR_REQUEST",
}

# every function the header declares, with its ctypes signature
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


class PaKvCache(ctypes.Structure):
    _fields_ = [
        ("k_cache", _vp),
        ("v_cache", _vp),
        ("num_blocks", _i32),
        ("block_size", _i32),
        ("num_kv_heads", _i32),
        ("head_dim", _i32),
        ("dtype", _i32),
        ("v_head_dim", _i32),
    ]


_PCACHE = ctypes.POINTER(PaKvCache)
_i64 = ctypes.c_int64
_pi32 = ctypes.POINTER(_i32)
_pi64 = ctypes.POINTER(_i64)


class PaKvmStats(ctypes.Structure):
    _fields_ = [(n, _i64) for n in (
        "num_blocks", "block_size", "free_blocks", "cached_blocks", "active_requests",
        "prefix_queries", "prefix_hit_blocks", "prefix_hit_tokens", "evictions")]


class PaSchedConfig(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "max_batched_tokens", "max_chunk_tokens", "max_decode_steps", "min_decode_steps", "max_seqs", "mixed")]


class PaStep(ctypes.Structure):
    _fields_ = [
        ("kind", _i32), ("num_seqs", _i32), ("num_tokens", _i32), ("max_query_len", _i32),
        ("max_context_len", _i32), ("max_blocks_per_seq", _i32),
        ("request_ids", _pi64), ("query_start_loc", _pi32), ("context_lens", _pi32),
        ("block_tables", _pi32), ("slot_mapping", _pi64),
        ("cap_seqs", _i32), ("cap_tokens", _i32), ("cap_blocks", _i32),
    ]

SIGNATURES = {
    "pa_kv_cache_write": (ctypes.c_int, [_PCACHE, _vp, _vp, _vp, _i32, _vp]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (ctypes.c_int, [_PCACHE, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32,
                                 _vp, _sz, _vp]),
    "pa_decode_static": (ctypes.c_int, [_PCACHE, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32, _vp]),
    "pa_decode_partition": (ctypes.c_int, [_PCACHE, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32,
                                           _i32, _vp, _sz, _vp]),
    "pa_decode_reduce": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _sz, _vp]),
    "pa_prefill_chunk": (ctypes.c_int, [_PCACHE, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp,
                                        _i32, _f32, _vp]),
    "pa_kv_cache_copy_blocks": (ctypes.c_int, [_PCACHE, _PCACHE, _vp, _vp, _i32, _vp]),
    "pa_decode_cascade_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_append": (ctypes.c_int, [_PCACHE, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32,
                                        _vp, _sz, _vp]),
    "pa_decode_cascade": (ctypes.c_int, [_PCACHE, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32, _i32, _i32,
                                         _vp, _vp, _i32, _i32, _vp, _sz, _vp]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_error_message": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_int, []),
    "pa_stream_read": (ctypes.c_int, [_vp, _sz, _vp, _vp]),
    "pa_clock_probe": (ctypes.c_int, [_vp, _i64, _vp]),
    "pa_mfma_peak": (ctypes.c_int, [_vp, _i32, _vp]),
    # host KV manager and step scheduler
    "pa_kvm_create": (_vp, [_i32, _i32, _i32]),
    "pa_kvm_destroy": (None, [_vp]),
    "pa_kvm_add_request": (ctypes.c_int, [_vp, _i64, _pi32, _i32]),
    "pa_kvm_append_tokens": (ctypes.c_int, [_vp, _i64, _pi32, _i32]),
    "pa_kvm_get_computed_blocks": (ctypes.c_int, [_vp, _i64, _pi32]),
    "pa_kvm_allocate_slots": (ctypes.c_int, [_vp, _i64, _i32]),
    "pa_kvm_commit": (ctypes.c_int, [_vp, _i64, _i32]),
    "pa_kvm_free": (ctypes.c_int, [_vp, _i64]),
    "pa_kvm_block_table": (ctypes.c_int, [_vp, _i64, _pi32, _i32, _pi32]),
    "pa_kvm_slot_mapping": (ctypes.c_int, [_vp, _i64, _i32, _i32, _pi64]),
    "pa_kvm_request_info": (ctypes.c_int, [_vp, _i64, _pi32, _pi32, _pi32]),
    "pa_kvm_get_stats": (ctypes.c_int, [_vp, ctypes.POINTER(PaKvmStats)]),
    "pa_kvm_grow": (ctypes.c_int, [_vp, _i32]),
    "pa_sched_create": (_vp, [_vp, ctypes.POINTER(PaSchedConfig)]),
    "pa_sched_destroy": (None, [_vp]),
    "pa_sched_add_request": (ctypes.c_int, [_vp, _i64, _pi32, _i32, _i32]),
    "pa_sched_next_step": (ctypes.c_int, [_vp, ctypes.POINTER(PaStep)]),
    "pa_sched_complete_step": (ctypes.c_int, [_vp, ctypes.POINTER(PaStep), _pi32, _pi32]),
    # native serving step (include/pagedattn_serve.h)
    "pa_serve_meta_bytes": (_sz, [_i32, _i32, _i32]),
    "pa_serve_create": (_vp, [_vp, _i32, _f32, _i32, _i32, _i32, _i32, _i32, _vp, _sz]),
    "pa_serve_destroy": (None, [_vp]),
    "pa_serve_plan": (ctypes.c_int, [_vp, ctypes.POINTER(PaStep), _vp]),
    "pa_serve_attend": (ctypes.c_int, [_vp, _PCACHE, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "pa_serve_complete": (ctypes.c_int, [_vp, _pi32, _pi32]),
    "pa_sched_counts": (ctypes.c_int, [_vp, _pi32, _pi32, _pi32]),
}

_lib = None
_lock = threading.Lock()


class PagedAttnError(RuntimeError):
    """A negative status from the library, with its message."""

    def __init__(self, func: str, code: int, message: str):
        self.func = func
        self.code = code
        self.status = STATUS.get(code, f"status {code}")
        self.message = message
        super().__init__(f"{func}: {self.status}: {message}")


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the shared library once and attach the ctypes signatures."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        # PA_LIBRARY names another build of the same library (the host
        # sanitizer build runs the host test suites on it)
        p = path or os.environ.get("PA_LIBRARY") or LIB_PATH
        # torch first: the library needs libamdhip64.so.7, which torch's own
        # HIP runtime provides once torch is imported.  Loaded before torch,
        # the library would bring up a second HIP runtime in the process,
        # and whichever initialises the GPU second finds no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(p):
            raise RuntimeError(
                f"{p} is not built; build it with `python -c \"import __graft_entry__ as g; g.build()\"` "
                "or `python paged_attention_kv_cache_amd/build.py` (there is no fallback path)")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def _check(func: str, code: int) -> None:
    if code != 0:
        msg = load_library().pa_last_error_message()
        raise PagedAttnError(func, code, msg.decode() if msg else "")


# ---------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected torch.float32 or torch.bfloat16")


def _dev(t, name: str, dtype=None, ndim: Optional[int] = None):
    """Device pointer of a contiguous GPU tensor (checks only)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def make_cache(k_cache, v_cache) -> PaKvCache:
    """Descriptor for one layer's pool: K ``[num_blocks, block_size,
    num_kv_heads, head_dim]`` and V ``[num_blocks, block_size, num_kv_heads,
    v_head_dim]`` (the value head dim may differ from the key head dim)."""
    if k_cache.dim() != 4 or v_cache.dim() != 4 or k_cache.shape[:3] != v_cache.shape[:3]:
        raise ValueError(f"k_cache {tuple(k_cache.shape)} and v_cache {tuple(v_cache.shape)} must be 4-d "
                         "shapes that agree in all but the last dim")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache dtypes differ")
    nb, bs, hkv, d = (int(x) for x in k_cache.shape)
    return PaKvCache(_dev(k_cache, "k_cache").value, _dev(v_cache, "v_cache").value, nb, bs, hkv, d,
                     _dtype_code(k_cache), int(v_cache.shape[3]))


# ------------------------------------------------------------ entry points

def pa_version() -> int:
    return int(load_library().pa_version())


def pa_status_string(code: int) -> str:
    return load_library().pa_status_string(code).decode()


def pa_last_error_message() -> str:
    return load_library().pa_last_error_message().decode()


def pa_decode_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                              partition_size: int) -> int:
    return int(load_library().pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                                        partition_size))


def pa_stream_read(buf, sink, stream=None) -> None:
    """Read the whole GPU tensor ``buf`` once (the HBM read-rate probe of
    ``include/pagedattn_bench.h``); ``sink`` is a GPU tensor of at least 4
    bytes."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    code = load_library().pa_stream_read(_dev(buf, "buf"), nbytes, _dev(sink, "sink"), _stream(stream))
    _check("pa_stream_read", code)


def pa_mfma_peak(sink, iters: int, stream=None) -> None:
    """Enqueue the matrix-unit ceiling kernel of ``include/pagedattn_bench.h``
    (``iters`` rounds of four bf16 MFMA chains per wave); ``sink`` is a GPU
    tensor of at least 4 bytes."""
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    code = load_library().pa_mfma_peak(_dev(sink, "sink"), int(iters), _stream(stream))
    _check("pa_mfma_peak", code)


def pa_clock_probe(out, ticks: int, stream=None) -> None:
    """Enqueue the shader-clock probe of ``include/pagedattn_bench.h``:
    ``out`` is a GPU int64 tensor of at least 3 elements that receives
    (shader cycles, 100 MHz reference ticks, sleep steps) over ``ticks``
    reference ticks."""
    if out.numel() * out.element_size() < 24:
        raise ValueError("out must hold at least 3 x 8 bytes")
    code = load_library().pa_clock_probe(_dev(out, "out"), int(ticks), _stream(stream))
    _check("pa_clock_probe", code)


def pa_kv_cache_write(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Scatter ``key [T, Hkv, D]`` / ``value [T, Hkv, Dv]`` into the pool at
    ``slot_mapping`` (int64 [T])."""
    torch = _torch()
    cache = make_cache(k_cache, v_cache)
    if (key.dim() != 3 or value.dim() != 3 or tuple(key.shape[1:]) != tuple(k_cache.shape[2:])
            or tuple(value.shape[1:]) != tuple(v_cache.shape[2:]) or key.shape[0] != value.shape[0]):
        raise ValueError(f"key/value {tuple(key.shape)}/{tuple(value.shape)} must be [T, "
                         f"{k_cache.shape[2]}, {k_cache.shape[3]}] / [T, {v_cache.shape[2]}, {v_cache.shape[3]}]")
    if slot_mapping.shape != (key.shape[0],):
        raise ValueError(f"slot_mapping {tuple(slot_mapping.shape)} must be [{key.shape[0]}]")
    code = load_library().pa_kv_cache_write(
        ctypes.byref(cache), _dev(key, "key", k_cache.dtype), _dev(value, "value", k_cache.dtype),
        _dev(slot_mapping, "slot_mapping", torch.int64), int(key.shape[0]), _stream(stream))
    _check("pa_kv_cache_write", code)


def pa_kv_cache_copy_blocks(src_k, src_v, dst_k, dst_v, src_ids=None, dst_ids=None, num_copies=None,
                            stream=None) -> None:
    """Copy whole blocks between pools (or inside one).  With no ids, blocks
    0 .. num_copies-1 (default: all of the source) go to the same ids."""
    torch = _torch()
    src = make_cache(src_k, src_v)
    dst = make_cache(dst_k, dst_v)
    if (src_ids is None) != (dst_ids is None):
        raise ValueError("give both src_ids and dst_ids, or neither")
    if src_ids is None:
        n = int(src_k.shape[0]) if num_copies is None else int(num_copies)
        ps = pd = ctypes.c_void_p(0)
    else:
        n = int(src_ids.numel())
        if int(dst_ids.numel()) != n:
            raise ValueError("src_ids and dst_ids differ in length")
        ps = _dev(src_ids, "src_ids", torch.int32)
        pd = _dev(dst_ids, "dst_ids", torch.int32)
    code = load_library().pa_kv_cache_copy_blocks(ctypes.byref(src), ctypes.byref(dst), ps, pd, n,
                                                  _stream(stream))
    _check("pa_kv_cache_copy_blocks", code)


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, out):
    torch = _torch()
    cache = make_cache(k_cache, v_cache)
    S, H, D = (int(x) for x in q.shape)
    if D != int(k_cache.shape[3]):
        raise ValueError(f"q head_dim {D} != cache head_dim {k_cache.shape[3]}")
    if block_tables.dim() != 2 or int(block_tables.shape[0]) != S:
        raise ValueError(f"block_tables {tuple(block_tables.shape)} must be [{S}, max_blocks_per_seq]")
    if tuple(context_lens.shape) != (S,):
        raise ValueError(f"context_lens {tuple(context_lens.shape)} must be [{S}]")
    Dv = int(v_cache.shape[3])
    if out is None:
        out = torch.empty((S, H, Dv), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (S, H, Dv) or out.dtype != q.dtype:
        raise ValueError(f"out must be [{S}, {H}, {Dv}] of q's dtype")
    ptrs = (_dev(out, "out", k_cache.dtype, 3), _dev(q, "q", k_cache.dtype, 3),
            _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32))
    return cache, S, H, Dv, out, ptrs


def _on_stream(tensor, stream) -> None:
    """A tensor allocated here and handed to kernels enqueued on ``stream``
    (not torch's current stream) is recorded on that stream, so the caching
    allocator does not reuse its memory before those kernels finish."""
    if stream is None:
        return
    torch = _torch()
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
        stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    if s != torch.cuda.current_stream():
        tensor.record_stream(s)


def _workspace(workspace, need: int, device, stream=None):
    torch = _torch()
    if need == 0:
        return ctypes.c_void_p(0), 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
        _on_stream(workspace, stream)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    return ctypes.c_void_p(workspace.data_ptr()), nbytes


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, max_context_len: int,
              partition_size: int = 512, out=None, workspace=None, stream=None, _stage: str = "both"):
    """Paged decode: ``q [S, H, D]`` -> ``out [S, H, Dv]``.

    ``partition_size`` 0 runs one pass per (sequence, kv head); otherwise
    split-K partitions of that many tokens plus the reduce kernel.
    ``workspace`` (uint8 GPU tensor) is allocated here when not given.
    """
    cache, S, H, Dv, out, (p_out, p_q, p_bt, p_cl) = _decode_args(q, k_cache, v_cache, block_tables,
                                                                 context_lens, out)
    lib = load_library()
    need = int(lib.pa_decode_workspace_bytes(S, H, Dv, int(max_context_len), int(partition_size)))
    p_ws, ws_bytes = _workspace(workspace, need, q.device, stream)
    st = _stream(stream)
    mbps = int(block_tables.shape[1])
    if _stage in ("both", "partition"):
        fn = lib.pa_decode if _stage == "both" else lib.pa_decode_partition
        code = fn(ctypes.byref(cache), p_out, p_q, S, H, p_bt, mbps, p_cl, int(max_context_len),
                  float(scale), int(partition_size), p_ws, ws_bytes, st)
        _check("pa_decode" if _stage == "both" else "pa_decode_partition", code)
    if _stage == "reduce":
        code = lib.pa_decode_reduce(p_out, cache.dtype, S, H, Dv, p_cl, int(max_context_len),
                                    int(partition_size), p_ws, ws_bytes, st)
        _check("pa_decode_reduce", code)
    return out


def pa_decode_static(q, k_cache, v_cache, block_tables, context_lens, scale: float, max_context_len: int,
                     partition_size: int = 512, out=None, stream=None):
    """:func:`pa_decode` whose split-K partials live in the library's static
    device scratch: nothing is allocated for them (``out`` is still
    allocated here when not given)."""
    cache, S, H, Dv, out, (p_out, p_q, p_bt, p_cl) = _decode_args(q, k_cache, v_cache, block_tables,
                                                                 context_lens, out)
    code = load_library().pa_decode_static(ctypes.byref(cache), p_out, p_q, S, H, p_bt, int(block_tables.shape[1]),
                                           p_cl, int(max_context_len), float(scale), int(partition_size),
                                           _stream(stream))
    _check("pa_decode_static", code)
    return out


def pa_decode_append(q, key, value, k_cache, v_cache, block_tables, context_lens, scale: float,
                     max_context_len: int, partition_size: int = 512, out=None, workspace=None, stream=None):
    """One decode step: writes ``key [S, Hkv, D]`` / ``value [S, Hkv, Dv]``
    (the newest token of each sequence, position ``context_lens[i] - 1``)
    into the cache and attends: ``q [S, H, D]`` -> ``out [S, H, Dv]``."""
    cache, S, H, Dv, out, (p_out, p_q, p_bt, p_cl) = _decode_args(q, k_cache, v_cache, block_tables,
                                                                  context_lens, out)
    if (key.dim() != 3 or value.dim() != 3 or tuple(key.shape) != (S,) + tuple(k_cache.shape[2:])
            or tuple(value.shape) != (S,) + tuple(v_cache.shape[2:])):
        raise ValueError(f"key/value {tuple(key.shape)}/{tuple(value.shape)} must be [{S}, {k_cache.shape[2]}, "
                         f"{k_cache.shape[3]}] / [{S}, {v_cache.shape[2]}, {v_cache.shape[3]}]")
    lib = load_library()
    need = int(lib.pa_decode_workspace_bytes(S, H, Dv, int(max_context_len), int(partition_size)))
    p_ws, ws_bytes = _workspace(workspace, need, q.device, stream)
    code = lib.pa_decode_append(ctypes.byref(cache), p_out, p_q, _dev(key, "key", k_cache.dtype),
                                _dev(value, "value", k_cache.dtype), S, H, p_bt, int(block_tables.shape[1]), p_cl,
                                int(max_context_len), float(scale), int(partition_size), p_ws, ws_bytes,
                                _stream(stream))
    _check("pa_decode_append", code)
    return out


def pa_decode_partition(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                        partition_size, out, workspace, stream=None):
    """First stage of :func:`pa_decode` (same arguments; ``out`` and
    ``workspace`` must be given)."""
    return pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                     partition_size, out=out, workspace=workspace, stream=stream, _stage="partition")


def pa_decode_reduce(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                     partition_size, out, workspace, stream=None):
    """Second stage of :func:`pa_decode` (same arguments as the first)."""
    return pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                     partition_size, out=out, workspace=workspace, stream=stream, _stage="reduce")


def pa_decode_cascade_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                                      partition_size: int) -> int:
    return int(load_library().pa_decode_cascade_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                                                partition_size))


def pa_decode_cascade(q, k_cache, v_cache, block_tables, context_lens, scale: float, max_context_len: int,
                      group_start, shared_len, max_group_size: int, partition_size: int = 256, out=None,
                      workspace=None, stream=None, max_shared_len: Optional[int] = None):
    """Decode of groups that share a prefix of whole blocks: the shared
    tokens are read once per group (``group_start [G+1]``, ``shared_len
    [G]`` int32 GPU tensors; ``max_group_size`` and ``max_shared_len`` host
    ints, the latter defaulting to ``max_context_len``)."""
    torch = _torch()
    cache, S, H, Dv, out, (p_out, p_q, p_bt, p_cl) = _decode_args(q, k_cache, v_cache, block_tables,
                                                                 context_lens, out)
    G = int(shared_len.numel())
    if tuple(group_start.shape) != (G + 1,):
        raise ValueError(f"group_start {tuple(group_start.shape)} must be [{G + 1}]")
    lib = load_library()
    need = int(lib.pa_decode_cascade_workspace_bytes(S, H, Dv, int(max_context_len), int(partition_size)))
    p_ws, ws_bytes = _workspace(workspace, need, q.device, stream)
    code = lib.pa_decode_cascade(ctypes.byref(cache), p_out, p_q, S, H, p_bt, int(block_tables.shape[1]), p_cl,
                                 int(max_context_len), float(scale), int(partition_size), G,
                                 _dev(group_start, "group_start", torch.int32),
                                 _dev(shared_len, "shared_len", torch.int32), int(max_group_size),
                                 int(max_context_len if max_shared_len is None else max_shared_len), p_ws,
                                 ws_bytes, _stream(stream))
    _check("pa_decode_cascade", code)
    return out


def pa_prefill_chunk(q, query_start_loc, k_cache, v_cache, block_tables, context_lens, scale: float,
                     max_query_len: int, max_context_len: int, out=None, stream=None):
    """Chunked prefill: packed ``q [Tq, H, D]`` -> ``out [Tq, H, Dv]``."""
    torch = _torch()
    cache = make_cache(k_cache, v_cache)
    Tq, H, D = (int(x) for x in q.shape)
    S = int(context_lens.shape[0])
    if tuple(query_start_loc.shape) != (S + 1,):
        raise ValueError(f"query_start_loc {tuple(query_start_loc.shape)} must be [{S + 1}]")
    if block_tables.dim() != 2 or int(block_tables.shape[0]) != S:
        raise ValueError(f"block_tables {tuple(block_tables.shape)} must be [{S}, max_blocks_per_seq]")
    if D != int(k_cache.shape[3]):
        raise ValueError(f"q head_dim {D} != cache head_dim {k_cache.shape[3]}")
    Dv = int(v_cache.shape[3])
    if out is None:
        out = torch.empty((Tq, H, Dv), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (Tq, H, Dv) or out.dtype != q.dtype:
        raise ValueError(f"out must be [{Tq}, {H}, {Dv}] of q's dtype")
    code = load_library().pa_prefill_chunk(
        ctypes.byref(cache), _dev(out, "out", k_cache.dtype, 3), _dev(q, "q", k_cache.dtype, 3),
        _dev(query_start_loc, "query_start_loc", torch.int32), S, H, Tq, int(max_query_len),
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), float(scale),
        _stream(stream))
    _check("pa_prefill_chunk", code)
    return out
