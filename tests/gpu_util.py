"""Helpers for GPU parity tests: move workload arrays to the device, run the
library, bring results back, and compare with the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads as W

# tolerances for floating-point parity
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3


def torch():
    import torch as _t
    return _t


def log(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a run that dies
    still says what it was doing."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(arr: np.ndarray, dtype: str):
    t = torch()
    if dtype == W.BF16:
        host = t.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(t.bfloat16)
    elif arr.dtype == np.float32:
        host = t.from_numpy(np.ascontiguousarray(arr))
    else:
        host = t.from_numpy(np.ascontiguousarray(arr))
    return host.to("cuda")


def to_host_bits(tensor) -> np.ndarray:
    t = torch()
    x = tensor.detach().cpu()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).numpy().view(np.uint16)
    return x.numpy()


def to_host_f32(tensor, dtype: str) -> np.ndarray:
    return W.storage_to_f32(to_host_bits(tensor), dtype)


def oracle_caches(case):
    """The oracle's own write of the new tokens into the pre-write caches,
    widened to float32 values."""
    k, v = oracle.kv_cache_write(case.k_cache, case.v_cache, case.new_key, case.new_value,
                                 case.slot_mapping)
    return W.storage_to_f32(k, case.dtype), W.storage_to_f32(v, case.dtype)


def oracle_decode(case, seqs=None):
    kf, vf = oracle_caches(case)
    q = W.storage_to_f32(case.q, case.dtype)
    return oracle.paged_decode(q, kf, vf, case.block_tables, case.context_lens, case.scale, seqs=seqs)


def oracle_prefill(case, seqs=None):
    kf, vf = oracle_caches(case)
    q = W.storage_to_f32(case.q, case.dtype)
    return oracle.paged_prefill(q, case.query_start_loc, kf, vf, case.block_tables, case.context_lens,
                                case.scale, seqs=seqs)


class DeviceCase:
    """A workload's arrays on the GPU (pre-write caches)."""

    def __init__(self, case):
        t = torch()
        self.case = case
        d = case.dtype
        self.k_cache = to_dev(case.k_cache, d)
        self.v_cache = to_dev(case.v_cache, d)
        self.new_key = to_dev(case.new_key, d)
        self.new_value = to_dev(case.new_value, d)
        self.slot_mapping = t.from_numpy(case.slot_mapping.astype(np.int64)).cuda()
        self.block_tables = t.from_numpy(case.block_tables.astype(np.int32)).cuda()
        self.context_lens = t.from_numpy(case.context_lens.astype(np.int32)).cuda()
        self.q = to_dev(case.q, d)
        if hasattr(case, "query_start_loc") and case.query_start_loc is not None:
            self.query_start_loc = t.from_numpy(case.query_start_loc.astype(np.int32)).cuda()

    def write(self):
        import paged_attention_kv_cache_amd as P
        P.pa_kv_cache_write(self.new_key, self.new_value, self.k_cache, self.v_cache, self.slot_mapping)

    def decode(self, partition_size, max_context_len=None, out=None, workspace=None):
        import paged_attention_kv_cache_amd as P
        c = self.case
        mcl = c.max_context_len if max_context_len is None else max_context_len
        return P.pa_decode(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                           c.scale, mcl, partition_size, out=out, workspace=workspace)

    def prefill(self, max_context_len=None, out=None):
        import paged_attention_kv_cache_amd as P
        c = self.case
        mcl = c.max_context_len if max_context_len is None else max_context_len
        return P.pa_prefill_chunk(self.q, self.query_start_loc, self.k_cache, self.v_cache,
                                  self.block_tables, self.context_lens, c.scale, c.max_query_len, mcl,
                                  out=out)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output at {np.argwhere(~np.isfinite(got))[:5]}"
    err = np.abs(got - ref)
    if dtype == W.F32:
        assert err.max() <= F32_MAX_ABS, f"{what}: max-abs {err.max():.3e} > {F32_MAX_ABS}"
    else:
        assert err.max() <= BF16_MAX_ABS, f"{what}: max-abs {err.max():.3e} > {BF16_MAX_ABS}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean-abs {err.mean():.3e} > {BF16_MEAN_ABS}"
    return float(err.max()), float(err.mean())
