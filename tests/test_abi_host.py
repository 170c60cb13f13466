"""The C ABI on the host (no GPU): the shared library loads, exports every
function the header declares, and rejects bad arguments with the documented
status codes and messages before anything is enqueued.  Every call here
fails validation, so no HIP work is ever issued."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import paged_attention_kv_cache_amd as P
from paged_attention_kv_cache_amd import _binding
from paged_attention_kv_cache_amd.contracts import (ContractError, check_decode_contracts,
                                                    check_prefill_contracts, check_slot_mapping)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(P.LIB_PATH):
        from paged_attention_kv_cache_amd import build
        build.build()
    return P.load_library()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ("pa_kv_cache_write", "pa_decode", "pa_decode_partition", "pa_decode_reduce",
              "pa_decode_workspace_bytes", "pa_prefill_chunk", "pa_status_string",
              "pa_last_error_message", "pa_version", "pa_kvm_create", "pa_kvm_get_computed_blocks",
              "pa_kvm_allocate_slots", "pa_kvm_free", "pa_sched_next_step", "pa_sched_complete_step"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(pa_[a-z0-9_]+)\b", out))
    for name in declared_functions():
        assert name in exported, f"{name} declared in include/ but not exported"
        assert hasattr(lib, name)
    # the binding knows every declared function and no other
    assert set(_binding.SIGNATURES) == set(declared_functions())


def test_version_and_status_strings(lib):
    assert P.pa_version() == 10100
    for code, name in _binding.STATUS.items():
        assert P.pa_status_string(code) == name
    assert P.pa_status_string(-99) == "PA_UNKNOWN_STATUS"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def cache(nb=10, bs=32, hkv=8, d=128, dtype=1, k=FAKE, v=FAKE, dv=0):
    return _binding.PaKvCache(k, v, nb, bs, hkv, d, dtype, dv)


def decode(lib, c, S=4, H=32, mbps=8, mcl=100, scale=0.1, ps=0, ws=None, ws_bytes=0, out=FAKE, q=FAKE,
           bt=FAKE, cl=FAKE):
    return lib.pa_decode(ctypes.byref(c), out, q, S, H, bt, mbps, cl, mcl, scale, ps, ws, ws_bytes, None)


def msg():
    return P.pa_last_error_message()


@pytest.mark.parametrize("bs", [0, 4, 24, 64, 12])
def test_decode_rejects_block_size(lib, bs):
    assert decode(lib, cache(bs=bs)) == -4
    assert f"block_size {bs}" in msg()


@pytest.mark.parametrize("d", [32, 96, 256])
def test_decode_rejects_head_dim(lib, d):
    assert decode(lib, cache(d=d)) == -5
    assert f"head_dim {d} not in {{64, 128}}" in msg()


def test_decode_rejects_gqa(lib):
    assert decode(lib, cache(hkv=8), H=30) == -6
    assert "not a multiple" in msg()
    assert decode(lib, cache(hkv=2), H=32) == -6          # group of 16
    assert "not in {1, 2, 4, 8}" in msg()


def test_decode_rejects_dtype_and_nulls(lib):
    assert decode(lib, cache(dtype=7)) == -2
    assert "dtype 7" in msg()
    assert decode(lib, cache(k=0)) == -1
    assert lib.pa_decode(None, FAKE, FAKE, 1, 32, FAKE, 8, FAKE, 100, 0.1, 0, None, 0, None) == -1
    assert decode(lib, cache(), q=0) == -1
    assert "all must be device pointers" in msg()


def test_decode_rejects_partition_and_workspace(lib):
    assert decode(lib, cache(), ps=48) == -10
    assert "partition_size 48" in msg()
    assert decode(lib, cache(), ps=-32) == -10
    need = P.pa_decode_workspace_bytes(4, 32, 128, 1000, 256)
    assert decode(lib, cache(), mcl=1000, ps=256) == -7
    assert f"{need} bytes needed" in msg()
    assert decode(lib, cache(), mcl=1000, ps=256, ws=FAKE, ws_bytes=need - 1) == -7
    assert f"< {need} needed" in msg()


def test_static_decode_rejects_partials_above_the_scratch(lib):
    """pa_decode_static refuses, on the host and before any HIP call, a
    request whose split-K partials exceed its static scratch."""
    need = P.pa_decode_workspace_bytes(64, 64, 128, 1 << 20, 32)
    assert need > 32 << 20
    c = cache(hkv=8)
    code = lib.pa_decode_static(ctypes.byref(c), FAKE, FAKE, 64, 64, FAKE, 1 << 15, FAKE, 1 << 20, 0.1, 32, None)
    assert code == -7
    assert f"need {need} bytes" in msg() and str(32 << 20) in msg()
    assert lib.pa_decode_static(ctypes.byref(cache(bs=24)), FAKE, FAKE, 4, 32, FAKE, 8, FAKE, 100, 0.1, 0,
                                None) == -4


def test_decode_rejects_shapes(lib):
    assert decode(lib, cache(), S=-1) == -3
    assert decode(lib, cache(), S=70000) == -3
    assert decode(lib, cache(), mbps=0) == -3
    assert decode(lib, cache(), mcl=-5) == -3
    assert decode(lib, cache(), scale=float("nan")) == -3
    assert decode(lib, cache(nb=0)) == -3


def test_workspace_formula(lib):
    def expect(S, H, D, mcl, ps):
        if ps <= 0 or mcl <= ps:
            return 0
        Pn = -(-mcl // ps)
        n = S * H * Pn
        a = lambda x: (x + 255) // 256 * 256
        return 2 * a(4 * n) + a(4 * n * D)
    for args in [(32, 32, 128, 4096, 256), (4, 32, 128, 131072, 512), (1, 8, 64, 100, 16),
                 (3, 8, 64, 100, 0), (3, 8, 64, 100, 100), (3, 8, 64, 101, 100)]:
        assert P.pa_decode_workspace_bytes(*args) == expect(*args), args
    assert P.pa_decode_workspace_bytes(-1, 32, 128, 4096, 256) == 0


def test_reduce_validation(lib):
    assert lib.pa_decode_reduce(FAKE, 3, 4, 32, 128, FAKE, 1000, 256, FAKE, 10 ** 9, None) == -2
    assert lib.pa_decode_reduce(FAKE, 1, 4, 32, 96, FAKE, 1000, 256, FAKE, 10 ** 9, None) == -5
    assert lib.pa_decode_reduce(FAKE, 1, 4, 32, 128, FAKE, 1000, 256, None, 0, None) == -7
    assert lib.pa_decode_reduce(FAKE, 1, 4, 32, 128, FAKE, 1000, 256, FAKE, 16, None) == -7
    # nothing to merge: a single partition, or no sequences
    assert lib.pa_decode_reduce(FAKE, 1, 4, 32, 128, FAKE, 100, 256, None, 0, None) == 0
    assert lib.pa_decode_reduce(None, 1, 0, 32, 128, None, 1000, 256, None, 0, None) == 0


def test_kv_cache_write_validation(lib):
    c = cache()
    assert lib.pa_kv_cache_write(ctypes.byref(c), FAKE, FAKE, FAKE, -1, None) == -3
    assert lib.pa_kv_cache_write(ctypes.byref(c), None, FAKE, FAKE, 5, None) == -1
    assert lib.pa_kv_cache_write(ctypes.byref(c), FAKE, FAKE, FAKE, 0, None) == 0   # nothing to do
    odd = cache(hkv=1, d=6)                                                            # 12-byte rows
    assert lib.pa_kv_cache_write(ctypes.byref(odd), FAKE, FAKE, FAKE, 5, None) == -3
    assert "multiple of 16" in msg()
    # write takes any block size (only attention restricts it)
    assert lib.pa_kv_cache_write(ctypes.byref(cache(bs=24)), FAKE, FAKE, FAKE, 0, None) == 0


def test_prefill_validation(lib):
    c = cache()
    args = lambda cc, **kw: (ctypes.byref(cc), kw.get("out", FAKE), FAKE, FAKE, kw.get("S", 2), kw.get("H", 32),
                             kw.get("T", 64), kw.get("mql", 32), FAKE, 8, FAKE, 100, kw.get("scale", 0.1), None)
    # fp32 runs a row per query token: at most 65535 rows (checked before any launch)
    assert lib.pa_prefill_chunk(*args(cache(dtype=0), T=70000)) == -8
    assert "at most 65535 query rows" in msg()
    assert lib.pa_prefill_chunk(*args(cache(bs=24))) == -4
    assert lib.pa_prefill_chunk(*args(c, H=33)) == -6
    assert lib.pa_prefill_chunk(*args(c, T=-1)) == -3
    assert lib.pa_prefill_chunk(*args(c, out=0)) == -1
    assert lib.pa_prefill_chunk(*args(c, scale=float("inf"))) == -3
    assert lib.pa_prefill_chunk(*args(c, T=0)) == 0
    assert lib.pa_prefill_chunk(*args(c, S=0)) == 0


def test_error_message_clears_on_success(lib):
    decode(lib, cache(bs=24))
    assert msg()
    assert lib.pa_kv_cache_write(ctypes.byref(cache()), FAKE, FAKE, FAKE, 0, None) == 0
    assert msg() == ""


def test_python_errors_carry_status(lib):
    err = _binding.PagedAttnError("pa_decode", -4, "block_size 24 not in {8, 16, 32}")
    assert err.status == "PA_ERR_BLOCK_SIZE" and "pa_decode" in str(err)


# ---------------------------------------------------------------- contracts

def test_contract_checks():
    check_slot_mapping([0, 5, -1, 7], 2, 4)
    with pytest.raises(ContractError, match="outside a pool"):
        check_slot_mapping([8], 2, 4)
    with pytest.raises(ContractError, match="written twice"):
        check_slot_mapping([3, 3], 2, 4)
    bt = np.array([[1, 0, 9], [2, 3, 9]])
    check_decode_contracts(bt, [5, 8], num_blocks=4, block_size=4, max_context_len=8)
    with pytest.raises(ContractError, match="block id"):
        check_decode_contracts(bt, [9, 8], num_blocks=4, block_size=4, max_context_len=12)
    with pytest.raises(ContractError, match="above max_context_len"):
        check_decode_contracts(bt, [5, 8], num_blocks=4, block_size=4, max_context_len=7)
    with pytest.raises(ContractError, match="needs more than"):
        check_decode_contracts(bt, [13, 8], num_blocks=10, block_size=4, max_context_len=20)
    check_prefill_contracts([0, 3, 5], bt, [5, 8], 4, 4, max_query_len=3, max_context_len=8, num_query_tokens=5)
    with pytest.raises(ContractError, match="longer than its context"):
        check_prefill_contracts([0, 6, 8], bt, [5, 8], 4, 4, max_query_len=6, max_context_len=8,
                                num_query_tokens=8)
    with pytest.raises(ContractError, match="max_query_len"):
        check_prefill_contracts([0, 3, 5], bt, [5, 8], 4, 4, max_query_len=2, max_context_len=8,
                                num_query_tokens=5)


def test_workloads_satisfy_contracts():
    import workloads as W
    for c in (W.make_config("tiny_fp32_decode"),
              W.random_decode(3, [1, 50, 300], block_size=8, dtype=W.BF16),
              W.random_prefill(4, [0, 33], [17, 64], block_size=16)):
        check_slot_mapping(c.slot_mapping, c.num_blocks, c.block_size)
        check_decode_contracts(c.block_tables, c.context_lens, c.num_blocks, c.block_size, c.max_context_len)


def test_copy_blocks_validation(lib):
    a, b = cache(nb=10), cache(nb=20)
    cp = lambda s, d, si=None, di=None, n=5: lib.pa_kv_cache_copy_blocks(ctypes.byref(s), ctypes.byref(d), si,
                                                                         di, n, None)
    assert cp(a, b, n=0) == 0                                    # nothing to do
    assert cp(a, cache(nb=20, dtype=0)) == -2
    assert cp(a, cache(nb=20, bs=16)) == -3 and "block shapes differ" in msg()
    assert cp(a, cache(nb=20, d=64)) == -3
    assert cp(a, b, si=FAKE) == -1 and "both or neither" in msg()
    assert cp(a, b, n=-1) == -3
    assert cp(a, b, n=11) == -3 and "identity copy of 11 blocks" in msg()
    assert cp(b, a, n=11) == -3
    assert cp(a, cache(k=0)) == -1


def test_measurement_helpers_validation(lib):
    """The stream-read, matrix-ceiling and clock probes reject their
    arguments before any launch."""
    assert lib.pa_stream_read(None, 16, FAKE, None) == -1
    assert lib.pa_stream_read(FAKE, 16, None, None) == -1
    assert lib.pa_stream_read(FAKE, 20, FAKE, None) == -3 and "multiple of 16" in msg()
    assert lib.pa_stream_read(FAKE, 0, FAKE, None) == 0  # nothing to read
    assert lib.pa_clock_probe(None, 1000, None) == -1
    assert lib.pa_clock_probe(FAKE, 0, None) == -3 and "ticks 0 outside" in msg()
    assert lib.pa_clock_probe(FAKE, 1000001, None) == -3
    assert lib.pa_mfma_peak(None, 16, None) == -1
    assert lib.pa_mfma_peak(FAKE, 0, None) == -3 and "iters 0 outside" in msg()
    assert lib.pa_mfma_peak(FAKE, 65537, None) == -3


def test_serve_validation(lib):
    """The native serving step rejects bad arguments before touching the
    device (no pinned allocation, no copy, no launch)."""
    assert lib.pa_serve_meta_bytes(0, 8, 16) == 0
    assert lib.pa_serve_meta_bytes(4, 8, 16) >= 16 * 8 + 5 * 4 + 4 * 4 + 4 * 8 * 4
    assert lib.pa_serve_meta_bytes(4, 8, 16) % 256 == 0
    assert not lib.pa_serve_create(None, 32, 0.1, 0, 0, 4, 8, 16, FAKE, 1 << 20) and "required" in msg()
    sched = FAKE  # never dereferenced: creation fails on the sizes first
    assert not lib.pa_serve_create(sched, 32, 0.1, 0, 0, 4, 8, 16, None, 1 << 20)
    assert not lib.pa_serve_create(sched, 32, 0.1, 0, 0, 0, 8, 16, FAKE, 1 << 20) and "positive" in msg()
    assert not lib.pa_serve_create(sched, 32, 0.1, 0, 0, 4, 8, 16, FAKE, 64) and "need" in msg()
    assert not lib.pa_serve_create(sched, 32, 0.1, -1, 0, 4, 8, 16, FAKE, 1 << 20)
    assert not lib.pa_serve_create(sched, 32, 0.1, 0, -1, 4, 8, 16, FAKE, 1 << 20) and "mixed_split_context" in msg()
    step = _binding.PaStep()
    fin = ctypes.c_int32(0)
    assert lib.pa_serve_plan(None, ctypes.byref(step), None) == -1
    assert lib.pa_serve_attend(None, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert lib.pa_serve_complete(None, None, ctypes.byref(fin)) == -1
    lib.pa_serve_destroy(None)


def test_value_head_dim_validation(lib):
    """A value head dim of its own (0 = the key head dim): attention takes
    64 or 128, the workspace is sized by it (cascade decode's too), and the
    copy checks it."""
    assert ctypes.sizeof(_binding.PaKvCache) == 2 * 8 + 6 * 4
    for dv in (32, 96, 256):
        assert decode(lib, cache(dv=dv)) == -5
        assert f"v_head_dim {dv} not in {{64, 128}}" in msg()
    assert decode(lib, cache(dv=-1)) == -5 and "v_head_dim -1" in msg()
    need = P.pa_decode_workspace_bytes(4, 32, 64, 1000, 256)
    assert need < P.pa_decode_workspace_bytes(4, 32, 128, 1000, 256)
    assert decode(lib, cache(dv=64), mcl=1000, ps=256) == -7 and f"{need} bytes needed" in msg()
    assert decode(lib, cache(d=64, dv=128), mcl=1000, ps=256, ws=FAKE, ws_bytes=need) == -7
    # write: each row width must be a multiple of 16 bytes
    odd_v = cache(hkv=1, d=8, dv=6)                                 # 16-byte K rows, 12-byte V rows
    assert lib.pa_kv_cache_write(ctypes.byref(odd_v), FAKE, FAKE, FAKE, 5, None) == -3
    assert "v_head_dim" in msg()
    assert lib.pa_kv_cache_write(ctypes.byref(cache(dv=24)), FAKE, FAKE, FAKE, 0, None) == 0
    # copy: both pools must agree on the value head dim (0 and the key dim are the same)
    cp = lambda s, d: lib.pa_kv_cache_copy_blocks(ctypes.byref(s), ctypes.byref(d), None, None, 0, None)
    assert cp(cache(dv=64), cache(dv=128)) == -3 and "v_head_dim" in msg()
    assert cp(cache(dv=0), cache(dv=128)) == 0
    # cascade decode: the partials take the value head dim
    need_v = P.pa_decode_cascade_workspace_bytes(4, 32, 64, 1000, 256)
    assert need_v < P.pa_decode_cascade_workspace_bytes(4, 32, 128, 1000, 256)
    assert lib.pa_decode_cascade(ctypes.byref(cache(dv=64)), FAKE, FAKE, 4, 32, FAKE, 8, FAKE, 1000, 0.1, 256, 2,
                                 FAKE, FAKE, 2, 512, FAKE, need_v - 1, None) == -7 and f"{need_v} needed" in msg()
    # prefill takes unequal dims
    assert lib.pa_prefill_chunk(ctypes.byref(cache(dv=64)), FAKE, FAKE, FAKE, 2, 32, 0, 32, FAKE, 8, FAKE, 100,
                                0.1, None) == 0
    assert lib.pa_prefill_chunk(ctypes.byref(cache(dv=96)), FAKE, FAKE, FAKE, 2, 32, 0, 32, FAKE, 8, FAKE, 100,
                                0.1, None) == -5


def test_cascade_validation(lib):
    c = cache()
    def casc(c=c, S=4, H=32, ps=256, ng=2, gs=FAKE, sl=FAKE, mg=2, ws=FAKE, ws_bytes=10 ** 9, mcl=1000, msl=512):
        return lib.pa_decode_cascade(ctypes.byref(c), FAKE, FAKE, S, H, FAKE, 8, FAKE, mcl, 0.1, ps, ng, gs, sl, mg,
                                     msl, ws, ws_bytes, None)
    assert casc(ps=0) == -10 and "partition_size > 0" in msg()
    assert casc(ps=48) == -10
    assert casc(c=cache(dtype=0)) == -8 and "bf16 only" in msg()
    assert casc(H=48) == -6                                   # 6 query heads per kv head
    assert casc(ng=0) == -3
    assert casc(gs=None) == -1
    assert casc(mg=0) == -3 and casc(mg=5) == -3
    assert casc(msl=-1) == -3 and "max_shared_len" in msg()
    need = P.pa_decode_cascade_workspace_bytes(4, 32, 128, 1000, 256)
    assert casc(ws=None) == -7 and f"{need} bytes needed" in msg()
    assert casc(ws_bytes=need - 1) == -7
    # slots: 512-token chunks of the shared part, then the row's partitions
    n = 4 * 32 * (-(-1000 // 512) + -(-1000 // 256))
    a = lambda x: (x + 255) // 256 * 256
    assert need == 2 * a(4 * n) + a(4 * n * 128)
    assert casc(S=0, ng=0) == 0
    # one launch runs every group's shared chunks (x their column tiles)
    # ahead of the rows' own partitions: more than 65,535 grid rows of
    # num_seqs items are rejected before any launch
    huge = 1 << 26
    assert casc(S=256, ng=256, mg=1, mcl=huge, msl=huge, ws_bytes=1 << 60) == -3 and "grid rows" in msg()


def test_decode_append_validation(lib):
    """pa_decode_append checks what pa_decode checks, then the new rows."""
    def app(c=None, key=FAKE, value=FAKE, S=4, H=32, ps=0, ws=None, ws_bytes=0):
        c = c or cache()
        return lib.pa_decode_append(ctypes.byref(c), FAKE, FAKE, key, value, S, H, FAKE, 8, FAKE, 100, 0.1, ps, ws,
                                    ws_bytes, None)
    assert app(c=cache(bs=24)) == -4
    assert app(H=30) == -6
    assert app(key=None) == -1 and "key=" in msg()
    assert app(value=None) == -1
    assert app(ps=48) == -10
    assert app(c=cache(hkv=1, d=8, dv=6), H=1) == -5          # v_head_dim 6 not an attention shape
    assert app(S=0, key=None, value=None) == 0                  # nothing to do
