"""The serving loop on the GPU (see serving_util): scheduler-built block
tables and slot mappings drive the library's write, prefill and decode
kernels, and every output row matches the oracle's attention over the
request's dense K/V.  The pool is small enough that requests are
preempted and recomputed, and half of them share a system prompt
(prefix-cache hits)."""

import pytest

import workloads as W

from gpu_util import BF16_MAX_ABS, log
from serving_util import LibraryBackend, NativeBackend, serve_and_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("partition_size", [0, 64])
def test_scheduled_serving_matches_dense_oracle(partition_size):
    tr = W.serving_trace(seed=6000, num_requests=12, num_blocks=64)
    r = serve_and_check(tr, LibraryBackend(tr), partition_size=partition_size)
    assert r["stats"]["prefix_hit_tokens"] > 0, r["stats"]
    assert r["recomputed"] > 0, "the pool was expected to force preemption"
    assert 1 in r["kinds"] and 2 in r["kinds"]
    assert r["worst"] <= BF16_MAX_ABS
    log(f"serving ps={partition_size}: {r['steps']} steps, worst max-abs {r['worst']:.2e}, "
        f"{r['recomputed']} recomputed, hits {r['stats']['prefix_hit_tokens']} tokens")


def test_serving_with_pool_growth():
    """The device pool grows twice mid-trace through pa_kv_cache_copy_blocks;
    outputs keep matching the oracle's dense attention."""
    tr = W.serving_trace(seed=6003, num_requests=12, num_blocks=40)
    r = serve_and_check(tr, LibraryBackend(tr), partition_size=64, grow_at={6: 56, 14: 160}, tag="-grow")
    assert r["stats"]["num_blocks"] == 160
    assert r["worst"] <= BF16_MAX_ABS


def test_mixed_batch_serving_matches_dense_oracle():
    """Mixed steps (every decode row, then prompt chunks, one prefill launch)
    through the library's kernels match the oracle's dense attention."""
    tr = W.serving_trace(seed=6005, num_requests=12, num_blocks=64)
    r = serve_and_check(tr, LibraryBackend(tr), partition_size=64, tag="-mixed", mixed=True)
    assert 3 in r["kinds"]
    assert r["worst"] <= BF16_MAX_ABS
    log(f"serving mixed: {r['steps']} steps ({r['kinds'].count(3)} mixed), worst max-abs {r['worst']:.2e}")


@pytest.mark.parametrize("partition_size", [0, 64])
def test_native_serving_matches_dense_oracle(partition_size):
    """The same trace through the library's native serving step (plan into
    pinned memory, one copy, write and attention launched by the library):
    every output row matches the oracle's dense attention."""
    tr = W.serving_trace(seed=6000, num_requests=12, num_blocks=64)
    r = serve_and_check(tr, NativeBackend(tr), partition_size=partition_size, tag="-native")
    assert r["recomputed"] > 0 and 1 in r["kinds"] and 2 in r["kinds"]
    assert r["worst"] <= BF16_MAX_ABS
    log(f"native serving ps={partition_size}: {r['steps']} steps, worst max-abs {r['worst']:.2e}")


@pytest.mark.parametrize("split", [1, 0])
def test_native_serving_mixed_and_growth(split):
    """Mixed batches through the native step, their decode rows through
    split-K decode (split 1: from any context) or with the chunks in one
    prefill launch (0), and a pool that grows mid-trace (the pool is passed
    to every attend call)."""
    tr = W.serving_trace(seed=6005, num_requests=12, num_blocks=64)
    be = NativeBackend(tr)
    be.mixed_split_context = split
    r = serve_and_check(tr, be, partition_size=64, tag=f"-native-mixed-split{split}", mixed=True)
    assert 3 in r["kinds"] and r["worst"] <= BF16_MAX_ABS
    tr = W.serving_trace(seed=6003, num_requests=12, num_blocks=40)
    r = serve_and_check(tr, NativeBackend(tr), partition_size=64, grow_at={6: 56, 14: 160}, tag="-native-grow")
    assert r["stats"]["num_blocks"] == 160 and r["worst"] <= BF16_MAX_ABS


def test_native_serving_asynchronous():
    """The native step as a serving loop runs it: no synchronisation between
    steps (the step's q/k/v rows uploaded from pinned memory without
    blocking, each step's output rows copied aside on the device), so the
    host plans step i+1 and i+2 while the GPU still runs step i and the two
    staging buffers alternate under load.  Every step's rows are checked
    against the oracle's dense attention after the loop."""
    import numpy as np

    import oracle
    import paged_attention_kv_cache_amd as P
    from gpu_util import assert_close, to_host_f32, torch
    from serving_util import DenseKV

    t = torch()
    tr = W.serving_trace(seed=6007, num_requests=12, num_blocks=96)
    H, Hkv, D = tr.num_heads, tr.num_kv_heads, tr.head_dim
    max_seqs, max_blocks, budget = 8, 32, 256
    m = P.KvManager(tr.num_blocks, tr.block_size)
    s = P.StepScheduler(m, max_batched_tokens=budget, max_chunk_tokens=128, max_seqs=max_seqs,
                        max_blocks_per_seq=max_blocks, mixed=True)
    for rid, prompt in tr.prompts.items():
        s.add_request(rid, prompt, tr.max_new[rid])
    srv = P.Server(s, H, tr.scale, 64, max_seqs, max_blocks, budget, mixed_split_context=1)
    ws = t.empty(P.pa_decode_workspace_bytes(max_seqs, H, D, max_blocks * tr.block_size, 64), dtype=t.uint8,
                 device="cuda")
    kc = t.zeros((tr.num_blocks, tr.block_size, Hkv, D), dtype=t.bfloat16, device="cuda")
    vc = t.zeros_like(kc)
    expected = {rid: list(p) for rid, p in tr.prompts.items()}
    gen = {rid: 0 for rid in tr.prompts}
    dense = DenseKV(tr)
    keep, records = [], []
    for step in range(2000):
        w, a, _ = s.counts()
        if w == 0 and a == 0:
            break
        st = srv.plan()
        ids = st.request_ids.tolist()
        qsl = st.query_start_loc.astype(np.int64).copy()
        ctx = st.context_lens.astype(np.int64).copy()
        T = st.num_tokens
        keys = np.empty((T, Hkv, D), np.uint16)
        vals = np.empty_like(keys)
        qs = np.empty((T, H, D), np.uint16)
        firsts = []
        for i, rid in enumerate(ids):
            n = int(qsl[i + 1] - qsl[i])
            first = int(ctx[i]) - n
            firsts.append(first)
            k, v = dense.get(rid, expected[rid], int(ctx[i]))
            keys[qsl[i]:qsl[i + 1]] = k[first:]
            vals[qsl[i]:qsl[i + 1]] = v[first:]
            qs[qsl[i]:qsl[i + 1]] = tr.q(rid, first, n)
        host = [t.from_numpy(x.view(np.int16)).pin_memory() for x in (keys, vals, qs)]
        dk, dv, dq = (h.cuda(non_blocking=True).view(t.bfloat16) for h in host)
        out = t.empty((T, H, D), dtype=t.bfloat16, device="cuda")
        srv.attend(kc, vc, dk, dv, dq, out, workspace=ws)
        keep.append((host, dk, dv, dq))
        records.append((st.kind, ids, qsl, ctx, firsts, qs, out))
        sampled = [tr.sampled_token(rid, int(ctx[i])) for i, rid in enumerate(ids)]
        srv.complete(sampled)
        for i, rid in enumerate(ids):
            if int(ctx[i]) >= len(expected[rid]) and gen[rid] < tr.max_new[rid]:
                expected[rid].append(sampled[i])
                gen[rid] += 1
    else:
        raise AssertionError("serving did not finish")
    t.cuda.synchronize()
    log(f"native serving, asynchronous: {len(records)} steps")
    worst = 0.0
    for step, (kind, ids, qsl, ctx, firsts, qs, out) in enumerate(records):
        got = to_host_f32(out, W.BF16)
        for i, rid in enumerate(ids):
            k, v = dense.get(rid, expected[rid], int(ctx[i]))
            ref = oracle.attention(W.storage_to_f32(qs[qsl[i]:qsl[i + 1]], W.BF16), W.storage_to_f32(k, W.BF16),
                                   W.storage_to_f32(v, W.BF16), tr.scale, np.arange(firsts[i], int(ctx[i])))
            err, _ = assert_close(got[qsl[i]:qsl[i + 1]], ref, W.BF16, f"async step {step} request {rid}")
            worst = max(worst, err)
    assert 3 in [r[0] for r in records]
    srv.close()
    s.close()
    m.close()
    assert worst <= BF16_MAX_ABS
