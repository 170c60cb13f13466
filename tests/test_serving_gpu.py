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
