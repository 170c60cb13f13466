"""The serving loop on the CPU: the oracle's paged functions over
scheduler-built block tables equal the oracle's attention over each
request's dense K/V at every step, with preemption and prefix-cache hits
in the trace.  This pins the manager's tables and slot mappings (and the
oracle's gather through them) before any kernel runs them."""

import workloads as W

from serving_util import OracleBackend, serve_and_check


def test_scheduled_serving_with_oracle_backend():
    tr = W.serving_trace(seed=6001, num_requests=8, num_blocks=16, prompt_range=(10, 150), new_range=(2, 10),
                         shared_prefix=32, num_heads=4, num_kv_heads=2, head_dim=64)
    r = serve_and_check(tr, OracleBackend(tr), max_batched_tokens=128, max_chunk_tokens=64, max_seqs=6,
                        max_blocks_per_seq=16, tag="-cpu")
    assert r["stats"]["prefix_hit_tokens"] > 0, r["stats"]
    assert r["recomputed"] > 0
    assert 1 in r["kinds"] and 2 in r["kinds"]
    assert r["worst"] < 1e-5  # oracle against oracle: float64 with bf16-valued inputs (rounding only)


def test_serving_with_pool_growth_oracle_backend():
    """The pool grows mid-trace (K/V of placed sequences carried over); every
    step still reads back exactly the dense attention."""
    tr = W.serving_trace(seed=6002, num_requests=8, num_blocks=16, prompt_range=(10, 150), new_range=(2, 10),
                         shared_prefix=32, num_heads=4, num_kv_heads=2, head_dim=64)
    r = serve_and_check(tr, OracleBackend(tr), max_batched_tokens=128, max_chunk_tokens=64, max_seqs=6,
                        max_blocks_per_seq=16, tag="-cpu-grow", grow_at={4: 24, 9: 64})
    assert r["stats"]["num_blocks"] == 64
    assert r["worst"] < 1e-5


def test_mixed_batch_serving_with_oracle_backend():
    """One batch per step (decode rows, then prompt chunks) through the
    prefill path: every row still equals the dense attention."""
    tr = W.serving_trace(seed=6004, num_requests=8, num_blocks=16, prompt_range=(10, 150), new_range=(2, 10),
                         shared_prefix=32, num_heads=4, num_kv_heads=2, head_dim=64)
    r = serve_and_check(tr, OracleBackend(tr), max_batched_tokens=128, max_chunk_tokens=64, max_seqs=6,
                        max_blocks_per_seq=16, tag="-cpu-mixed", mixed=True)
    assert 3 in r["kinds"]
    assert r["recomputed"] > 0
    assert r["worst"] < 1e-5
