"""CPU oracle (test infrastructure only) for paged attention over a
block-table KV cache.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package; the library never does, and this package
imports nothing from the library.  See ``oracle.attention`` for what each
function computes and which passage it follows.
"""

from .attention import (  # noqa: F401
    attention,
    attention_weights,
    gather_sequence,
    kv_cache_write,
    paged_decode,
    paged_prefill,
)
