"""Paged attention over a block-table KV cache for AMD Instinct MI355X (gfx950).

The work is done by hand-written HIP kernels behind the C ABI in
``include/pagedattn.h`` (``libpagedattn.so``, built in-tree by
``paged_attention_kv_cache_amd.build``).  This package is only the binding:

* ``pa_kv_cache_write``  - slot-mapping scatter of new K/V into the pool
* ``pa_kv_cache_copy_blocks`` - whole-block copies (pool growth, copy of a
  shared block)
* ``pa_decode``          - one query per sequence over its context; split-K
  partitions plus reduce (``pa_decode_partition`` / ``pa_decode_reduce``
  run the two stages separately)
* ``pa_decode_static``   - ``pa_decode`` with its split-K partials in a
  static device scratch of the library, for callers that cannot allocate
* ``pa_decode_cascade``  - decode of groups sharing a prefix of whole blocks,
  the shared tokens read once per group (an MFMA pass) and merged with each
  sequence's own split-K partitions
* ``pa_prefill_chunk``   - causal attention of packed chunks over their
  cached prefixes (bf16 MFMA)

Host side (``include/pagedattn_kvm.h``): ``KvManager`` (block pool, LRU free
list, block-hash prefix cache) and ``StepScheduler`` (alternating prompt /
decode steps) produce the block tables and slot mappings those kernels take.
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    PA_DTYPE_BF16,
    PA_DTYPE_F32,
    STATUS,
    PagedAttnError,
    PaKvCache,
    load_library,
    make_cache,
    pa_decode,
    pa_decode_append,
    pa_decode_cascade,
    pa_decode_cascade_workspace_bytes,
    pa_decode_partition,
    pa_decode_reduce,
    pa_decode_static,
    pa_decode_workspace_bytes,
    pa_kv_cache_copy_blocks,
    pa_kv_cache_write,
    pa_last_error_message,
    pa_prefill_chunk,
    pa_status_string,
    pa_stream_read,
    pa_clock_probe,
    pa_mfma_peak,
    pa_version,
)
from .kv_manager import (KIND_DECODE, KIND_IDLE, KIND_MIXED, KIND_PROMPT, KvManager, Server, Step,  # noqa: F401
                         StepScheduler, grow_pool)
from .contracts import check_decode_contracts, check_prefill_contracts, check_slot_mapping  # noqa: F401
