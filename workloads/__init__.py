"""Seeded synthetic inputs for paged attention over a block-table KV cache.

This package only *generates inputs*: context lengths, block pools, block
tables, slot mappings and Q/K/V values.  It contains none of the attention
arithmetic, so both the CPU oracle and the HIP path can consume what it
produces without sharing any computation.
"""

from .generate import (  # noqa: F401
    BF16,
    F32,
    DecodeCase,
    PrefillCase,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    storage_to_f32,
    tiny_fp32_decode,
    decode_batch,
    long_context_decode,
    chunked_prefill,
    prefix_shared_decode,
    random_decode,
    random_prefill,
    CONFIG_NAMES,
    make_config,
)
from .serving import ServingTrace, serving_trace  # noqa: F401
