"""Seeded request traces for the serving loop (block manager + scheduler +
kernels): prompts, generation lengths, and per-token Q/K/V.

Input construction only.  A token's K and V depend on the token ids up to
and including it (a running hash of the prefix seeds their draw), as in a
real model, so a block reused through the prefix cache holds exactly the
values the reusing request would have computed itself.  Q depends on the
request and position (queries are never cached).  Values are standard
normal, rounded to bf16 (nearest, ties to even) for bf16 traces.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .generate import BF16, f32_to_bf16_bits

_MASK = (1 << 63) - 1


def _prefix_hash(h: int, token: int) -> int:
    return (h * 1000003 + token + 1) & _MASK


@dataclasses.dataclass
class ServingTrace:
    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    prompts: dict            # request id -> list of token ids
    max_new: dict            # request id -> tokens to generate
    seed: int
    dtype: str = BF16

    def sampled_token(self, rid: int, pos: int) -> int:
        """The token 'sampled' after position pos - 1 (a fixed function:
        the trace does not depend on attention outputs)."""
        return (rid * 7919 + pos * 131 + self.seed) % 32000 + 1

    def kv(self, tokens, start: int = 0, state=None):
        """K and V ``[len(tokens) - start, num_kv_heads, head_dim]`` (storage
        bits for bf16) of positions start .. len(tokens) - 1 of a token
        sequence, and the prefix state after the last one.  ``state`` is the
        state returned for the first ``start`` tokens (None when start = 0)."""
        if start and state is None:
            raise ValueError("state of the first `start` tokens is required")
        shape = (self.num_kv_heads, self.head_dim)
        n = len(tokens) - start
        k = np.empty((n,) + shape, np.float32)
        v = np.empty_like(k)
        h = self.seed if state is None else state
        for i in range(n):
            h = _prefix_hash(h, int(tokens[start + i]))
            g = np.random.default_rng(h)
            k[i] = g.standard_normal(shape, dtype=np.float32)
            v[i] = g.standard_normal(shape, dtype=np.float32)
        return self._store(k), self._store(v), h

    def q(self, rid: int, first: int, count: int) -> np.ndarray:
        """Queries ``[count, num_heads, head_dim]`` of positions first ..
        first + count - 1 of a request."""
        out = np.empty((count, self.num_heads, self.head_dim), np.float32)
        for i in range(count):
            g = np.random.default_rng([self.seed, rid, first + i])
            out[i] = g.standard_normal((self.num_heads, self.head_dim), dtype=np.float32)
        return self._store(out)

    def _store(self, x: np.ndarray) -> np.ndarray:
        return f32_to_bf16_bits(x) if self.dtype == BF16 else x


def serving_trace(seed: int = 6000, num_requests: int = 12, num_blocks: int = 64,
                  prompt_range=(20, 300), new_range=(4, 24), shared_prefix: int = 64,
                  num_heads: int = 8, num_kv_heads: int = 2, head_dim: int = 128,
                  block_size: int = 16) -> ServingTrace:
    """Requests with uniform prompt and generation lengths; every other
    request starts with a common ``shared_prefix``-token system prompt.  The
    pool is deliberately small so that the scheduler preempts."""
    rng = np.random.default_rng(seed)
    system = rng.integers(1, 32000, shared_prefix).tolist()
    prompts, max_new = {}, {}
    for r in range(num_requests):
        n = int(rng.integers(prompt_range[0], prompt_range[1] + 1))
        body = rng.integers(1, 32000, n).tolist()
        prompts[r] = system + body if r % 2 == 0 else body
        max_new[r] = int(rng.integers(new_range[0], new_range[1] + 1))
    return ServingTrace(f"serving_s{seed}", num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        1.0 / float(np.sqrt(head_dim)), prompts, max_new, seed)
