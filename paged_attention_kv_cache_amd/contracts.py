"""Host-side checks of the content contracts the kernels rely on.

The C ABI cannot check the contents of device buffers without reading them
back, so it only bounds every access.  These checks run on host (NumPy)
copies of the same inputs and name the first violation.  They are meant for
callers that stage inputs on the host, and for tests.
"""

from __future__ import annotations

import numpy as np


class ContractError(ValueError):
    pass


def check_slot_mapping(slot_mapping, num_blocks: int, block_size: int) -> None:
    s = np.asarray(slot_mapping, dtype=np.int64)
    used = s[s >= 0]
    if used.size and used.max() >= num_blocks * block_size:
        raise ContractError(f"slot {int(used.max())} outside a pool of {num_blocks} x {block_size} slots")
    if np.unique(used).size != used.size:
        vals, counts = np.unique(used, return_counts=True)
        raise ContractError(f"slot {int(vals[counts > 1][0])} is written twice")


def check_decode_contracts(block_tables, context_lens, num_blocks: int, block_size: int,
                           max_context_len: int) -> None:
    bt = np.asarray(block_tables)
    cl = np.asarray(context_lens, dtype=np.int64)
    if bt.ndim != 2 or bt.shape[0] != cl.shape[0]:
        raise ContractError(f"block_tables {bt.shape} and context_lens {cl.shape} disagree")
    if cl.size and cl.min() < 0:
        raise ContractError(f"negative context length {int(cl.min())}")
    if cl.size and cl.max() > max_context_len:
        raise ContractError(f"context length {int(cl.max())} above max_context_len {max_context_len}")
    cap = bt.shape[1] * block_size
    if cl.size and cl.max() > cap:
        raise ContractError(f"context length {int(cl.max())} needs more than {bt.shape[1]} blocks of {block_size}")
    for i, n in enumerate(cl.tolist()):
        used = bt[i, :-(-n // block_size)] if n else bt[i, :0]
        if used.size and (used.min() < 0 or used.max() >= num_blocks):
            raise ContractError(f"sequence {i}: block id outside [0, {num_blocks})")


def check_prefill_contracts(query_start_loc, block_tables, context_lens, num_blocks: int,
                            block_size: int, max_query_len: int, max_context_len: int,
                            num_query_tokens: int) -> None:
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    cl = np.asarray(context_lens, dtype=np.int64)
    if qsl.shape != (cl.shape[0] + 1,):
        raise ContractError(f"query_start_loc {qsl.shape} must have {cl.shape[0] + 1} entries")
    ql = np.diff(qsl)
    if qsl[0] < 0 or (ql < 0).any():
        raise ContractError("query_start_loc must be non-decreasing from >= 0")
    if qsl[-1] > num_query_tokens:
        raise ContractError(f"query_start_loc ends at {int(qsl[-1])} > {num_query_tokens} rows")
    if ql.size and ql.max() > max_query_len:
        raise ContractError(f"chunk of {int(ql.max())} rows above max_query_len {max_query_len}")
    if (ql > cl).any():
        raise ContractError("a chunk is longer than its context")
    check_decode_contracts(block_tables, context_lens, num_blocks, block_size, max_context_len)
