"""pa_decode_static (split-K partials in the library's static device scratch,
no allocation) against pa_decode with a caller workspace, through the C ABI.

Two calls in a row on the same GPU scratch, the second with a smaller batch
and shorter contexts, each compared bit for bit with pa_decode on the same
inputs (same kernels, same partition order) and with the CPU oracle at the
bf16 / fp32 tolerances.  The scratch keeps the first call's partials when
the second runs, so a partial the second call failed to rewrite would show.
"""

import numpy as np
import pytest

import paged_attention_kv_cache_amd as P
import workloads as W
from gpu_util import DeviceCase, assert_close, log, oracle_decode, to_host_bits, to_host_f32, torch

pytestmark = pytest.mark.gpu


def _both(case, partition_size):
    dev = DeviceCase(case)
    dev.write()
    c = case
    ref_out = P.pa_decode(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens, c.scale,
                          c.max_context_len, partition_size)
    got_out = P.pa_decode_static(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens, c.scale,
                                 c.max_context_len, partition_size)
    torch().cuda.synchronize()
    return to_host_bits(got_out), to_host_bits(ref_out), to_host_f32(got_out, c.dtype)


@pytest.mark.parametrize("partition_size", [512, 256])
def test_static_scratch_decode_two_calls(partition_size):
    big = W.make_config("decode_batch_bs32")
    small = W.random_decode(4242, [5, 33, 600, 1500, 2047], num_heads=32, num_kv_heads=8, head_dim=128,
                            block_size=32, dtype=W.BF16)
    for name, case in (("bs32 batch", big), ("5 short sequences", small)):
        need = P.pa_decode_workspace_bytes(len(case.context_lens), case.q.shape[1], case.v_cache.shape[3],
                                           case.max_context_len, partition_size)
        log(f"pa_decode_static {name} partition={partition_size} partials={need} bytes")
        assert 0 < need <= 32 << 20
        got_bits, ref_bits, got = _both(case, partition_size)
        assert np.array_equal(got_bits, ref_bits), f"{name}: static-scratch decode differs from pa_decode"
        assert_close(got, oracle_decode(case), case.dtype, f"{name} vs oracle")


def test_static_scratch_decode_fp32_and_single_pass():
    case = W.make_config("tiny_fp32_decode")
    for ps in (16, 0):
        log(f"pa_decode_static tiny fp32 partition={ps}")
        got_bits, ref_bits, got = _both(case, ps)
        assert np.array_equal(got_bits, ref_bits)
        assert_close(got, oracle_decode(case), W.F32, f"tiny fp32 ps{ps}")
