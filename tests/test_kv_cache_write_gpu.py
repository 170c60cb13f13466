"""kv_cache_write on the GPU against the oracle's scatter: bit-exact, and every
slot not named by the slot mapping left untouched (pools poisoned with NaN)."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import DeviceCase, log, to_dev, to_host_bits, torch

pytestmark = pytest.mark.gpu


def _check_write(case, what):
    log(f"kv_cache_write {what}: T={case.slot_mapping.size} pool={case.k_cache.shape} {case.dtype}")
    dev = DeviceCase(case)
    dev.write()
    torch().cuda.synchronize()
    k_ref, v_ref = oracle.kv_cache_write(case.k_cache, case.v_cache, case.new_key, case.new_value,
                                         case.slot_mapping)
    k_got, v_got = to_host_bits(dev.k_cache), to_host_bits(dev.v_cache)
    bits = np.uint16 if case.dtype == W.BF16 else np.uint32
    assert np.array_equal(k_got.view(bits), k_ref.view(bits)), f"{what}: K pool differs"
    assert np.array_equal(v_got.view(bits), v_ref.view(bits)), f"{what}: V pool differs"


def test_write_tiny_fp32_one_token():
    _check_write(W.make_config("tiny_fp32_decode"), "tiny fp32, 1 token")


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_write_prefill_chunks(bs, dtype):
    case = W.random_prefill(100 + bs, [0, 7, 33, 100], [5, 64, 31, 1], num_heads=8, num_kv_heads=2,
                            head_dim=64, block_size=bs, dtype=dtype)
    _check_write(case, f"prefill chunks bs{bs}")


def test_write_skips_negative_and_out_of_pool_slots():
    case = W.random_prefill(7, [3, 10], [9, 4], num_heads=4, num_kv_heads=4, head_dim=128,
                            block_size=16, dtype=W.BF16)
    sm = case.slot_mapping.copy()
    sm[2] = -1
    sm[5] = case.num_blocks * case.block_size          # one past the pool
    sm[7] = case.num_blocks * case.block_size + 12345
    case.slot_mapping = sm
    log("kv_cache_write with skipped slots")
    dev = DeviceCase(case)
    dev.write()
    torch().cuda.synchronize()
    sm_oracle = sm.copy()
    sm_oracle[sm_oracle >= case.num_blocks * case.block_size] = -1   # documented: skipped
    k_ref, v_ref = oracle.kv_cache_write(case.k_cache, case.v_cache, case.new_key, case.new_value, sm_oracle)
    assert np.array_equal(to_host_bits(dev.k_cache), k_ref)
    assert np.array_equal(to_host_bits(dev.v_cache), v_ref)


def test_write_chunked_prefill_full_size():
    case = W.make_config("chunked_prefill")
    _check_write(case, "chunked prefill 8 x 512")


def test_copy_blocks_grow_and_remap():
    """Identity copy of a pool into a larger one, and an id-mapped copy inside
    one pool, are bit-exact; untouched and out-of-range targets stay as they
    were."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    rng = np.random.default_rng(5)
    for dtype, shape in ((W.BF16, (37, 16, 8, 128)), (W.F32, (11, 8, 2, 64))):
        n = shape[0]
        k = rng.standard_normal(shape).astype(np.float32)
        v = rng.standard_normal(shape).astype(np.float32)
        if dtype == W.BF16:
            k, v = W.f32_to_bf16_bits(k), W.f32_to_bf16_bits(v)
        dk, dv = to_dev(k, dtype), to_dev(v, dtype)
        log(f"copy blocks grow {dtype} {shape}")
        big_k = t.full((n + 9,) + shape[1:], float("nan"), dtype=dk.dtype, device="cuda")
        big_v = t.full_like(big_k, float("nan"))
        P.pa_kv_cache_copy_blocks(dk, dv, big_k, big_v)
        t.cuda.synchronize()
        gk, gv = to_host_bits(big_k), to_host_bits(big_v)
        assert np.array_equal(gk[:n], k) and np.array_equal(gv[:n], v)
        assert np.isnan(W.storage_to_f32(gk[n:], dtype)).all()
        # id map inside one pool, with one out-of-range pair skipped
        src = np.array([0, 3, 5, n + 100], dtype=np.int32)
        dst = np.array([7, 1, 2, 4], dtype=np.int32)
        log(f"copy blocks remap {dtype}")
        P.pa_kv_cache_copy_blocks(dk, dv, dk, dv, t.from_numpy(src).cuda(), t.from_numpy(dst).cuda())
        t.cuda.synchronize()
        ek, ev = k.copy(), v.copy()
        for a, b in zip(src[:3], dst[:3]):
            ek[b], ev[b] = k[a], v[a]
        assert np.array_equal(to_host_bits(dk), ek) and np.array_equal(to_host_bits(dv), ev)


@pytest.mark.parametrize("dims", [(128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_write_and_copy_separate_value_dim(dims, dtype):
    """K and V rows of different widths: the write stores each at its own
    width, bit-exact, and a grow copy moves both pools whole."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    D, Dv = dims
    case = W.random_prefill(900 + D, [0, 7, 33, 100], [5, 64, 31, 1], num_heads=8, num_kv_heads=2,
                            head_dim=D, v_head_dim=Dv, block_size=16, dtype=dtype)
    assert case.v_cache.shape[3] == Dv and case.new_value.shape[2] == Dv
    _check_write(case, f"separate value dim D={D} Dv={Dv}")
    dev = DeviceCase(case)
    n = case.num_blocks
    log(f"copy blocks grow with D={D} Dv={Dv} {dtype}")
    big_k = t.zeros((n + 3,) + tuple(dev.k_cache.shape[1:]), dtype=dev.k_cache.dtype, device="cuda")
    big_v = t.zeros((n + 3,) + tuple(dev.v_cache.shape[1:]), dtype=dev.v_cache.dtype, device="cuda")
    P.pa_kv_cache_copy_blocks(dev.k_cache, dev.v_cache, big_k, big_v)
    t.cuda.synchronize()
    bits = np.uint16 if dtype == W.BF16 else np.uint32
    assert np.array_equal(to_host_bits(big_k)[:n].view(bits), case.k_cache.view(bits))
    assert np.array_equal(to_host_bits(big_v)[:n].view(bits), case.v_cache.view(bits))
    assert not to_host_bits(big_v)[n:].any()
