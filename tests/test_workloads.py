"""Seeded input generators: determinism and structure (no GPU)."""

import numpy as np
import pytest

import workloads as W


def _same(a, b):
    for f in ("q", "k_cache", "v_cache", "new_key", "new_value", "slot_mapping", "block_tables",
              "context_lens"):
        x, y = getattr(a, f), getattr(b, f)
        assert x.dtype == y.dtype and x.shape == y.shape
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38, np.nan],
                 dtype=np.float32)
    b = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa is 1.0
    assert back[0] == 1.0 and back[1] == 1.0
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert back[2] == 1.0 + 2 ** -6
    assert back[3] == 1.0
    assert back[4] == -2.5
    assert np.isnan(back[6])
    # every bf16 value survives a round trip
    allbits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    vals = W.bf16_bits_to_f32(allbits)
    ok = ~np.isnan(vals)
    assert np.array_equal(W.f32_to_bf16_bits(vals[ok]), allbits[ok])


def test_tiny_decode_shape_and_determinism():
    a = W.make_config("tiny_fp32_decode")
    b = W.make_config("tiny_fp32_decode")
    _same(a, b)
    assert a.num_blocks == 64 and a.block_size == 16 and a.head_dim == 64
    assert a.num_heads == 8 and a.num_kv_heads == 2
    assert a.context_lens.tolist() == [100]
    assert len(set(a.block_tables[0, :7].tolist())) == 7
    # the new token is position 99: block-table entry 6, offset 3
    assert a.slot_mapping.tolist() == [int(a.block_tables[0, 6]) * 16 + 3]
    assert a.scale == 1.0 / 8.0


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_random_decode_structure(bs):
    c = W.random_decode(5, [1, 31, 32, 33, 100], num_heads=8, num_kv_heads=2, head_dim=64,
                        block_size=bs, dtype=W.BF16)
    kf = W.storage_to_f32(c.k_cache, c.dtype).reshape(-1, 2, 64)
    referenced = set()
    for i, n in enumerate(c.context_lens.tolist()):
        nblk = -(-n // bs)
        row = c.block_tables[i]
        assert (row[nblk:] == c.pad_block).all()
        for p in range(n - 1):
            s = int(row[p // bs]) * bs + p % bs
            referenced.add(s)
            assert np.isfinite(kf[s]).all()
        s_new = int(row[(n - 1) // bs]) * bs + (n - 1) % bs
        assert c.slot_mapping[i] == s_new
        assert np.isnan(kf[s_new]).all()          # poisoned until written
    unref = np.array(sorted(set(range(kf.shape[0])) - referenced))
    assert np.isnan(kf[unref]).all()
    # distinct physical blocks across sequences
    used = [b for i, n in enumerate(c.context_lens.tolist()) for b in c.block_tables[i, :-(-n // bs)]]
    assert len(used) == len(set(used))
    assert c.pad_block not in used


def test_prefill_slot_mapping_continues_prefix_block():
    c = W.random_prefill(9, [0, 5, 40], [7, 3, 33], block_size=16)
    assert c.query_start_loc.tolist() == [0, 7, 10, 43]
    r = 0
    for i, (p, t) in enumerate(zip([0, 5, 40], [7, 3, 33])):
        for j in range(t):
            pos = p + j
            assert c.slot_mapping[r] == int(c.block_tables[i, pos // 16]) * 16 + pos % 16
            r += 1
    assert c.context_lens.tolist() == [7, 8, 73]


def test_prefix_shared_groups_share_blocks():
    c = W.prefix_shared_decode(7, block_size=8, groups=2, per_group=3, shared_blocks=4, tail_high=20)
    t = c.block_tables
    for g in range(2):
        rows = t[g * 3:(g + 1) * 3, :4]
        assert (rows == rows[0]).all()
    assert not set(t[0, :4].tolist()) & set(t[3, :4].tolist())
    # private tails are not shared
    priv = []
    for i, n in enumerate(c.context_lens.tolist()):
        priv.extend(t[i, 4:-(-n // 8)].tolist())
    assert len(priv) == len(set(priv))
    assert c.unique_blocks() == 8 + len(priv)


def test_boost_scales_by_eight():
    c = W.random_decode(3, [300, 200], num_heads=8, num_kv_heads=2, head_dim=16, block_size=32,
                        dtype=W.BF16, boost_frac=0.05, poison=False)
    d = W.random_decode(3, [300, 200], num_heads=8, num_kv_heads=2, head_dim=16, block_size=32,
                        dtype=W.BF16, boost_frac=0.0, poison=False)
    kc = W.storage_to_f32(c.k_cache, c.dtype)
    kd = W.storage_to_f32(d.k_cache, d.dtype)
    ratio_rows = np.all((kc == kd) | (kc == 8 * kd), axis=-1)
    assert ratio_rows.all()
    boosted = np.any(kc != kd, axis=-1)
    frac = boosted.sum() / (500 * 2)
    assert 0.02 < frac < 0.09


def test_serving_trace_kv_depends_only_on_the_token_prefix():
    tr = W.serving_trace(seed=11, num_requests=4)
    a = tr.prompts[0]
    b = a[:30] + [a[30] + 1] + a[31:]
    ka, va, _ = tr.kv(a)
    kb, vb, _ = tr.kv(b)
    assert np.array_equal(ka[:30], kb[:30]) and np.array_equal(va[:30], vb[:30])
    assert not np.array_equal(ka[30:], kb[30:])  # every later position changes
    assert all(not np.array_equal(ka[i], kb[i]) for i in range(30, len(a)))
    # incremental extension equals the draw from scratch
    k1, v1, st = tr.kv(a[:17])
    k2, v2, _ = tr.kv(a, start=17, state=st)
    assert np.array_equal(np.concatenate([k1, k2]), ka) and np.array_equal(np.concatenate([v1, v2]), va)
    # even requests share the system prompt; queries differ by request
    assert tr.prompts[0][:64] == tr.prompts[2][:64]
    assert not np.array_equal(tr.q(0, 0, 1), tr.q(2, 0, 1))
    assert ka.dtype == np.uint16 and tr.q(1, 5, 3).shape == (3, tr.num_heads, tr.head_dim)


def test_separate_value_dim_case():
    """A value head dim of its own changes only the V side of a case: Q, K,
    the layout and the slots are those of the equal-dim case of the seed."""
    a = W.random_decode(41, [5, 40, 17], head_dim=128, block_size=8, dtype=W.BF16)
    b = W.random_decode(41, [5, 40, 17], head_dim=128, v_head_dim=64, block_size=8, dtype=W.BF16)
    assert b.v_head_dim == 64 and a.v_head_dim == 128
    assert b.v_cache.shape == b.k_cache.shape[:3] + (64,) and b.new_value.shape == (3, 2, 64)
    for f in ("q", "k_cache", "new_key", "slot_mapping", "block_tables", "context_lens"):
        x, y = getattr(a, f), getattr(b, f)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f
    assert b.scale == a.scale == 1.0 / np.sqrt(128)
    assert b.kv_bytes_logical() == 62 * 2 * (128 + 64) * 2
    # the new tokens' V rows are the pool rows at their slots, NaN until written
    vflat = b.v_cache.reshape(-1, 2, 64)
    assert np.isnan(W.storage_to_f32(vflat[b.slot_mapping], W.BF16)).all()
    c = W.random_prefill(42, [3, 0], [4, 9], head_dim=64, v_head_dim=128, block_size=16)
    assert c.v_cache.shape[3] == 128 and c.q.shape == (13, 8, 64)
