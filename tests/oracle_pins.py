"""Pins for the CPU oracle: facts fixed by the pages or by mathematics that
the oracle must reproduce.  Each ``pin_*`` takes an oracle module (the real
one, or a copy with a planted mistake) and raises ``AssertionError`` when
the oracle disagrees.

What pins what:

* ``pin_golden_slot_scatter``       - hand-derived slot scatter + gather (write, gather)
* ``pin_golden_attention``          - hand-worked outputs (scores, softmax, GQA, causal placement)
* ``pin_write_scatter``             - written slots equal inputs, all others untouched (write)
* ``pin_gather_any_permutation``    - paged == dense for any block permutation (gather)
* ``pin_decode_matches_sdpa``       - torch SDPA on the CPU, GQA by repeat_interleave (whole formula)
* ``pin_prefill_matches_sdpa``      - prefix-0 chunk == SDPA is_causal (whole formula, mask)
* ``pin_chunked_equals_full``       - a chunk after its prefix == the same rows of a full prefill (causal placement)
* ``pin_causal_independence``       - later tokens cannot change earlier outputs (mask)
* ``pin_softmax_rows``              - weights >= 0, masked weights exactly 0, rows sum to 1 (normalisation)
* ``pin_single_token``              - context of 1 returns that token's V exactly
* ``pin_index_probe``               - one-hot scores pick exactly V[p*] at every position (indexing)
* ``pin_uniform_query``             - q = 0 gives the mean of the visible V (closed form)
* ``pin_leak_probe``                - a huge masked score never leaks (mask boundary)
* ``pin_brute_force``               - scalar loops with math.exp on tiny inputs
* ``pin_fp32_close_to_fp64``        - the float32 mode stays within 1e-5 of float64
* ``pin_decode_is_prefill_of_one``  - a chunk of one token is the decode step
* ``pin_empty_context``             - a context of 0 tokens gives zeros
* ``pin_separate_value_dim``        - value head dim != key head dim: SDPA with a narrower/wider V (write, decode, prefill)
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# helpers that build inputs without using the oracle's indexing formula
# --------------------------------------------------------------------------

def _blocks_from_dense(dense, block_size, rng, num_blocks=None, fill=np.nan):
    """Cut a dense ``[n, H, D]`` sequence into blocks (reshape, zero-padded
    tail replaced by ``fill``) and place them at random distinct pool
    positions.  Returns ``(pool, table)``."""
    n, H, D = dense.shape
    nblk = -(-n // block_size)
    padded = np.full((nblk * block_size, H, D), fill, dtype=dense.dtype)
    padded[:n] = dense
    blocks = padded.reshape(nblk, block_size, H, D)
    if num_blocks is None:
        num_blocks = nblk + 3
    pool = np.full((num_blocks, block_size, H, D), fill, dtype=dense.dtype)
    table = rng.permutation(num_blocks)[:nblk]
    pool[table] = blocks
    return pool, table.astype(np.int32)


def _sequences_into_pool(denses_k, denses_v, block_size, rng, extra=3):
    """Several sequences into one pool, each block at a random place."""
    nblks = [-(-d.shape[0] // block_size) for d in denses_k]
    total = sum(nblks) + extra
    H, D = denses_k[0].shape[1:]
    Dv = denses_v[0].shape[2]
    kpool = np.full((total, block_size, H, D), np.nan)
    vpool = np.full((total, block_size, H, Dv), np.nan)
    perm = rng.permutation(total)
    tables = np.full((len(denses_k), max(nblks)), perm[-1], dtype=np.int32)
    c = 0
    for i, (dk, dv) in enumerate(zip(denses_k, denses_v)):
        n = dk.shape[0]
        ids = perm[c:c + nblks[i]]
        c += nblks[i]
        for dense, pool in ((dk, kpool), (dv, vpool)):
            width = dense.shape[2]
            padded = np.full((nblks[i] * block_size, H, width), np.nan)
            padded[:n] = dense
            pool[ids] = padded.reshape(nblks[i], block_size, H, width)
        tables[i, :nblks[i]] = ids
    return kpool, vpool, tables


def _torch():
    import torch
    return torch


def _sdpa(q, k, v, scale, causal):
    """torch SDPA on the CPU in float64; q [Tq, Hq, D], k [n, Hkv, D],
    v [n, Hkv, Dv]; GQA by repeating each kv head over its group of query
    heads."""
    torch = _torch()
    Hq, Hkv = q.shape[1], k.shape[1]
    tq = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).permute(1, 0, 2)
    tv = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).permute(1, 0, 2)
    tk = tk.repeat_interleave(Hq // Hkv, dim=0)[None].contiguous()
    tv = tv.repeat_interleave(Hq // Hkv, dim=0)[None].contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(tq.contiguous(), tk, tv, is_causal=causal, scale=scale)
    return out[0].permute(1, 0, 2).numpy()


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_golden_slot_scatter(orc):
    g = json.load(open(os.path.join(GOLDEN, "slot_scatter_example.json")))
    shape = (g["num_blocks"], g["block_size"], g["num_kv_heads"], g["head_dim"])
    kpool = np.full(shape, np.nan)
    vpool = np.full(shape, np.nan)
    key = np.array(g["key"], dtype=np.float64).reshape(-1, 1, 1)
    val = np.array(g["value"], dtype=np.float64).reshape(-1, 1, 1)
    k2, v2 = orc.kv_cache_write(kpool, vpool, key, val, np.array(g["slot_mapping"]))
    for got, exp in ((k2, g["expected_key_pool_flat"]), (v2, g["expected_value_pool_flat"])):
        flat = got.reshape(-1)
        for i, e in enumerate(exp):
            if e is None:
                assert np.isnan(flat[i]), f"slot {i} should be untouched"
            else:
                assert flat[i] == e, f"slot {i}: {flat[i]} != {e}"
    dense = orc.gather_sequence(k2, np.array(g["block_table"]), len(g["positions"]))
    assert np.array_equal(dense.reshape(-1), np.array(g["key"], dtype=np.float64))


def pin_golden_attention(orc):
    g = json.load(open(os.path.join(GOLDEN, "attention_hand_examples.json")))
    rng = np.random.default_rng(7)
    for ex in g["examples"]:
        q = np.array(ex["q"], dtype=np.float64)
        k = np.array(ex["k"], dtype=np.float64)
        v = np.array(ex["v"], dtype=np.float64)
        exp = np.array(ex["expected"], dtype=np.float64)
        n = k.shape[0]
        # dense call
        if ex["kind"] == "decode":
            pos = np.array([n - 1])
        else:
            pos = ex["prefix_len"] + np.arange(q.shape[0])
        dense = orc.attention(q, k, v, ex["scale"], pos)
        assert np.allclose(dense, exp, rtol=0, atol=1e-12), (ex["name"], dense, exp)
        # the same through a paged pool with 2-token blocks at shuffled places
        kpool, vpool, tables = _sequences_into_pool([k], [v], 2, rng)
        ctx = np.array([n], dtype=np.int32)
        if ex["kind"] == "decode":
            got = orc.paged_decode(q, kpool, vpool, tables, ctx, ex["scale"])
        else:
            qsl = np.array([0, q.shape[0]], dtype=np.int32)
            got = orc.paged_prefill(q, qsl, kpool, vpool, tables, ctx, ex["scale"])
        assert np.allclose(got, exp, rtol=0, atol=1e-12), (ex["name"], got, exp)


def pin_write_scatter(orc):
    rng = np.random.default_rng(11)
    nb, bs, H, D = 9, 4, 3, 5
    kpool = np.full((nb, bs, H, D), np.nan, dtype=np.float32)
    vpool = np.full((nb, bs, H, D), np.nan, dtype=np.float32)
    T = 13
    # never the pool's last slot, which index -1 would alias
    slots = rng.permutation(nb * bs - 1)[:T].astype(np.int64)
    slots[4] = -1                                    # skipped tokens
    slots[T - 1] = -1
    key = rng.standard_normal((T, H, D)).astype(np.float32)
    val = rng.standard_normal((T, H, D)).astype(np.float32)
    k2, v2 = orc.kv_cache_write(kpool, vpool, key, val, slots)
    kf = k2.reshape(nb * bs, H, D)
    vf = v2.reshape(nb * bs, H, D)
    written = np.zeros(nb * bs, bool)
    for t, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        written[s] = True
        assert np.array_equal(kf[s].view(np.uint32), key[t].view(np.uint32)), f"token {t}"
        assert np.array_equal(vf[s].view(np.uint32), val[t].view(np.uint32)), f"token {t}"
    assert np.isnan(kf[~written]).all() and np.isnan(vf[~written]).all(), "untouched slots changed"
    assert np.isnan(kpool).all(), "input cache modified in place"


def pin_gather_any_permutation(orc):
    rng = np.random.default_rng(12)
    for bs in (1, 3, 8):
        n, Hq, Hkv, D = 29, 6, 3, 4
        k = rng.standard_normal((n, Hkv, D))
        v = rng.standard_normal((n, Hkv, D))
        q = rng.standard_normal((1, Hq, D))
        ref = orc.attention(q, k, v, 0.37, np.array([n - 1]))
        outs = []
        for _ in range(3):
            kpool, table = _blocks_from_dense(k, bs, rng, num_blocks=-(-n // bs) + 5)
            vpool = np.full_like(kpool, np.nan)
            nblk = -(-n // bs)
            padded = np.full((nblk * bs, Hkv, D), np.nan)
            padded[:n] = v
            vpool[table] = padded.reshape(nblk, bs, Hkv, D)
            assert np.array_equal(orc.gather_sequence(kpool, table, n), k)
            assert np.array_equal(orc.gather_sequence(vpool, table, n), v)
            out = orc.paged_decode(q, kpool, vpool, table[None], np.array([n]), 0.37)
            outs.append(out)
            assert np.array_equal(out, ref), "paged != dense"
        assert all(np.array_equal(outs[0], o) for o in outs[1:])


def pin_decode_matches_sdpa(orc):
    rng = np.random.default_rng(13)
    for (Hq, Hkv, D) in ((8, 2, 16), (4, 4, 8), (6, 1, 5)):
        lens = [1, 7, 33]
        ks = [rng.standard_normal((n, Hkv, D)) for n in lens]
        vs = [rng.standard_normal((n, Hkv, D)) for n in lens]
        q = rng.standard_normal((len(lens), Hq, D))
        kpool, vpool, tables = _sequences_into_pool(ks, vs, 4, rng)
        scale = 1.0 / math.sqrt(D)
        out = orc.paged_decode(q, kpool, vpool, tables, np.array(lens), scale)
        for i in range(len(lens)):
            ref = _sdpa(q[i:i + 1], ks[i], vs[i], scale, causal=False)
            assert np.allclose(out[i:i + 1], ref, rtol=0, atol=1e-12), f"seq {i}"


def pin_prefill_matches_sdpa(orc):
    rng = np.random.default_rng(14)
    Hq, Hkv, D = 8, 2, 16
    lens = [1, 5, 40]
    ks = [rng.standard_normal((n, Hkv, D)) for n in lens]
    vs = [rng.standard_normal((n, Hkv, D)) for n in lens]
    qs = [rng.standard_normal((n, Hq, D)) for n in lens]
    kpool, vpool, tables = _sequences_into_pool(ks, vs, 8, rng)
    q = np.concatenate(qs)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = orc.paged_prefill(q, qsl, kpool, vpool, tables, np.array(lens), 0.25)
    for i, n in enumerate(lens):
        ref = _sdpa(qs[i], ks[i], vs[i], 0.25, causal=True)
        assert np.allclose(out[qsl[i]:qsl[i + 1]], ref, rtol=0, atol=1e-12), f"seq {i}"


def pin_chunked_equals_full(orc):
    """Rows of a chunk processed after its cached prefix equal the same rows
    of the whole sequence processed as one causal chunk from position 0."""
    rng = np.random.default_rng(15)
    Hq, Hkv, D, n = 4, 2, 8, 37
    k = rng.standard_normal((n, Hkv, D))
    v = rng.standard_normal((n, Hkv, D))
    q = rng.standard_normal((n, Hq, D))
    kpool, vpool, tables = _sequences_into_pool([k], [v], 4, rng)
    ctx = np.array([n])
    full = orc.paged_prefill(q, np.array([0, n]), kpool, vpool, tables, ctx, 0.3)
    for c in (1, 2, 11, n):
        part = orc.paged_prefill(q[n - c:], np.array([0, c]), kpool, vpool, tables, ctx, 0.3)
        assert np.allclose(part, full[n - c:], rtol=0, atol=1e-12), f"chunk {c}"


def pin_causal_independence(orc):
    rng = np.random.default_rng(16)
    Hq, Hkv, D, n, prefix = 4, 2, 8, 30, 12
    k = rng.standard_normal((n, Hkv, D))
    v = rng.standard_normal((n, Hkv, D))
    q = rng.standard_normal((n - prefix, Hq, D))
    kpool, vpool, tables = _sequences_into_pool([k], [v], 4, rng)
    qsl = np.array([0, n - prefix])
    base = orc.paged_prefill(q, qsl, kpool, vpool, tables, np.array([n]), 0.3)
    for t in (0, 5, n - prefix - 2):
        pos = prefix + t
        k2, v2, q2 = k.copy(), v.copy(), q.copy()
        k2[pos + 1:] = rng.standard_normal(k2[pos + 1:].shape) * 10
        v2[pos + 1:] = rng.standard_normal(v2[pos + 1:].shape) * 10
        q2[t + 1:] = rng.standard_normal(q2[t + 1:].shape) * 10
        kp2, vp2, tb2 = _sequences_into_pool([k2], [v2], 4, rng)
        out = orc.paged_prefill(q2, qsl, kp2, vp2, tb2, np.array([n]), 0.3)
        assert np.allclose(out[:t + 1], base[:t + 1], rtol=0, atol=1e-13), f"row {t} saw later tokens"
        assert not np.allclose(out[t + 1:], base[t + 1:]), "perturbation had no effect"


def pin_softmax_rows(orc):
    rng = np.random.default_rng(17)
    for n in (1, 2, 50, 700):
        D = 16
        q = rng.standard_normal((9, D)) * 3
        k = rng.standard_normal((n, D)) * 3
        pos = rng.integers(0, n, size=9)
        w = orc.attention_weights(q, k, 0.25, pos)
        assert (w >= 0).all()
        for t in range(9):
            assert (w[t, pos[t] + 1:] == 0).all(), "masked weight not exactly 0"
            assert abs(float(np.sum(w[t], dtype=np.float64)) - 1.0) <= (n + 1) * 2.0 ** -52
        # large logits: no overflow, still normalised
        w = orc.attention_weights(q * 100, k * 100, 1.0, pos)
        assert np.isfinite(w).all()
        assert np.allclose(w.sum(1), 1.0, atol=1e-12)


def pin_single_token(orc):
    rng = np.random.default_rng(18)
    Hq, Hkv, D = 8, 2, 16
    k = rng.standard_normal((1, Hkv, D))
    v = rng.standard_normal((1, Hkv, D))
    q = rng.standard_normal((1, Hq, D)) * 50
    kpool, vpool, tables = _sequences_into_pool([k], [v], 16, rng)
    out = orc.paged_decode(q, kpool, vpool, tables, np.array([1]), 0.3)
    for h in range(Hq):
        assert np.array_equal(out[0, h], v[0, h // (Hq // Hkv)]), f"head {h}"


def pin_index_probe(orc):
    """Keys with a zero first component everywhere except position p*, and
    q = c e0: every score is exactly 0 but the target's, which is so large
    that every other weight underflows to exactly 0.  The output is then
    V[p*] exactly, for every p*."""
    rng = np.random.default_rng(19)
    Hq, Hkv, D, n, bs = 4, 2, 8, 23, 4
    c = 100.0                                    # c^2 * scale = 2500 >> 745
    v = rng.standard_normal((n, Hkv, D))
    for target in range(n):
        k = rng.standard_normal((n, Hkv, D))
        k[:, :, 0] = 0.0
        k[target, :, :] = 0.0
        k[target, :, 0] = c
        q = np.zeros((1, Hq, D))
        q[0, :, 0] = c
        kpool, vpool, tables = _sequences_into_pool([k], [v], bs, rng)
        out = orc.paged_decode(q, kpool, vpool, tables, np.array([n]), 0.25)
        for h in range(Hq):
            assert np.array_equal(out[0, h], v[target, h // (Hq // Hkv)]), f"target {target} head {h}"


def pin_uniform_query(orc):
    rng = np.random.default_rng(20)
    Hq, Hkv, D = 6, 3, 8
    lens = [3, 17]
    ks = [rng.standard_normal((n, Hkv, D)) for n in lens]
    vs = [rng.standard_normal((n, Hkv, D)) for n in lens]
    kpool, vpool, tables = _sequences_into_pool(ks, vs, 4, rng)
    q = np.zeros((2, Hq, D))
    out = orc.paged_decode(q, kpool, vpool, tables, np.array(lens), 0.5)
    for i, n in enumerate(lens):
        for h in range(Hq):
            mean = vs[i][:, h // 2].mean(axis=0)
            assert np.allclose(out[i, h], mean, rtol=0, atol=1e-14)
    # prefill: query t sees prefix + t + 1 keys
    n, prefix = 17, 9
    qp = np.zeros((n - prefix, Hq, D))
    kp, vp, tb = _sequences_into_pool([ks[1]], [vs[1]], 4, rng)
    outp = orc.paged_prefill(qp, np.array([0, n - prefix]), kp, vp, tb, np.array([n]), 0.5)
    for t in range(n - prefix):
        for h in range(Hq):
            mean = vs[1][:prefix + t + 1, h // 2].mean(axis=0)
            assert np.allclose(outp[t, h], mean, rtol=0, atol=1e-14), f"row {t}"


def pin_leak_probe(orc):
    """For each chunk row t, an allowed target key gets score gap 2500 and
    the first masked key (position prefix + t + 1) gets 5000.  A mask that
    holds returns V[target] exactly; a leak returns V[leak]."""
    rng = np.random.default_rng(21)
    Hq, Hkv, D, n, prefix = 4, 2, 8, 20, 9
    v = rng.standard_normal((n, Hkv, D))
    for t in range(n - prefix - 1):
        pos = prefix + t
        target = int(rng.integers(0, pos + 1))
        k = rng.standard_normal((n, Hkv, D))
        k[:, :, 0] = 0.0
        k[target, :, 0] = 100.0
        k[pos + 1, :, 0] = 200.0
        q = np.zeros((n - prefix, Hq, D))
        q[:, :, 0] = 100.0
        kpool, vpool, tables = _sequences_into_pool([k], [v], 4, rng)
        out = orc.paged_prefill(q, np.array([0, n - prefix]), kpool, vpool, tables, np.array([n]), 0.25)
        for h in range(Hq):
            assert np.array_equal(out[t, h], v[target, h // 2]), f"row {t} head {h} leaked"


def pin_brute_force(orc):
    """Scalar loops with math.exp, no arrays, on tiny inputs."""
    rng = np.random.default_rng(22)
    Hq, Hkv, D = 4, 2, 3
    lens, qlens = [4, 6], [2, 3]
    ks = [rng.standard_normal((n, Hkv, D)) for n in lens]
    vs = [rng.standard_normal((n, Hkv, D)) for n in lens]
    qs = [rng.standard_normal((m, Hq, D)) for m in qlens]
    kpool, vpool, tables = _sequences_into_pool(ks, vs, 2, rng)
    q = np.concatenate(qs)
    qsl = np.array([0, 2, 5])
    scale = 0.7
    out = orc.paged_prefill(q, qsl, kpool, vpool, tables, np.array(lens), scale)
    for i, (n, m) in enumerate(zip(lens, qlens)):
        for t in range(m):
            pos = n - m + t
            for h in range(Hq):
                g = h // (Hq // Hkv)
                s = [sum(float(qs[i][t, h, d]) * float(ks[i][p, g, d]) for d in range(D)) * scale
                     for p in range(pos + 1)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = math.fsum(e)
                for d in range(D):
                    ref = math.fsum(e[p] / tot * float(vs[i][p, g, d]) for p in range(pos + 1))
                    got = out[qsl[i] + t, h, d]
                    assert abs(got - ref) <= 1e-12, (i, t, h, d, got, ref)


def pin_fp32_close_to_fp64(orc):
    rng = np.random.default_rng(23)
    Hq, Hkv, D = 8, 2, 64
    lens = [100, 37, 1]
    ks = [rng.standard_normal((n, Hkv, D)) for n in lens]
    vs = [rng.standard_normal((n, Hkv, D)) for n in lens]
    kpool, vpool, tables = _sequences_into_pool(ks, vs, 16, rng)
    q = rng.standard_normal((3, Hq, D))
    o64 = orc.paged_decode(q, kpool, vpool, tables, np.array(lens), 0.125)
    o32 = orc.paged_decode(q.astype(np.float32), kpool.astype(np.float32), vpool.astype(np.float32),
                           tables, np.array(lens), 0.125, acc_dtype=np.float32)
    assert o32.dtype == np.float32
    assert np.abs(o32 - o64).max() <= 1e-5


def pin_decode_is_prefill_of_one(orc):
    rng = np.random.default_rng(24)
    Hq, Hkv, D = 8, 4, 8
    lens = [5, 12, 31]
    ks = [rng.standard_normal((n, Hkv, D)) for n in lens]
    vs = [rng.standard_normal((n, Hkv, D)) for n in lens]
    kpool, vpool, tables = _sequences_into_pool(ks, vs, 4, rng)
    q = rng.standard_normal((3, Hq, D))
    dec = orc.paged_decode(q, kpool, vpool, tables, np.array(lens), 0.3)
    pre = orc.paged_prefill(q, np.arange(4), kpool, vpool, tables, np.array(lens), 0.3)
    assert np.array_equal(dec, pre)
    # and the last row of a full causal prefill
    for i, n in enumerate(lens):
        qf = rng.standard_normal((n, Hq, D))
        qf[-1] = q[i]
        full = orc.paged_prefill(qf, np.array([0, n]), kpool, vpool, tables[i:i + 1], np.array([n]), 0.3)
        assert np.allclose(full[-1], dec[i], rtol=0, atol=1e-13)


def pin_empty_context(orc):
    """A sequence with no context token attends to nothing: its output is
    zeros (no NaN), and its neighbours in the batch are unaffected."""
    rng = np.random.default_rng(25)
    Hq, Hkv, D = 4, 2, 8
    lens = [0, 6]
    ks = [rng.standard_normal((max(n, 1), Hkv, D)) for n in lens]
    vs = [rng.standard_normal((max(n, 1), Hkv, D)) for n in lens]
    kpool, vpool, tables = _sequences_into_pool(ks, vs, 4, rng)
    q = rng.standard_normal((2, Hq, D))
    out = orc.paged_decode(q, kpool, vpool, tables, np.array(lens), 0.3)
    assert np.array_equal(out[0], np.zeros((Hq, D)))
    alone = orc.paged_decode(q[1:], kpool, vpool, tables[1:], np.array(lens[1:]), 0.3)
    assert np.array_equal(out[1], alone[0])


def pin_separate_value_dim(orc):
    """Key and value head dims differ (TensorSharp, section 4.1: separate
    key and value lengths): the write stores each row at its own width and
    decode / prefill agree with SDPA, which takes a V of any width."""
    rng = np.random.default_rng(23)
    Hq, Hkv = 4, 2
    for D, Dv in ((8, 3), (4, 12)):
        # write: rows of both widths land in their slots, nothing else moves
        kpool = np.full((5, 2, Hkv, D), np.nan)
        vpool = np.full((5, 2, Hkv, Dv), np.nan)
        key = rng.standard_normal((3, Hkv, D))
        val = rng.standard_normal((3, Hkv, Dv))
        k2, v2 = orc.kv_cache_write(kpool, vpool, key, val, np.array([7, -1, 2]))
        assert np.array_equal(k2[3, 1], key[0]) and np.array_equal(v2[3, 1], val[0])
        assert np.array_equal(k2[1, 0], key[2]) and np.array_equal(v2[1, 0], val[2])
        assert np.isnan(k2).sum() == k2.size - 2 * Hkv * D and np.isnan(v2).sum() == v2.size - 2 * Hkv * Dv
        # decode and prefill against SDPA
        lens = [1, 6, 19]
        ks = [rng.standard_normal((n, Hkv, D)) for n in lens]
        vs = [rng.standard_normal((n, Hkv, Dv)) for n in lens]
        kpool, vpool, tables = _sequences_into_pool(ks, vs, 4, rng)
        q = rng.standard_normal((len(lens), Hq, D))
        out = orc.paged_decode(q, kpool, vpool, tables, np.array(lens), 0.4)
        assert out.shape == (len(lens), Hq, Dv)
        for i in range(len(lens)):
            ref = _sdpa(q[i:i + 1], ks[i], vs[i], 0.4, causal=False)
            assert np.allclose(out[i:i + 1], ref, rtol=0, atol=1e-12), f"decode seq {i}"
        qs = [rng.standard_normal((n, Hq, D)) for n in lens]
        qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        out = orc.paged_prefill(np.concatenate(qs), qsl, kpool, vpool, tables, np.array(lens), 0.4)
        assert out.shape == (sum(lens), Hq, Dv)
        for i in range(len(lens)):
            ref = _sdpa(qs[i], ks[i], vs[i], 0.4, causal=True)
            assert np.allclose(out[qsl[i]:qsl[i + 1]], ref, rtol=0, atol=1e-12), f"prefill seq {i}"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
