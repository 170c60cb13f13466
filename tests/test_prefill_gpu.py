"""pa_prefill_chunk on the GPU against the CPU oracle: the 8 x 512-token
chunked-prefill workload at full size, a sweep of shapes and ragged
chunks, bit-exact causal-boundary probes, and consistency with decode."""

import numpy as np
import pytest

import workloads as W
from gpu_util import DeviceCase, assert_close, log, oracle_decode, oracle_prefill, to_host_bits, to_host_f32, torch

pytestmark = pytest.mark.gpu


def _run(case, max_context_len=None):
    dev = DeviceCase(case)
    dev.write()
    out = dev.prefill(max_context_len=max_context_len)
    torch().cuda.synchronize()
    return dev, to_host_f32(out, case.dtype)


@pytest.mark.parametrize("block_size", [32, 16, 8])
def test_chunked_prefill_full(block_size):
    case = W.chunked_prefill(block_size=block_size)
    log(f"chunked prefill 8 x 512 over prefixes {(case.context_lens - 512).tolist()}, block size {block_size}")
    _, got = _run(case)
    ref = oracle_prefill(case)
    mx, mean = assert_close(got, ref, W.BF16, f"chunked prefill bs{block_size}")
    print(f"chunked prefill bs{block_size}: max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_chunked_prefill_eight_heads_per_kv_head_full():
    """The 8 x 512 chunk workload at 64 query over 8 kv heads: 16 query tiles
    of 32 per sequence, 128 (sequence, query tile) items per kv head, more
    than the longest-first ranking takes (the plain dispatch order)."""
    case = W.chunked_prefill(num_heads=64)
    log("chunked prefill 8 x 512, 64 q / 8 kv heads")
    _, got = _run(case)
    ref = oracle_prefill(case)
    mx, mean = assert_close(got, ref, W.BF16, "chunked prefill 64q")
    print(f"chunked prefill 64q: max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_mixed_step_full_size():
    """One full-size mixed step as the mixed scheduler policy issues it: 64
    decode rows (one token each, contexts U[128, 4096]) and prompt chunks
    (seven of 512 tokens and one of 448 over prefixes U[0, 2048]) in a single
    4096-token prefill launch: 72 sequences (two lanes' worth of sequences
    in the work-groups' cost ranking), 1,152 (sequence, 32-query tile) items
    per kv head."""
    rng = np.random.default_rng(4242)
    dec_ctx = rng.integers(128, 4097, size=64)
    pro_prefix = rng.integers(0, 2049, size=8)
    prefixes = [int(c) - 1 for c in dec_ctx] + [int(p) for p in pro_prefix]
    qlens = [1] * 64 + [512] * 7 + [448]
    assert sum(qlens) == 4096
    case = W.random_prefill(4243, prefixes, qlens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=32,
                            dtype=W.BF16)
    log("mixed step: 64 decode rows + 8 prompt chunks, 4096 tokens")
    _, got = _run(case)
    ref = oracle_prefill(case)
    mx, mean = assert_close(got, ref, W.BF16, "mixed step")
    print(f"mixed step: max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("scale", [0.37, 0.0, -0.05, 1.0 / 64])
def test_prefill_other_scales(scale):
    """Scales other than 1/sqrt(head_dim), zero and negative included: the
    scale multiplies every q.k, so a negative one reverses the order of the
    scores and zero gives uniform weights."""
    case = W.random_prefill(91, [0, 70, 300, 5], [100, 64, 130, 1], num_heads=32, num_kv_heads=8, head_dim=128,
                            block_size=16, dtype=W.BF16)
    case.scale = float(scale)
    log(f"prefill scale {scale}")
    _, got = _run(case)
    ref = oracle_prefill(case)
    assert_close(got, ref, W.BF16, f"scale {scale}")


PREFIXES = [0, 0, 5, 31, 32, 64, 100, 257]
QLENS = [1, 64, 33, 1, 32, 95, 128, 200]


@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_prefill_shapes(head_dim, group):
    hkv = 2
    for bs in (8, 16, 32):
        case = W.random_prefill(300 + 10 * group + bs + head_dim, PREFIXES, QLENS, num_heads=hkv * group,
                                num_kv_heads=hkv, head_dim=head_dim, block_size=bs, dtype=W.BF16,
                                extra_table_cols=2)
        log(f"prefill D={head_dim} G={group} bs={bs}")
        _, got = _run(case)
        ref = oracle_prefill(case)
        assert_close(got, ref, W.BF16, f"D{head_dim} G{group} bs{bs}")


@pytest.mark.parametrize("dims", [(128, 64), (64, 128)])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_prefill_separate_value_dim(dims, group):
    """Key head dim D, value head dim Dv != D: outputs are [Tq, H, Dv]."""
    D, Dv = dims
    hkv = 2
    for bs in (8, 16, 32):
        case = W.random_prefill(800 + 10 * group + bs + D, PREFIXES, QLENS, num_heads=hkv * group,
                                num_kv_heads=hkv, head_dim=D, v_head_dim=Dv, block_size=bs, dtype=W.BF16,
                                extra_table_cols=2)
        log(f"prefill D={D} Dv={Dv} G={group} bs={bs}")
        _, got = _run(case)
        ref = oracle_prefill(case)
        assert ref.shape == (sum(QLENS), hkv * group, Dv)
        assert_close(got, ref, W.BF16, f"D{D} Dv{Dv} G{group} bs{bs}")


def test_prefill_empty_and_single_token_chunks():
    case = W.random_prefill(7, [10, 0, 40, 3], [0, 1, 0, 5], num_heads=8, num_kv_heads=2, head_dim=128,
                            block_size=16, dtype=W.BF16)
    log("prefill with empty chunks")
    _, got = _run(case)
    ref = oracle_prefill(case)
    assert_close(got, ref, W.BF16, "empty chunks")


def test_prefill_chunk_of_one_matches_decode():
    """A chunk of one token per sequence is a decode step."""
    case = W.random_prefill(17, [0, 40, 511, 1000], [1, 1, 1, 1], num_heads=32, num_kv_heads=8,
                            head_dim=128, block_size=32, dtype=W.BF16)
    log("prefill q_len=1 vs decode")
    dev, got = _run(case)
    import paged_attention_kv_cache_amd as P
    dec = P.pa_decode(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens, case.scale,
                      case.max_context_len, 0)
    torch().cuda.synchronize()
    got_dec = to_host_f32(dec, W.BF16)
    assert_close(got, got_dec, W.BF16, "prefill vs decode")
    ref = oracle_prefill(case)
    assert_close(got, ref, W.BF16, "prefill q_len=1")


def test_prefill_no_cross_sequence_leakage():
    import paged_attention_kv_cache_amd as P
    t = torch()
    case = W.random_prefill(23, [0, 300, 77], [100, 64, 130], num_heads=32, num_kv_heads=8, head_dim=128,
                            block_size=16, dtype=W.BF16)
    dev = DeviceCase(case)
    dev.write()
    log("prefill batch for leakage check")
    full = to_host_bits(dev.prefill())
    qsl = case.query_start_loc
    for i in range(case.num_seqs):
        r0, r1 = int(qsl[i]), int(qsl[i + 1])
        log(f"prefill sequence {i} alone")
        one = P.pa_prefill_chunk(dev.q[r0:r1].contiguous(), t.tensor([0, r1 - r0], dtype=t.int32, device="cuda"),
                                 dev.k_cache, dev.v_cache, dev.block_tables[i:i + 1].contiguous(),
                                 dev.context_lens[i:i + 1].contiguous(), case.scale, r1 - r0,
                                 case.max_context_len)
        t.cuda.synchronize()
        assert np.array_equal(to_host_bits(one), full[r0:r1]), f"sequence {i}"


def _bf16(x):
    return W.f32_to_bf16_bits(np.float32(x).reshape(1))[0]


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_prefill_causal_boundary_probe(bs):
    """Every query is 40 e0; every key has a zero first component except a
    target key at position 3 (visible to every chunk row: score gap 141
    nats) and, in sequence i, a key 80 e0 at position prefix + t_i + 1 (four
    times the target's score).  Rows t <= t_i must return V[3] bit for bit
    (the big key is above their diagonal), rows t > t_i must return the big
    key's V bit for bit (it is visible to them and dominates)."""
    prefix, q_len = 40, 200
    probe_rows = [0, 30, 31, 32, 63, 64, 100, 127, 128, q_len - 2]
    S = len(probe_rows)
    case = W.random_prefill(60 + bs, [prefix] * S, [q_len] * S, num_heads=32, num_kv_heads=8, head_dim=128,
                            block_size=bs, dtype=W.BF16, poison=False)
    c40, c80, zero = _bf16(40.0), _bf16(80.0), np.uint16(0)
    nb = case.num_blocks
    kflat = case.k_cache.reshape(nb * bs, 8, 128)
    kflat[case.slot_mapping] = case.new_key
    ctx = prefix + q_len
    for i, ti in enumerate(probe_rows):
        row = case.block_tables[i]
        for p in range(ctx):
            s = int(row[p // bs]) * bs + p % bs
            kflat[s, :, 0] = zero
            if p == 3:
                kflat[s] = zero
                kflat[s, :, 0] = c40
            if p == prefix + ti + 1:
                kflat[s] = zero
                kflat[s, :, 0] = c80
    case.new_key = kflat[case.slot_mapping].copy()
    case.q[:] = zero
    case.q[:, :, 0] = c40
    log(f"prefill causal probe bs={bs}")
    _, got = _run(case)
    vflat = W.storage_to_f32(case.v_cache, W.BF16).reshape(-1, 8, 128)
    vnew = W.storage_to_f32(case.new_value, W.BF16)
    qsl = case.query_start_loc
    for i, ti in enumerate(probe_rows):
        row = case.block_tables[i]
        s3 = int(row[3 // bs]) * bs + 3 % bs
        v_target = vflat[s3]
        big = prefix + ti + 1
        v_big = vnew[int(qsl[i]) + (big - prefix)]       # the big key is one of the chunk's tokens
        for t in range(q_len):
            exp = np.repeat(v_target if t <= ti else v_big, 4, axis=0)
            assert np.array_equal(got[int(qsl[i]) + t], exp), f"bs{bs} seq {i} (t_i={ti}) row {t}"


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("group", [1, 4, 8])
def test_prefill_fp32(dims, group):
    """fp32 chunked prefill: each packed row as a single-pass decode over
    its own causal prefix, within the fp32 tolerance of the oracle."""
    D, Dv = dims
    hkv = 2
    for bs in (8, 16, 32):
        case = W.random_prefill(1300 + 10 * group + bs + D + Dv, PREFIXES, QLENS, num_heads=hkv * group,
                                num_kv_heads=hkv, head_dim=D, v_head_dim=Dv, block_size=bs, dtype=W.F32,
                                extra_table_cols=2)
        log(f"fp32 prefill D={D} Dv={Dv} G={group} bs={bs}")
        _, got = _run(case)
        ref = oracle_prefill(case)
        assert_close(got, ref, W.F32, f"fp32 D{D} Dv{Dv} G{group} bs{bs}")


def test_prefill_fp32_rows_outside_sequences_untouched():
    """Rows past the last sequence's chunk keep their contents; an empty
    chunk writes nothing; the rows of the other sequences match the oracle."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    case = W.random_prefill(77, [10, 0, 40, 3], [0, 1, 0, 5], num_heads=8, num_kv_heads=2, head_dim=64,
                            block_size=16, dtype=W.F32)
    dev = DeviceCase(case)
    dev.write()
    Tq = int(case.query_start_loc[-1])
    q = t.cat([dev.q, t.zeros((3,) + tuple(dev.q.shape[1:]), dtype=dev.q.dtype, device="cuda")])
    out = t.full((Tq + 3,) + tuple(dev.q.shape[1:]), 7.0, dtype=dev.q.dtype, device="cuda")
    log("fp32 prefill with trailing unowned rows")
    P.pa_prefill_chunk(q, dev.query_start_loc, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                       case.scale, case.max_query_len, case.max_context_len, out=out)
    t.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[Tq:] == 7.0).all(), "rows outside every sequence were written"
    assert_close(got[:Tq], oracle_prefill(case), W.F32, "owned rows")


@pytest.mark.parametrize("seed", range(24))
def test_prefill_random_shapes(seed):
    """Seeded random chunked-prefill shapes against the oracle: query heads
    per kv head, kv heads, key and value head dims, block size, 1 to 10
    sequences with cached prefixes of 0 to ~1,500 tokens and chunks of 0 to
    ~300 new tokens (some of one token, some empty), and the storage type
    (one seed in four in fp32)."""
    rng = np.random.default_rng(7700 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 3, 5, 8]))
    D, Dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32]))
    dtype = W.F32 if seed % 4 == 3 else W.BF16
    S = int(rng.integers(1, 11))
    prefixes = rng.integers(0, 1500, size=S).tolist()
    qlens = rng.integers(0, 300, size=S).tolist()
    for i in rng.choice(S, size=min(S, 2), replace=False):
        qlens[int(i)] = int(rng.choice([0, 1, 31, 32, 33]))
        prefixes[int(i)] = int(rng.choice([0, bs - 1, bs, prefixes[int(i)]]))
    case = W.random_prefill(7800 + seed, prefixes, qlens, num_heads=hkv * G, num_kv_heads=hkv, head_dim=D,
                            v_head_dim=Dv, block_size=bs, dtype=dtype, extra_table_cols=1)
    what = f"seed {seed} {dtype} G{G} hkv{hkv} D{D} Dv{Dv} bs{bs} prefixes {prefixes} chunks {qlens}"
    log(what)
    _, got = _run(case)
    ref = oracle_prefill(case)
    assert ref.shape == (sum(qlens), hkv * G, Dv)
    assert_close(got, ref, dtype, what)


@pytest.mark.parametrize("num_seqs", [130, 256, 257, 300])
def test_prefill_many_sequences(num_seqs):
    """Batches of more sequences than a wave has lanes: up to 256 sequences
    the work-groups rank the items by cost over several sequences per lane
    (130: three, 256: four), past 256 they take the plain order.  Short
    chunks (0 to 40 tokens, some of one) over prefixes of 0 to 300 tokens,
    every sequence's output against the oracle."""
    rng = np.random.default_rng(9100 + num_seqs)
    prefixes = rng.integers(0, 301, size=num_seqs).tolist()
    qlens = rng.integers(0, 41, size=num_seqs).tolist()
    for i in rng.choice(num_seqs, size=8, replace=False):
        qlens[int(i)] = int(rng.choice([0, 1, 32, 33]))
    case = W.random_prefill(9200 + num_seqs, prefixes, qlens, num_heads=8, num_kv_heads=2, head_dim=64,
                            block_size=16, dtype=W.BF16)
    what = f"{num_seqs} sequences, {sum(qlens)} query rows"
    log(what)
    _, got = _run(case)
    assert_close(got, oracle_prefill(case), W.BF16, what)
