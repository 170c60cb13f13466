"""pa_decode on the GPU against the CPU oracle: the five workloads at full
size (sampled where the oracle would be slow), a sweep of shapes, the
bit-exact index and leak probes, and edge cases."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (DeviceCase, assert_close, log, oracle_decode, to_dev, to_host_bits, to_host_f32,
                      torch)

pytestmark = pytest.mark.gpu

BENCH_PARTITION = 320     # the split-K partition the benchmark times for the bs32 batch (and its G = 8 form)
BENCH_PARTITION_V64 = 192  # ... and for its 64-wide-value form
CASCADE_BENCH_PARTITION = 640  # own-token partition of the benchmark's cascade decode (prefix-shared batches)


def _run(case, partition_size, max_context_len=None):
    dev = DeviceCase(case)
    dev.write()
    out = dev.decode(partition_size, max_context_len=max_context_len)
    torch().cuda.synchronize()
    return dev, to_host_f32(out, case.dtype)


def test_tiny_fp32_decode():
    case = W.make_config("tiny_fp32_decode")
    ref = oracle_decode(case)
    for ps in (0, 16, 32, 48, 64, 512):
        log(f"tiny fp32 decode partition={ps}")
        _, got = _run(case, ps)
        assert_close(got, ref, W.F32, f"partition {ps}")


CTX_MIX = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 257, 700]


@pytest.mark.parametrize("dtype,head_dim", [(W.BF16, 128), (W.BF16, 64), (W.F32, 64), (W.F32, 128)])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_decode_shapes(dtype, head_dim, group):
    hkv = 2
    for bs in (8, 16, 32):
        case = W.random_decode(1000 * group + bs + head_dim, CTX_MIX, num_heads=hkv * group,
                               num_kv_heads=hkv, head_dim=head_dim, block_size=bs, dtype=dtype,
                               extra_table_cols=2)
        ref = oracle_decode(case)
        for ps in (0, bs, 4 * bs, 256):
            log(f"decode {dtype} D={head_dim} G={group} bs={bs} partition={ps}")
            _, got = _run(case, ps)
            assert_close(got, ref, dtype, f"{dtype} D{head_dim} G{group} bs{bs} ps{ps}")



@pytest.mark.parametrize("hkv,group", [(1, 8), (3, 4), (5, 2), (6, 1), (12, 4)])
def test_decode_kv_head_counts(hkv, group):
    """Key head dim 128 reads the rows of 4 kv heads per load: kv-head
    counts that are not a multiple of 4 leave rows past the last kv head in
    the last work-group (they read a real head and are dropped), and 12 kv
    heads make three groups.  bf16, both value widths, with and without
    split-K and through the fused append."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    for dv in (128, 64):
        case = W.random_decode(7100 + 10 * hkv + group + dv, [1, 33, 200, 513, 1100], num_heads=hkv * group,
                               num_kv_heads=hkv, head_dim=128, v_head_dim=dv, block_size=16, dtype=W.BF16,
                               extra_table_cols=1)
        ref = oracle_decode(case)
        dev = DeviceCase(case)
        dev.write()
        for ps in (0, 64, 256):
            log(f"decode Hkv={hkv} G={group} Dv={dv} partition={ps}")
            got = to_host_f32(dev.decode(ps), W.BF16)
            assert_close(got, ref, W.BF16, f"Hkv{hkv} G{group} Dv{dv} ps{ps}")
        key, val = _append_rows(case)
        dev2 = DeviceCase(case)
        log(f"decode append Hkv={hkv} G={group} Dv={dv}")
        out = P.pa_decode_append(dev2.q, to_dev(key, W.BF16), to_dev(val, W.BF16), dev2.k_cache, dev2.v_cache,
                                 dev2.block_tables, dev2.context_lens, case.scale, case.max_context_len, 64)
        t.cuda.synchronize()
        assert_close(to_host_f32(out, W.BF16), ref, W.BF16, f"append Hkv{hkv} G{group} Dv{dv}")
        k_ref, v_ref = oracle.kv_cache_write(case.k_cache, case.v_cache, case.new_key, case.new_value,
                                             case.slot_mapping)
        assert np.array_equal(to_host_bits(dev2.k_cache).view(np.uint16), k_ref.view(np.uint16)), "K pool"
        assert np.array_equal(to_host_bits(dev2.v_cache).view(np.uint16), v_ref.view(np.uint16)), "V pool"

@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("dims", [(128, 64), (64, 128)])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_decode_separate_value_dim(dtype, dims, group):
    """Key head dim D, value head dim Dv != D: outputs are [S, H, Dv]."""
    D, Dv = dims
    hkv = 2
    for bs in (8, 16, 32):
        case = W.random_decode(7000 + 100 * group + bs + D, CTX_MIX, num_heads=hkv * group, num_kv_heads=hkv,
                               head_dim=D, v_head_dim=Dv, block_size=bs, dtype=dtype, extra_table_cols=2)
        ref = oracle_decode(case)
        assert ref.shape == (len(CTX_MIX), hkv * group, Dv)
        for ps in (0, bs, 256):
            log(f"decode {dtype} D={D} Dv={Dv} G={group} bs={bs} partition={ps}")
            _, got = _run(case, ps)
            assert_close(got, ref, dtype, f"{dtype} D{D} Dv{Dv} G{group} bs{bs} ps{ps}")


@pytest.mark.parametrize("ps", [0, 192, 256, 512, BENCH_PARTITION])
def test_decode_batch_bs32_full(ps):
    case = W.make_config("decode_batch_bs32")
    ref = oracle_decode(case)
    log(f"decode batch 32 x U[512,4096] partition={ps}")
    _, got = _run(case, ps)
    mx, mean = assert_close(got, ref, W.BF16, f"bs32 batch ps{ps}")
    print(f"bs32 batch ps={ps}: max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_decode_batch_bs32_eight_heads_per_kv_head_full():
    """The bs32 batch with 64 query heads over its 8 kv heads (G = 8)."""
    case = W.decode_batch(2000, num_heads=64)
    ref = oracle_decode(case)
    for ps in (BENCH_PARTITION, 512):
        log(f"decode batch 32 x U[512,4096], 64 q / 8 kv heads, partition={ps}")
        _, got = _run(case, ps)
        mx, mean = assert_close(got, ref, W.BF16, f"bs32 batch G8 ps{ps}")
        print(f"bs32 batch G=8 ps {ps}: max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_decode_batch_bs32_ctx4096_full_sampled():
    """The metric's literal shape, 32 sequences of exactly 4096 tokens, at
    the partition the benchmark times it with (1024) and at 512; every
    output row computed by the kernel, 8 of the 32 sequences (every fourth)
    compared with the oracle, so that the fp64 oracle stays within seconds."""
    case = W.decode_batch(2000, fixed_ctx=4096)
    sample = list(range(0, 32, 4))
    ref = oracle_decode(case, seqs=sample)[sample]
    for ps in (1024, 512):
        log(f"decode batch 32 x 4096 partition={ps}")
        _, got = _run(case, ps)
        mx, mean = assert_close(got[sample], ref, W.BF16, f"bs32 ctx4096 ps{ps}")
        print(f"bs32 ctx4096 ps={ps}: max-abs {mx:.2e} mean-abs {mean:.2e} (8 sampled sequences)")


def test_decode_batch_bs32_k128_v64_full():
    """The bs32 batch with 64-wide values under its 128-wide keys, at the
    benchmark's partition."""
    case = W.decode_batch(2000, v_head_dim=64)
    ref = oracle_decode(case)
    for ps in (BENCH_PARTITION_V64, 512):
        log(f"decode batch 32 x U[512,4096], key dim 128, value dim 64, partition={ps}")
        _, got = _run(case, ps)
        mx, mean = assert_close(got, ref, W.BF16, f"bs32 k128 v64 ps{ps}")
        print(f"bs32 k128 v64 ps={ps}: max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.timeout(900)
def test_long_context_split_k_full():
    case = W.make_config("long_context_decode")
    log(f"long-context decode ctx={case.context_lens.tolist()} partition=512")
    _, got = _run(case, 512)
    ref = oracle_decode(case)
    mx, mean = assert_close(got, ref, W.BF16, "long context")
    print(f"long context: max-abs {mx:.2e} mean-abs {mean:.2e} |o| mean {np.abs(ref).mean():.3f}")


@pytest.mark.parametrize("name", ["prefix_shared_decode_bs8", "prefix_shared_decode_bs16"])
def test_prefix_shared_full(name):
    case = W.make_config(name)
    ref = oracle_decode(case)
    for ps in (0, 256):
        log(f"{name} partition={ps}")
        _, got = _run(case, ps)
        assert_close(got, ref, W.BF16, f"{name} ps{ps}")


def test_stages_equal_fused_call():
    import paged_attention_kv_cache_amd as P
    case = W.random_decode(77, [5, 300, 1000, 2049], num_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=32, dtype=W.BF16)
    dev = DeviceCase(case)
    dev.write()
    t = torch()
    ps = 128
    need = P.pa_decode_workspace_bytes(4, 32, 128, case.max_context_len, ps)
    ws = t.empty(need, dtype=t.uint8, device="cuda")
    log("decode stages vs fused")
    fused = dev.decode(ps, workspace=ws).clone()
    out = t.empty_like(dev.q)
    args = (dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens, case.scale,
            case.max_context_len, ps)
    P.pa_decode_partition(*args, out=out, workspace=ws)
    P.pa_decode_reduce(*args, out=out, workspace=ws)
    t.cuda.synchronize()
    assert np.array_equal(to_host_bits(out), to_host_bits(fused))


@pytest.mark.parametrize("dtype,group", [(W.BF16, 4), (W.BF16, 8), (W.F32, 4)])
def test_reduce_ignores_stale_workspace(dtype, group):
    """Workspace slots past a row's partitions are never written; the reduce
    loads some of them before it knows the row's partition count and must
    select them out.  A workspace full of NaN bit patterns gives the same
    bits as a zeroed one."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    case = W.random_decode(91 + group, [1, 40, 513, 700, 2049, 64], num_heads=8 * group, num_kv_heads=8,
                           head_dim=128, block_size=16, dtype=dtype)
    dev = DeviceCase(case)
    dev.write()
    ref = oracle_decode(case)
    ps, mcl = 64, 4096  # 64 slots per row, most of them unused
    need = P.pa_decode_workspace_bytes(6, 8 * group, 128, mcl, ps)
    bits = []
    for fill in (0x00, 0xFF):
        log(f"decode {dtype} G={group} partition={ps} workspace filled with {fill:#x}")
        ws = t.full((need,), fill, dtype=t.uint8, device="cuda")
        out = dev.decode(ps, max_context_len=mcl, workspace=ws)
        t.cuda.synchronize()
        assert_close(to_host_f32(out, dtype), ref, dtype, f"{dtype} G{group} fill {fill:#x}")
        bits.append(to_host_bits(out).copy())
    assert np.array_equal(bits[0], bits[1])


@pytest.mark.parametrize("num_seqs", [5, 65])
def test_no_cross_sequence_leakage(num_seqs):
    """Each sequence reads only its own blocks: with every pool block that
    sequence i does not own overwritten by NaN, row i of the batch keeps
    its bits; and the sequence run alone gives the same bits as in the
    batch.  Five sequences take the size-ordered dispatch, 65 the plain
    order."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    base = [40, 1, 513, 2000, 77]
    ctx = (base * 13)[:num_seqs]
    case = W.random_decode(31, ctx, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype=W.BF16)
    dev = DeviceCase(case)
    dev.write()
    ps = 256
    log(f"decode batch of {num_seqs} for leakage check")
    full = to_host_bits(dev.decode(ps))
    k0, v0 = dev.k_cache.clone(), dev.v_cache.clone()
    nan = t.tensor(0x7FC0, dtype=t.int16).view(t.bfloat16).item()
    for i in range(min(num_seqs, 5)):
        nb = -(-ctx[i] // case.block_size)
        own = set(int(b) for b in case.block_tables[i, :nb])
        others = t.tensor([b for b in range(case.num_blocks) if b not in own], dtype=t.long, device="cuda")
        dev.k_cache.copy_(k0)
        dev.v_cache.copy_(v0)
        dev.k_cache.index_fill_(0, others, nan)
        dev.v_cache.index_fill_(0, others, nan)
        log(f"decode with every block but sequence {i}'s set to NaN")
        got = to_host_bits(dev.decode(ps))
        assert np.array_equal(got[i], full[i]), f"sequence {i}"
        log(f"decode sequence {i} alone")
        one = P.pa_decode(dev.q[i:i + 1].contiguous(), dev.k_cache, dev.v_cache,
                          dev.block_tables[i:i + 1].contiguous(), dev.context_lens[i:i + 1].contiguous(),
                          case.scale, case.max_context_len, ps)
        t.cuda.synchronize()
        assert np.array_equal(to_host_bits(one)[0], full[i]), f"sequence {i} alone"


def _bf16(x):
    return W.f32_to_bf16_bits(np.float32(x).reshape(1))[0]


def _probe_case(seed, ctx, bs, num_seqs, targets, leak=False):
    """Index probe: q = 40 e0 for every head; in sequence i every key has a
    zero first component except the one at position targets[i], which is
    40 e0.  Every score is exactly 0 but the target's (40^2 / sqrt(128) =
    141 nats above), so every other weight underflows to exactly 0 and the
    output is V[target] bit for bit.  With ``leak`` the slot just past the
    context and every padding block hold keys 80 e0, four times the
    target's score: any read of them shows up."""
    case = W.random_decode(seed, [ctx] * num_seqs, num_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=bs, dtype=W.BF16, poison=not leak, extra_table_cols=1)
    c40, c80, zero = _bf16(40.0), _bf16(80.0), np.uint16(0)
    nb = case.num_blocks
    kflat = case.k_cache.reshape(nb * bs, 8, 128)
    kflat[case.slot_mapping] = case.new_key        # edit the real values of the new tokens too
    for i in range(num_seqs):
        row = case.block_tables[i]
        for p in range(ctx):
            s = int(row[p // bs]) * bs + p % bs
            if p == targets[i]:
                kflat[s] = zero
                kflat[s, :, 0] = c40
            else:
                kflat[s, :, 0] = zero
        if leak:
            past = ctx  # first position outside the context
            blk = int(row[past // bs])
            s = blk * bs + past % bs
            kflat[s] = zero
            kflat[s, :, 0] = c80
    if leak:
        pad = case.pad_block
        case.k_cache[pad] = zero
        case.k_cache[pad, :, :, 0] = c80
    # the new tokens carry the edited values; their slots stay poisoned
    # until the write
    case.new_key = kflat[case.slot_mapping].copy()
    if not leak:
        kflat[case.slot_mapping] = np.uint16(0x7FC0)
    case.q[:] = zero
    case.q[:, :, 0] = c40
    return case


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_index_probe_every_position(bs):
    ctx = 3 * 64 + 5           # several partitions of 64 and a ragged tail
    targets = list(range(ctx))
    case = _probe_case(5 + bs, ctx, bs, ctx, targets)
    vflat = W.storage_to_f32(case.v_cache, W.BF16).reshape(-1, 8, 128)
    vnew = W.storage_to_f32(case.new_value, W.BF16)
    for ps in (0, 64, 2 * bs):
        log(f"index probe bs={bs} partition={ps}")
        _, got = _run(case, ps)
        for i, p in enumerate(targets):
            s = int(case.block_tables[i, p // bs]) * bs + p % bs
            v = vnew[i] if p == ctx - 1 else vflat[s]
            exp = np.repeat(v, 4, axis=0)                  # head h reads kv head h // 4
            assert np.array_equal(got[i], exp), f"bs{bs} ps{ps} target {p}"


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_leak_probe_past_context(bs):
    ctx = 2 * 32 + 3           # partial last block at every block size
    targets = [(7 * i) % ctx for i in range(6)]
    case = _probe_case(50 + bs, ctx, bs, 6, targets, leak=True)
    vflat = W.storage_to_f32(case.v_cache, W.BF16).reshape(-1, 8, 128)
    vnew = W.storage_to_f32(case.new_value, W.BF16)
    for ps in (0, bs, 32):
        log(f"leak probe bs={bs} partition={ps}")
        _, got = _run(case, ps)
        for i, p in enumerate(targets):
            s = int(case.block_tables[i, p // bs]) * bs + p % bs
            v = vnew[i] if p == ctx - 1 else vflat[s]
            assert np.array_equal(got[i], np.repeat(v, 4, axis=0)), f"bs{bs} ps{ps} seq {i} leaked"


def test_context_zero_and_one():
    case = W.random_decode(9, [0, 1, 5], num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                           dtype=W.F32)
    ref = oracle_decode(case)
    for ps in (0, 16):
        log(f"ctx 0/1 partition={ps}")
        _, got = _run(case, ps)
        assert np.array_equal(got[0], np.zeros_like(got[0]))
        assert np.array_equal(got[1], np.repeat(W.storage_to_f32(case.new_value, W.F32)[0], 4, axis=0))
        assert_close(got, ref, W.F32, f"ps{ps}")


@pytest.mark.parametrize("num_seqs", [63, 64, 65])
def test_dispatch_order_edge_batches(num_seqs):
    """The partition kernel hands out (sequence, partition) pairs by size for
    batches of up to 64 sequences (65 takes the plain order): contexts of 0
    and 1, exact multiples of the partition size, one token past them, and
    long ones, so that full, partial and empty pairs all occur."""
    rng = np.random.default_rng(num_seqs)
    base = [0, 1, 32, 33, 64, 511, 512, 513, 1024, 1537, 2048]
    ctx = (base * 6)[:num_seqs]
    ctx = [int(c) for c in rng.permutation(ctx)]
    case = W.random_decode(500 + num_seqs, ctx, num_heads=8, num_kv_heads=2, head_dim=128, block_size=32,
                           dtype=W.BF16)
    ref = oracle_decode(case)
    for ps in (32, 512):
        log(f"{num_seqs} sequences, partition {ps}")
        _, got = _run(case, ps)
        assert_close(got, ref, W.BF16, f"S{num_seqs} ps{ps}")
        assert np.array_equal(got[ctx.index(0)], np.zeros_like(got[0]))


def test_loose_max_context_len():
    """A host bound above the real maximum only adds empty partitions."""
    case = W.random_decode(12, [100, 37], num_heads=16, num_kv_heads=4, head_dim=128, block_size=32,
                           dtype=W.BF16, extra_table_cols=10)
    ref = oracle_decode(case)
    log("loose max_context_len")
    _, got = _run(case, 32, max_context_len=400)
    assert_close(got, ref, W.BF16, "loose bound")



def test_many_partitions():
    """Hundreds of partitions of one sequence merged by the reduce kernel."""
    case = W.random_decode(67, [300 * 32 + 5, 40], num_heads=32, num_kv_heads=8, head_dim=128, block_size=32,
                           dtype=W.BF16)
    ref = oracle_decode(case)
    for ps in (32, 64):
        log(f"{-(-case.max_context_len // ps)} partitions")
        _, got = _run(case, ps)
        assert_close(got, ref, W.BF16, f"ps{ps}")



BOUNDARY_CTX = [64, 64, 0, 128, 1, 63, 65, 200, 0, 3, 5, 7, 700, 64, 1, 130]


@pytest.mark.parametrize("group,dims", [(1, (128, 128)), (4, (128, 128)), (8, (128, 128)), (4, (128, 64))])
def test_partition_boundary_contexts(group, dims):
    """Contexts of exactly one or two partitions, one token either side of
    a partition boundary, 0 and 1 tokens, beside long ones (bf16, head dim
    128, partitions of 64 and 128 tokens): pa_decode, its two stages over a
    workspace of NaN bit patterns, and the fused append all agree with the
    oracle, and the stages give the fused call's bits."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    D, Dv = dims
    case = W.random_decode(8800 + group + Dv, BOUNDARY_CTX, num_heads=4 * group, num_kv_heads=4, head_dim=D,
                           v_head_dim=Dv, block_size=16, dtype=W.BF16, extra_table_cols=1)
    ref = oracle_decode(case)
    dev = DeviceCase(case)
    dev.write()
    for ps in (64, 128):
        log(f"boundary contexts G={group} D={D} Dv={Dv} partition={ps}")
        need = P.pa_decode_workspace_bytes(len(BOUNDARY_CTX), 4 * group, Dv, case.max_context_len, ps)
        ws = t.full((need,), 0xFF, dtype=t.uint8, device="cuda")
        fused = dev.decode(ps, workspace=ws).clone()
        t.cuda.synchronize()
        got = to_host_f32(fused, W.BF16)
        assert_close(got, ref, W.BF16, f"boundary G{group} ps{ps}")
        for i, n in enumerate(BOUNDARY_CTX):
            if n == 0:
                assert np.array_equal(got[i], np.zeros_like(got[i]))
        out = t.empty((len(BOUNDARY_CTX), 4 * group, Dv), dtype=fused.dtype, device="cuda")
        args = (dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens, case.scale,
                case.max_context_len, ps)
        P.pa_decode_partition(*args, out=out, workspace=ws)
        P.pa_decode_reduce(*args, out=out, workspace=ws)
        t.cuda.synchronize()
        assert np.array_equal(to_host_bits(out), to_host_bits(fused))
    k_ref, v_ref = oracle.kv_cache_write(case.k_cache, case.v_cache, case.new_key, case.new_value,
                                         case.slot_mapping)
    key, val = _append_rows(case)
    log(f"boundary contexts, fused append G={group}")
    dev2 = DeviceCase(case)
    out = P.pa_decode_append(dev2.q, to_dev(key, W.BF16), to_dev(val, W.BF16), dev2.k_cache, dev2.v_cache,
                             dev2.block_tables, dev2.context_lens, case.scale, case.max_context_len, 64)
    t.cuda.synchronize()
    assert_close(to_host_f32(out, W.BF16), ref, W.BF16, f"boundary append G{group}")
    assert np.array_equal(to_host_bits(dev2.k_cache).view(np.uint16), k_ref.view(np.uint16)), "K pool"
    assert np.array_equal(to_host_bits(dev2.v_cache).view(np.uint16), v_ref.view(np.uint16)), "V pool"


# ------------------------------------------------------------ cascade decode

def _cascade(case, group_start, shared_len, partition_size=256, max_context_len=None, max_shared_len=None):
    import paged_attention_kv_cache_amd as P
    t = torch()
    dev = DeviceCase(case)
    dev.write()
    gs = t.tensor(group_start, dtype=t.int32, device="cuda")
    sl = t.tensor(shared_len, dtype=t.int32, device="cuda")
    mg = max(b - a for a, b in zip(group_start[:-1], group_start[1:]))
    mcl = case.max_context_len if max_context_len is None else max_context_len
    msl = max(shared_len) if max_shared_len is None else max_shared_len
    out = P.pa_decode_cascade(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens, case.scale, mcl,
                              gs, sl, mg, partition_size, max_shared_len=msl)
    t.cuda.synchronize()
    return to_host_f32(out, case.dtype)


@pytest.mark.parametrize("name", ["prefix_shared_decode_bs8", "prefix_shared_decode_bs16"])
def test_cascade_prefix_shared_full(name):
    case = W.make_config(name)
    bs = case.block_size
    ref = oracle_decode(case)
    for ps in (256, 512, CASCADE_BENCH_PARTITION):
        log(f"cascade {name} partition={ps}")
        got = _cascade(case, [0, 16, 32, 48, 64], [64 * bs] * 4, ps)
        mx, mean = assert_close(got, ref, W.BF16, f"cascade {name} ps{ps}")
        print(f"cascade {name} ps={ps}: max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("scale", [0.37, 0.0, -0.05])
def test_cascade_other_scales(scale):
    """Cascade decode and plain decode under scales other than
    1/sqrt(head_dim) (zero and negative included) against the oracle."""
    sizes = [5, 12]
    starts = np.cumsum([0] + sizes).tolist()
    group_of = [g for g, n in enumerate(sizes) for _ in range(n)]
    bs, shared_blocks = 16, 20
    rng = np.random.default_rng(99)
    ctx = [int(x) for x in rng.integers(shared_blocks * bs + 1, 1200, size=sum(sizes))]
    case = W.random_decode(990, ctx, num_heads=32, num_kv_heads=8, head_dim=128, block_size=bs, dtype=W.BF16,
                           shared_blocks=shared_blocks, group_of=group_of)
    case.scale = float(scale)
    ref = oracle_decode(case)
    log(f"cascade scale {scale}")
    got = _cascade(case, starts, [shared_blocks * bs] * 2, 256)
    assert_close(got, ref, W.BF16, f"cascade scale {scale}")
    log(f"decode scale {scale}")
    _, got = _run(case, 256)
    assert_close(got, ref, W.BF16, f"decode scale {scale}")


@pytest.mark.parametrize("dims", [(128, 64), (64, 128)])
@pytest.mark.parametrize("group", [2, 8])
def test_cascade_separate_value_dim(dims, group):
    """Cascade decode with a value head dim of its own: the shared chunks
    and the own-token partitions write partials of the value width."""
    D, Dv = dims
    sizes = [3, 40, 5]
    starts = np.cumsum([0] + sizes).tolist()
    group_of = [g for g, n in enumerate(sizes) for _ in range(n)]
    bs, shared_blocks = 16, 10
    rng = np.random.default_rng(77 + group + D)
    ctx = [int(x) for x in rng.integers(shared_blocks * bs + 1, 900, size=sum(sizes))]
    ctx[0] = 3 * bs                            # a row that ends inside the shared part
    hkv = 2
    case = W.random_decode(900 + group + D, ctx, num_heads=hkv * group, num_kv_heads=hkv, head_dim=D, block_size=bs,
                           dtype=W.BF16, shared_blocks=shared_blocks, group_of=group_of, v_head_dim=Dv)
    ref = oracle_decode(case)
    assert ref.shape[-1] == Dv
    shared = [shared_blocks * bs, shared_blocks * bs, 4 * bs]
    for ps in (64, 256):
        log(f"cascade D={D} Dv={Dv} G={group} partition={ps}")
        got = _cascade(case, starts, shared, ps)
        assert_close(got, ref, W.BF16, f"cascade D{D} Dv{Dv} G{group} ps{ps}")


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_cascade_irregular_groups(group):
    """Groups of 1, 3, 70 (two member tiles) and 6 rows; shared lengths below
    the true sharing, 0, and rows whose context ends inside or exactly at
    the shared part (no own tokens)."""
    sizes = [1, 3, 70, 6]
    starts = np.cumsum([0] + sizes).tolist()
    group_of = [g for g, n in enumerate(sizes) for _ in range(n)]
    bs, shared_blocks = 16, 12
    rng = np.random.default_rng(group)
    ctx = [int(x) for x in rng.integers(shared_blocks * bs + 1, 1500, size=sum(sizes))]
    ctx[1], ctx[2] = 5 * bs, 8 * bs           # group 1: its first row ends inside the shared part, one exactly at it
    ctx[4] = 2 * bs - 3                        # group 2: a row far shorter than the shared part
    hkv = 2
    case = W.random_decode(300 + group, ctx, num_heads=hkv * group, num_kv_heads=hkv, head_dim=128, block_size=bs,
                           dtype=W.BF16, shared_blocks=shared_blocks, group_of=group_of)
    ref = oracle_decode(case)
    shared = [shared_blocks * bs, 8 * bs, shared_blocks * bs, 0]
    for ps in (64, 256):
        log(f"cascade irregular G={group} partition={ps}")
        got = _cascade(case, starts, shared, ps)
        assert_close(got, ref, W.BF16, f"cascade irregular G{group} ps{ps}")
    # max_shared_len below the largest shared_len (one 512-token chunk
    # still covers the 192 shared tokens)
    for msl in (0, 100):
        log(f"cascade irregular G={group} max_shared_len={msl}")
        got = _cascade(case, starts, shared, 64, max_shared_len=msl)
        assert_close(got, ref, W.BF16, f"cascade irregular G{group} clamp{msl}")


@pytest.mark.parametrize("group", [4, 8])
def test_cascade_shared_clamp(group):
    """Shared parts longer than one 512-token chunk (640 and 900 tokens)
    under max_shared_len 0, 100 and 600: one chunk each (the tokens past 512
    then run in the members' own partitions) or two (no clamp)."""
    sizes = [3, 5, 2]
    starts = np.cumsum([0] + sizes).tolist()
    group_of = [g for g, n in enumerate(sizes) for _ in range(n)]
    bs, shared_blocks = 16, 57
    rng = np.random.default_rng(60 + group)
    ctx = [int(x) for x in rng.integers(shared_blocks * bs + 1, 1600, size=sum(sizes))]
    ctx[3] = 700                               # a row ending inside its group's shared part
    hkv = 2
    case = W.random_decode(6000 + group, ctx, num_heads=hkv * group, num_kv_heads=hkv, head_dim=128, block_size=bs,
                           dtype=W.BF16, shared_blocks=shared_blocks, group_of=group_of)
    ref = oracle_decode(case)
    shared = [640, 900, 0]
    for msl in (0, 100, 600, None):
        log(f"cascade clamp G={group} max_shared_len={msl}")
        got = _cascade(case, starts, shared, 384, max_shared_len=msl)
        assert_close(got, ref, W.BF16, f"cascade clamp G{group} msl{msl}")


@pytest.mark.parametrize("group,dims", [(4, (128, 128)), (8, (128, 128)), (2, (64, 128)), (4, (128, 64))])
def test_cascade_unaligned_shared_lengths(group, dims):
    """Shared lengths that are not multiples of 8 (100, 37, 3 tokens over 7
    truly shared blocks of 16): every member's own tokens then start inside
    a block and inside a tile of the partition kernel, whose first tile
    masks the tokens before them."""
    D, Dv = dims
    sizes = [4, 7, 2]
    starts = np.cumsum([0] + sizes).tolist()
    group_of = [g for g, n in enumerate(sizes) for _ in range(n)]
    bs, shared_blocks = 16, 7
    rng = np.random.default_rng(40 + group + D + Dv)
    ctx = [int(x) for x in rng.integers(shared_blocks * bs + 1, 700, size=sum(sizes))]
    ctx[5] = 40                                # a row ending just past its group's 37 shared tokens
    hkv = 2
    case = W.random_decode(4000 + group + D + Dv, ctx, num_heads=hkv * group, num_kv_heads=hkv, head_dim=D,
                           v_head_dim=Dv, block_size=bs, dtype=W.BF16, shared_blocks=shared_blocks,
                           group_of=group_of)
    ref = oracle_decode(case)
    for ps in (64, 256):
        log(f"cascade unaligned shared G={group} D={D} Dv={Dv} partition={ps}")
        got = _cascade(case, starts, [100, 37, 3], ps)
        assert_close(got, ref, W.BF16, f"cascade unaligned G{group} D{D} Dv{Dv} ps{ps}")


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_cascade_index_probe(bs):
    """Index probe through cascade decode: groups of one row that claim a
    shared part, so the target is read by the MFMA pass or by the
    partitions; the output is that row's V bit for bit."""
    ctx = 3 * 64 + 5
    targets = list(range(0, ctx, 3))
    case = _probe_case(70 + bs, ctx, bs, len(targets), targets)
    vflat = W.storage_to_f32(case.v_cache, W.BF16).reshape(-1, 8, 128)
    vnew = W.storage_to_f32(case.new_value, W.BF16)
    S = len(targets)
    starts = list(range(S + 1))
    shared = [((i % 5) * 2 * bs) for i in range(S)]    # 0 .. 8 blocks, some past the context
    log(f"cascade index probe bs={bs}")
    got = _cascade(case, starts, shared, 64)
    for i, p in enumerate(targets):
        s = int(case.block_tables[i, p // bs]) * bs + p % bs
        v = vnew[i] if p == ctx - 1 else vflat[s]
        assert np.array_equal(got[i], np.repeat(v, 4, axis=0)), f"bs{bs} target {p} shared {shared[i]}"


def _append_rows(case):
    """The newest token's K and V rows of every sequence, [S, Hkv, D] / [S,
    Hkv, Dv] in storage dtype (zeros for a sequence with no context): the
    case's new rows are in sequence order, one per sequence with a context."""
    S = case.num_seqs
    key = np.zeros((S,) + case.new_key.shape[1:], dtype=case.new_key.dtype)
    val = np.zeros((S,) + case.new_value.shape[1:], dtype=case.new_value.dtype)
    j = 0
    for i, n in enumerate(case.context_lens.tolist()):
        if n > 0:
            key[i], val[i] = case.new_key[j], case.new_value[j]
            j += 1
    assert j == case.new_key.shape[0]
    return key, val


@pytest.mark.parametrize("dtype,group,dims", [(W.BF16, 1, (128, 128)), (W.BF16, 2, (64, 64)), (W.BF16, 4, (128, 128)),
                                              (W.BF16, 8, (128, 128)), (W.BF16, 8, (64, 64)), (W.F32, 4, (64, 64)),
                                              (W.BF16, 4, (128, 64)), (W.BF16, 2, (64, 128)),
                                              (W.BF16, 8, (64, 128))])
def test_decode_append(dtype, group, dims):
    """pa_decode_append = the cache write of each sequence's newest token
    plus pa_decode: outputs within tolerance of the oracle and the pools
    bit-exact with the oracle's write.  Every bf16 case (all G, equal or
    separate head dims) takes the fused kernel, which writes the rows inside
    the partition kernel; the fp32 case is the only one that runs the
    separate slot-deriving write kernel first."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    D, Dv = dims
    hkv = 2
    for bs in (8, 16, 32):
        case = W.random_decode(9100 + 10 * group + bs + D + Dv, CTX_MIX + [0], num_heads=hkv * group,
                               num_kv_heads=hkv, head_dim=D, v_head_dim=Dv, block_size=bs, dtype=dtype,
                               extra_table_cols=2)
        ref = oracle_decode(case)
        k_ref, v_ref = oracle.kv_cache_write(case.k_cache, case.v_cache, case.new_key, case.new_value,
                                             case.slot_mapping)
        key, val = _append_rows(case)
        for ps in (0, bs, 256):
            log(f"decode append {dtype} G={group} D={D} Dv={Dv} bs={bs} partition={ps}")
            dev = DeviceCase(case)   # fresh pools: the new tokens' slots still hold NaN
            out = P.pa_decode_append(dev.q, to_dev(key, dtype), to_dev(val, dtype), dev.k_cache, dev.v_cache,
                                     dev.block_tables, dev.context_lens, case.scale, case.max_context_len, ps)
            t.cuda.synchronize()
            assert_close(to_host_f32(out, dtype), ref, dtype, f"append {dtype} G{group} bs{bs} ps{ps}")
            bits = np.uint16 if dtype == W.BF16 else np.uint32
            assert np.array_equal(to_host_bits(dev.k_cache).view(bits), k_ref.view(bits)), "K pool"
            assert np.array_equal(to_host_bits(dev.v_cache).view(bits), v_ref.view(bits)), "V pool"


def test_decode_append_bs32_full():
    """The bs32 batch through the fused step at the benchmark's partition."""
    import paged_attention_kv_cache_amd as P
    case = W.make_config("decode_batch_bs32")
    ref = oracle_decode(case)
    key, val = _append_rows(case)
    dev = DeviceCase(case)
    log("decode append bs32 batch")
    out = P.pa_decode_append(dev.q, to_dev(key, W.BF16), to_dev(val, W.BF16), dev.k_cache, dev.v_cache,
                             dev.block_tables, dev.context_lens, case.scale, case.max_context_len, BENCH_PARTITION)
    torch().cuda.synchronize()
    mx, mean = assert_close(to_host_f32(out, W.BF16), ref, W.BF16, "append bs32")
    print(f"append bs32: max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("seed", range(36))
def test_decode_random_shapes(seed):
    """Seeded random shapes through the bf16 decode kernel against the
    oracle: query heads per kv head, kv heads (not always a multiple of
    four), key and value head dims, block size, partition size (0 = single
    pass), contexts from 0 to ~2,500 tokens, and the mode: plain decode,
    fused append (pools bit-exact with the oracle's write) or cascade over
    random groups with random shared lengths up to their true sharing."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    rng = np.random.default_rng(8800 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 3, 5, 8]))
    D, Dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32]))
    S = int(rng.integers(1, 41))
    mode = ["plain", "append", "cascade"][seed % 3]
    ps = int(rng.choice([0, bs, 64, 192, 512])) if mode != "cascade" else int(rng.choice([bs, 64, 192, 384]))
    ctx = rng.integers(0, 2500, size=S).tolist()
    for i in rng.choice(S, size=min(S, 3), replace=False):
        ctx[int(i)] = int(rng.choice([0, 1, bs - 1, bs, bs + 1, 63, 64, 65]))
    group_of, shared_blocks = None, 0
    if mode == "cascade":
        shared_blocks = int(rng.integers(1, 24))
        sizes, left = [], S
        while left > 0:
            sizes.append(int(min(left, rng.integers(1, 12))))
            left -= sizes[-1]
        group_of = [g for g, n in enumerate(sizes) for _ in range(n)]
    case = W.random_decode(9900 + seed, ctx, num_heads=hkv * G, num_kv_heads=hkv, head_dim=D, v_head_dim=Dv,
                           block_size=bs, dtype=W.BF16, shared_blocks=shared_blocks, group_of=group_of,
                           extra_table_cols=1)
    ref = oracle_decode(case)
    what = f"seed {seed} {mode} G{G} hkv{hkv} D{D} Dv{Dv} bs{bs} S{S} ps{ps}"
    log(what)
    if mode == "plain":
        _, got = _run(case, ps)
    elif mode == "append":
        key, val = _append_rows(case)
        k_ref, v_ref = oracle.kv_cache_write(case.k_cache, case.v_cache, case.new_key, case.new_value,
                                             case.slot_mapping)
        dev = DeviceCase(case)
        out = P.pa_decode_append(dev.q, to_dev(key, W.BF16), to_dev(val, W.BF16), dev.k_cache, dev.v_cache,
                                 dev.block_tables, dev.context_lens, case.scale, case.max_context_len, ps)
        t.cuda.synchronize()
        got = to_host_f32(out, W.BF16)
        assert np.array_equal(to_host_bits(dev.k_cache).view(np.uint16), k_ref.view(np.uint16)), what + " K pool"
        assert np.array_equal(to_host_bits(dev.v_cache).view(np.uint16), v_ref.view(np.uint16)), what + " V pool"
    else:
        starts = np.cumsum([0] + sizes).tolist()
        shared = [int(rng.integers(0, shared_blocks * bs + 1)) for _ in sizes]
        got = _cascade(case, starts, shared, ps, max_shared_len=int(rng.choice([0, 256, 4096])))
    assert_close(got, ref, W.BF16, what)
