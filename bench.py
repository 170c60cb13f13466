"""Benchmark of the paged-attention hot path on one MI355X.

A step is one decode step of the bs32 batch (32 sequences with contexts
uniform in [512, 4096], 32 q / 8 kv heads, head_dim 128, block_size 32,
bf16): the 32 new tokens' K/V rows written into the cache, attention of
each sequence's query over its whole context, and the merge of the
split-K partials.  The headline runs it as ``pa_decode_append`` (the
partition kernel that attends to the newest token also writes its rows)
and the reduce; the same step as three launches (``pa_kv_cache_write``,
``pa_decode_partition``, ``pa_decode_reduce``) is timed beside it.  Inputs
are resident in HBM before timing starts.  Each step uses the next of R copies of the KV pool (about
2 GB in total), so the 256 MB Infinity Cache cannot serve the KV from an
earlier step.

Prints one JSON line: throughput in tokens/s, the KV bytes per second of
the step and of the decode partition kernel alone (against 8 TB/s and
against the read rate a plain sequential read reaches on the same device
in the same run), the roofline of the partition kernel, timing statistics
(median, p10, p90 over the timed steps; a warm number beside the cold
headline), a secondary prefill-chunk measurement (MFMA fraction), other
decode workloads, the scheduler-driven serving loop, and the CPU oracle
timed on the host as a baseline.

    python bench.py [--steps K] [--warmup W] [--partition P] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode tokens/s + achieved KV GB/s (% HBM peak), bs32 ctx4K GQA 32/8 bf16"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_CLOCK_GHZ = 2.4  # the engine clock the published MFMA peak is quoted at
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition", type=int, default=320, help="split-K partition of the bs32 step (tokens)")
    ap.add_argument("--rotate-gb", type=float, default=2.0, help="total size of rotated KV pools")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the long-context and prefix-shared decode lines")
    ap.add_argument("--cpu-seconds", type=float, default=3.0, help="per run of the CPU oracle's decode leg")
    ap.add_argument("--only", default=None, choices=sorted(ONLY),
                    help="time one workload alone (for per-workload counter runs); prints its own JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device-to-device (a kernel of known traffic for counter runs)")
    return ap.parse_args()


# workloads --only can time alone, each in its own process
ONLY = ("decode_bs32", "tiny_fp32_decode", "long_context_decode", "decode_batch_bs32_ctx4096",
        "decode_batch_bs32_64q_8kv", "decode_batch_bs32_k128_v64", "prefix_shared_decode_bs16",
        "prefix_shared_decode_bs8", "chunked_prefill", "chunked_prefill_bs16", "chunked_prefill_bs8",
        "stream_read", "mfma_ceiling")


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_attention_kv_cache_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key: str, src_hash: str, partition_size=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (and, for decode, at the same split-K
    partition, which sets the bytes of partials written); else None."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        rec = data.get(kernel_key)
        if rec and rec.get("source_hash") == src_hash and rec.get("partition_size") == partition_size:
            return rec.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None
    return None


def stats_ms(samples_ms):
    """median, p10, p90 (microseconds) of per-iteration times in ms"""
    a = np.asarray(samples_ms, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def timed_each(fn, n):
    """run fn(i) n times with an event pair around each call; per-call ms"""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def bench_stream_ceiling(nbytes=1 << 30, launches=20):
    """The library's plain sequential read kernel over buffers of ``nbytes``
    taken in turn, enough of them that together they exceed 2 GiB (no
    buffer stays in the 256 MB Infinity Cache between its reads): GB/s."""
    import torch
    import paged_attention_kv_cache_amd as P
    n = int(nbytes) // 16 * 16
    nbuf = max(2, -(-(2 << 30) // n))
    bufs = [torch.ones(n // 2, dtype=torch.int16, device="cuda") for _ in range(nbuf)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(2 * nbuf):
        P.pa_stream_read(bufs[i % nbuf], sink)
    ms = timed_each(lambda i: P.pa_stream_read(bufs[i % nbuf], sink), launches)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(launches):
        P.pa_stream_read(bufs[i % nbuf], sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / launches
    del bufs
    torch.cuda.empty_cache()
    return {"bytes_per_launch": n, "buffers": nbuf, "gbps": round(n / (t * 1e-3) / 1e9, 1),
            "gbps_median_launch": round(n / (float(np.median(ms)) * 1e-3) / 1e9, 1),
            "frac_of_nominal": round(n / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def to_dev(arr, dtype):
    import torch
    import workloads as W
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def bench_decode(args):
    import torch
    import paged_attention_kv_cache_amd as P
    import workloads as W

    log("building the bs32 decode workload")
    case = W.make_config("decode_batch_bs32", poison=False)
    S, H, D = case.q.shape
    kv_bytes = case.kv_bytes_logical()
    pool_bytes = 2 * case.k_cache.nbytes
    R = max(2, int(math.ceil(args.rotate_gb * 1e9 / pool_bytes)))
    log(f"S={S} ctx sum={int(case.context_lens.sum())} KV={kv_bytes / 1e6:.1f} MB, "
        f"pool={pool_bytes / 1e6:.1f} MB x {R} rotations")

    k0 = to_dev(case.k_cache, case.dtype)
    v0 = to_dev(case.v_cache, case.dtype)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
    q = to_dev(case.q, case.dtype)
    new_k = to_dev(case.new_key, case.dtype)
    new_v = to_dev(case.new_value, case.dtype)
    slots = torch.from_numpy(case.slot_mapping).cuda()
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    out = torch.empty_like(q)
    ps = args.partition
    mcl = case.max_context_len
    need = P.pa_decode_workspace_bytes(S, H, D, mcl, ps)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step(r, ev=None):
        k, v = pools[r]
        if ev is not None:
            ev[0].record()
        P.pa_kv_cache_write(new_k, new_v, k, v, slots)
        if ev is not None:
            ev[1].record()
        P.pa_decode_partition(q, k, v, bt, cl, case.scale, mcl, ps, out=out, workspace=ws)
        if ev is not None:
            ev[2].record()
        P.pa_decode_reduce(q, k, v, bt, cl, case.scale, mcl, ps, out=out, workspace=ws)
        if ev is not None:
            ev[3].record()

    def step_fused(r):
        # the same step through pa_decode_append: the new K/V rows are
        # written by the partition kernel that attends to them (all 32
        # sequences have a context, so the rows are new_k / new_v in order)
        k, v = pools[r]
        P.pa_decode_append(q, new_k, new_v, k, v, bt, cl, case.scale, mcl, ps, out=out, workspace=ws)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step_fused(i % R)
    torch.cuda.synchronize()

    # the headline: exactly K steps (pa_decode_append + reduce) between one
    # pair of events, right after the warmup
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step_fused(i % R)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step_head = start.elapsed_time(end) / args.steps

    # per-step statistics: the same steps, an event pair around each
    step_each = timed_each(lambda i: step_fused(i % R), args.steps)
    # warm: every step on the same pool, which the Infinity Cache then
    # partly holds (the cold headline rotates R pools)
    for i in range(args.warmup):
        step_fused(0)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step_fused(0)
    end.record()
    torch.cuda.synchronize()
    ms_step_warm = start.elapsed_time(end) / args.steps

    # the same step as three launches (write, partition, reduce), K steps
    # after a warmup of its own
    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i % R)
    end.record()
    torch.cuda.synchronize()
    ms_step_three = start.elapsed_time(end) / args.steps

    # diagnostics: per-kernel durations from events around each launch (on
    # the launch stream), which add gaps of their own
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i % R, evs[i])
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    t_write = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    t_part = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    t_red = np.mean([e[2].elapsed_time(e[3]) for e in evs])

    # the partition kernel alone, launched back to back on the rotated pools
    # between one pair of events: its average launch duration, without the
    # gaps that an event pair around every launch adds
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        k, v = pools[i % R]
        P.pa_decode_partition(q, k, v, bt, cl, case.scale, mcl, ps, out=out, workspace=ws)
    end.record()
    torch.cuda.synchronize()
    t_part_b2b = start.elapsed_time(end) / args.steps
    part_each = timed_each(lambda i: P.pa_decode_partition(q, *pools[i % R], bt, cl, case.scale, mcl, ps, out=out,
                                                           workspace=ws), args.steps)

    # algorithmic bytes of one decode partition launch: every context
    # token's K and V row for all kv heads, q read once, the output (for
    # single-partition sequences) or nothing else counted
    q_bytes = case.q.nbytes
    part_bytes = kv_bytes + q_bytes + case.context_lens.nbytes + int(
        sum(-(-int(n) // case.block_size) for n in case.context_lens)) * 4
    achieved = part_bytes / (t_part_b2b * 1e-3) / 1e9
    src = source_hash("pa_decode.hip", "pa_common.h")
    res = dict(
        case=case, S=S, R=R, ms_step=ms_step_head, ms_step_three=ms_step_three,
        ms_step_with_events=ms_step, wall=wall, ms_step_warm=ms_step_warm,
        step_stats=stats_ms(step_each), part_stats=stats_ms(part_each),
        t_write=t_write, t_part=t_part, t_red=t_red, t_part_b2b=t_part_b2b, kv_bytes=kv_bytes,
        part_bytes=part_bytes,
        achieved=achieved, src=src, ps=ps,
    )
    log(f"step {ms_step_head * 1e3:.1f} us fused, {ms_step_three * 1e3:.1f} us as three launches "
        f"(events {ms_step * 1e3:.1f}); write {t_write * 1e3:.1f} us, "
        f"partition {t_part * 1e3:.1f} us (back to back {t_part_b2b * 1e3:.1f}), reduce {t_red * 1e3:.1f} us; "
        f"partition {achieved:.0f} GB/s")
    del pools
    torch.cuda.empty_cache()
    return res


def bench_decode_secondary(name, ps, steps=30, groups=None, case=None, cascade_ps=None):
    """Decode partition + reduce on another workload: time per launch pair
    (back to back over rotated pools), logical KV GB/s (every context token
    of every sequence) and unique KV GB/s (each shared physical block once)."""
    import torch
    import paged_attention_kv_cache_amd as P
    import workloads as W

    log(f"building {name}")
    if case is None:
        case = W.make_config(name, poison=False)
    S, H, D = case.q.shape
    Dv = case.v_cache.shape[-1]  # width of the output rows and partials
    pool_bytes = case.k_cache.nbytes + case.v_cache.nbytes
    R = max(2, int(math.ceil(2.0e9 / pool_bytes)))
    k0 = to_dev(case.k_cache, case.dtype)
    v0 = to_dev(case.v_cache, case.dtype)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
    q = to_dev(case.q, case.dtype)
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    out = torch.empty((S, H, Dv), dtype=q.dtype, device="cuda")
    mcl = case.max_context_len
    ws = torch.empty(max(P.pa_decode_workspace_bytes(S, H, Dv, mcl, ps), 1), dtype=torch.uint8, device="cuda")

    def part(i):
        k, v = pools[i % R]
        P.pa_decode_partition(q, k, v, bt, cl, case.scale, mcl, ps, out=out, workspace=ws)

    def red(i):
        k, v = pools[i % R]
        P.pa_decode_reduce(q, k, v, bt, cl, case.scale, mcl, ps, out=out, workspace=ws)

    for i in range(4):
        part(i)
        red(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        part(i)
    e1.record()
    torch.cuda.synchronize()
    t_part = e0.elapsed_time(e1) / steps
    e0.record()
    for i in range(steps):
        part(i)
        red(i)
    e1.record()
    torch.cuda.synchronize()
    t_both = e0.elapsed_time(e1) / steps
    logical = case.kv_bytes_logical()
    row_bytes = case.num_kv_heads * (case.head_dim + case.v_head_dim) * 2  # K+V of one token, all kv heads
    unique_tokens = 0
    seen = set()
    for i, n in enumerate(case.context_lens.tolist()):
        for j in range(-(-n // case.block_size)):
            b = int(case.block_tables[i, j])
            if b in seen:
                continue
            seen.add(b)
            unique_tokens += min(case.block_size, n - j * case.block_size)
    unique = unique_tokens * row_bytes
    res = {
        "workload": name, "num_seqs": S, "context_tokens": int(case.context_lens.sum()), "partition_size": ps,
        "partition_us": round(t_part * 1e3, 2), "partition_plus_reduce_us": round(t_both * 1e3, 2),
        "tokens_per_s": round(S / (t_both * 1e-3), 1),
        "logical_kv_gbps": round(logical / (t_part * 1e-3) / 1e9, 1),
        "unique_kv_gbps": round(unique / (t_part * 1e-3) / 1e9, 1),
        "unique_kv_hbm_frac": round(unique / (t_part * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "logical_kv_bytes": logical, "unique_kv_bytes": unique,
    }
    if groups:
        # cascade decode: the shared blocks read once per group
        gs = torch.tensor(groups[0], dtype=torch.int32, device="cuda")
        sl = torch.tensor(groups[1], dtype=torch.int32, device="cuda")
        mg = max(b - a for a, b in zip(groups[0][:-1], groups[0][1:]))
        cps = cascade_ps or ps  # the own tokens after the shared ones are shorter than whole contexts
        wsc = torch.empty(max(P.pa_decode_cascade_workspace_bytes(S, H, Dv, mcl, cps), 1), dtype=torch.uint8,
                          device="cuda")

        def casc(i):
            k, v = pools[i % R]
            P.pa_decode_cascade(q, k, v, bt, cl, case.scale, mcl, gs, sl, mg, cps, out=out, workspace=wsc,
                                max_shared_len=max(groups[1]))

        for i in range(4):
            casc(i)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            casc(i)
        e1.record()
        torch.cuda.synchronize()
        t_c = e0.elapsed_time(e1) / steps
        res["cascade_partition_size"] = cps
        res["cascade_us"] = round(t_c * 1e3, 2)
        res["cascade_tokens_per_s"] = round(S / (t_c * 1e-3), 1)
        res["cascade_unique_kv_gbps"] = round(unique / (t_c * 1e-3) / 1e9, 1)
        res["cascade_unique_kv_hbm_frac"] = round(unique / (t_c * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        log(f"{name}: cascade {t_c * 1e3:.1f} us, unique {res['cascade_unique_kv_gbps']:.0f} GB/s")
    log(f"{name}: partition {t_part * 1e3:.1f} us, +reduce {t_both * 1e3:.1f} us, "
        f"logical {res['logical_kv_gbps']:.0f} GB/s, unique {res['unique_kv_gbps']:.0f} GB/s")
    del pools
    torch.cuda.empty_cache()
    return res


def bench_serving(seed=7000, num_requests=96, num_blocks=12000, mixed=False, native=True):
    """The scheduler driving the kernels over a request trace: every step the
    host plans, copies the step's tables to the device through pinned memory
    (one copy), and launches kv_cache_write plus prefill or decode; the step
    is then committed with 'sampled' tokens.  K/V/Q values are random device
    data (they do not change the work).  Reports prompt + generated tokens
    per second of wall time, and the share of it the GPU was busy.  With
    ``mixed`` each step is one batch (decode rows, then prompt chunks) and a
    step holding both runs as one prefill launch.  With ``native`` (the
    default) each step is the library's native serving step
    (``include/pagedattn_serve.h``: plan into pinned memory and copy, then
    write and attend, then complete, one library call each); otherwise the
    loop here stages the arrays and launches the kernels through the
    Python binding."""
    import torch
    import paged_attention_kv_cache_amd as P
    import workloads as W

    Hq, Hkv, D, bs = 32, 8, 128, 32
    rng = np.random.default_rng(seed)
    system = rng.integers(1, 32000, 512).tolist()
    prompts, max_new = {}, {}
    for r in range(num_requests):
        body = rng.integers(1, 32000, int(rng.integers(128, 2049))).tolist()
        prompts[r] = (system + body) if r % 3 == 0 else body
        max_new[r] = int(rng.integers(32, 257))
    kvm = P.KvManager(num_blocks, bs)
    cap_seqs, cap_tokens, cap_blocks = 64, 4096, 128
    sched = P.StepScheduler(kvm, max_batched_tokens=cap_tokens, max_chunk_tokens=512, max_decode_steps=8,
                            min_decode_steps=1, max_seqs=cap_seqs, max_blocks_per_seq=cap_blocks, mixed=mixed)
    for r in range(num_requests):
        sched.add_request(r, prompts[r], max_new[r])
    kc = torch.randn((num_blocks, bs, Hkv, D), device="cuda").to(torch.bfloat16)
    vc = torch.randn_like(kc)
    src_k = torch.randn((cap_tokens, Hkv, D), device="cuda").to(torch.bfloat16)
    src_v = torch.randn_like(src_k)
    src_q = torch.randn((cap_tokens, Hq, D), device="cuda").to(torch.bfloat16)
    out = torch.empty_like(src_q)
    # the step's host arrays travel in one pinned buffer and one copy:
    # int32 words [query_start_loc | context_lens | block tables | slot
    # mapping (int64, 8-byte aligned)]; two such buffers, the host filling
    # one while the other's copy may still wait in the stream behind earlier
    # kernels, a buffer refilled only after the event recorded behind its copy
    o_ctx = cap_seqs + 1
    o_tab = o_ctx + cap_seqs
    o_slots = (o_tab + cap_seqs * cap_blocks + 1) // 2 * 2
    words = o_slots + 2 * cap_tokens

    def views(buf):
        return dict(qsl=buf[:o_ctx], ctx=buf[o_ctx:o_tab],
                    tab=buf[o_tab:o_tab + cap_seqs * cap_blocks].view(cap_seqs, cap_blocks),
                    slots=buf[o_slots:words].view(torch.int64))

    pin_bufs = [torch.zeros(words, dtype=torch.int32).pin_memory() for _ in range(2)]
    pins = [views(b) for b in pin_bufs]
    copied = [None, None]
    dev_buf = torch.empty(words, dtype=torch.int32, device="cuda")
    dev = views(dev_buf)
    ws = torch.zeros(P.pa_decode_workspace_bytes(cap_seqs, Hq, D, cap_blocks * bs, 256), dtype=torch.uint8,
                     device="cuda")
    scale = 1.0 / math.sqrt(D)
    srv = P.Server(sched, Hq, scale, 256, cap_seqs, cap_blocks, cap_tokens) if native else None
    busy = []
    prompt_tokens = decode_tokens = steps = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while True:
        w, a, _ = sched.counts()
        if w == 0 and a == 0:
            break
        if native:
            st = srv.plan()
            n, T = st.num_seqs, st.num_tokens
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            srv.attend(kc, vc, src_k[:T], src_v[:T], src_q[:T], out[:T], workspace=ws)
            e1.record()
            busy.append((e0, e1))
            nd = T if st.kind == P.KIND_DECODE else 0
            if st.kind == P.KIND_MIXED:
                longer = np.flatnonzero(np.diff(st.query_start_loc) != 1)
                nd = int(longer[0]) if longer.size else n
            prompt_tokens += T - nd
            decode_tokens += nd
            srv.complete(rng.integers(1, 32000, n, dtype=np.int32))
            steps += 1
            continue
        st = sched.next_step()
        n, T = st.num_seqs, st.num_tokens
        b = steps % 2
        if copied[b] is not None:
            copied[b].synchronize()  # this set's previous copies have run
        pin = pins[b]
        pin["qsl"][: n + 1].numpy()[:] = st.query_start_loc
        pin["ctx"][:n].numpy()[:] = st.context_lens
        pin["tab"][:n].numpy()[:] = st.block_tables
        pin["slots"][:T].numpy()[:] = st.slot_mapping
        dev_buf.copy_(pin_bufs[b], non_blocking=True)
        copied[b] = torch.cuda.Event()
        copied[b].record()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        P.pa_kv_cache_write(src_k[:T], src_v[:T], kc, vc, dev["slots"][:T])
        if st.kind in (P.KIND_PROMPT, P.KIND_MIXED):
            P.pa_prefill_chunk(src_q[:T], dev["qsl"][: n + 1], kc, vc, dev["tab"][:n], dev["ctx"][:n], scale,
                               st.max_query_len, st.max_context_len, out=out[:T])
            # a mixed step's decode rows come first, one token each
            nd = 0
            if st.kind == P.KIND_MIXED:
                longer = np.flatnonzero(np.diff(st.query_start_loc) != 1)
                nd = int(longer[0]) if longer.size else n
            prompt_tokens += T - nd
            decode_tokens += nd
        else:
            P.pa_decode(src_q[:n], kc, vc, dev["tab"][:n], dev["ctx"][:n], scale, st.max_context_len, 256,
                        out=out[:n], workspace=ws)
            decode_tokens += T
        e1.record()
        busy.append((e0, e1))
        sched.complete_step(rng.integers(1, 32000, n, dtype=np.int32))
        steps += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = sum(a.elapsed_time(b) for a, b in busy)
    st = kvm.stats()
    res = {
        "workload": f"{num_requests} requests, prompts U[128,2048] (+512-token shared system prompt on a third), "
                    f"generation U[32,256]; 32q/8kv, D128, BS32, bf16; budget 4096 tokens, 512-token chunks, "
                    + ("one mixed batch per step" if mixed else "<= 8 decode steps in a row")
                    + f", pool {num_blocks} blocks",
        "policy": "mixed" if mixed else "alternating",
        "driver": "native step (pa_serve_plan / attend / complete)" if native else "python loop over the binding",
        "steps": steps, "prompt_tokens": prompt_tokens, "generated_tokens": decode_tokens,
        "wall_s": round(wall, 3), "tokens_per_s": round((prompt_tokens + decode_tokens) / wall, 1),
        "gpu_busy_frac": round(gpu_ms * 1e-3 / wall, 3),
        "prefix_hit_tokens": st["prefix_hit_tokens"],
    }
    log(f"serving ({res['policy']}): {steps} steps, {prompt_tokens} prompt + {decode_tokens} generated tokens in {wall:.2f} s "
        f"({res['tokens_per_s']:.0f} tokens/s, GPU busy {res['gpu_busy_frac']:.0%})")
    if srv is not None:
        srv.close()
    sched.close()
    kvm.close()
    del kc, vc
    torch.cuda.empty_cache()
    return res


def bench_mfma_ceiling(iters=2048, launches=20):
    """The library's matrix-unit ceiling kernel (pa_mfma_peak: 4 waves per
    SIMD, each 4 independent bf16 MFMA chains, no memory traffic), launched
    back to back: dense bf16 TFLOP/s the device sustains, and the clock
    beside it."""
    import torch
    import paged_attention_kv_cache_amd as P
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    flops = cus * 4 * 4 * iters * 4 * 32768.0
    for _ in range(3):
        P.pa_mfma_peak(sink, iters)
    ms = timed_each(lambda i: P.pa_mfma_peak(sink, iters), launches)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(launches):
        P.pa_mfma_peak(sink, iters)
    e1.record()
    torch.cuda.synchronize()
    t_ms = e0.elapsed_time(e1) / launches
    clk = measure_clock(lambda: P.pa_mfma_peak(sink, iters), launches=12)
    tflops = flops / (t_ms * 1e-3) / 1e12
    log(f"matrix-unit ceiling: {tflops:.0f} TFLOP/s dense bf16 at {clk['ghz']} GHz")
    return {"tflops": round(tflops, 1), "frac_of_nominal": round(tflops / BF16_DENSE_PEAK_TFLOPS, 4),
            "launch_us": round(t_ms * 1e3, 2), "stats": stats_ms(ms), "flops_per_launch": flops,
            "clock_ghz": clk["ghz"]}


def measure_clock(fn=None, launches=30, ticks=200_000):
    """Shader clock in GHz over `ticks` ticks of the GPU's 100 MHz reference
    counter, from the library's clock probe (one wave).  With `fn`, the probe
    runs on a second stream (default priority) while `launches` back-to-back
    calls of fn run on the current one, starting after the second call has
    finished, so it sees the clock those kernels run at; without, the clock
    of an otherwise idle device.  None if the counters disagree with any
    plausible clock."""
    import torch
    import paged_attention_kv_cache_amd as P
    out = torch.zeros(3, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    if fn is None:
        P.pa_clock_probe(out, ticks)
    else:
        side = torch.cuda.Stream()
        ev = torch.cuda.Event()
        for i in range(launches):
            fn()
            if i == 1:
                ev.record()
                side.wait_event(ev)
                P.pa_clock_probe(out, ticks, stream=side)
    torch.cuda.synchronize()
    cycles, tk, steps = (int(x) for x in out.cpu().tolist())
    ghz = cycles / tk * 0.1 if tk > 0 else 0.0
    return {"ghz": round(ghz, 4) if 0.1 < ghz < 4.0 else None, "cycles": cycles, "ref_ticks": tk, "sleep_steps": steps}


def bench_prefill(args, block_size=32):
    import torch
    import paged_attention_kv_cache_amd as P
    import workloads as W

    case = W.chunked_prefill(poison=False, block_size=block_size)
    k = to_dev(case.k_cache, case.dtype)
    v = to_dev(case.v_cache, case.dtype)
    q = to_dev(case.q, case.dtype)
    qsl = torch.from_numpy(case.query_start_loc).cuda()
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    nk = to_dev(case.new_key, case.dtype)
    nv = to_dev(case.new_value, case.dtype)
    sm = torch.from_numpy(case.slot_mapping).cuda()
    out = torch.empty_like(q)
    P.pa_kv_cache_write(nk, nv, k, v, sm)

    def run():
        P.pa_prefill_chunk(q, qsl, k, v, bt, cl, case.scale, case.max_query_len, case.max_context_len,
                           out=out)

    try:
        run()
    except P.PagedAttnError as e:
        if e.status == "PA_ERR_UNSUPPORTED":
            return None
        raise
    for _ in range(5):
        run()
    torch.cuda.synchronize()
    n = 50
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for i in range(n):
        evs[i][0].record()
        run()
        evs[i][1].record()
    torch.cuda.synchronize()
    each = [a.elapsed_time(b) for a, b in evs]
    t_ms = float(np.mean(each))
    # algorithmic FLOPs: 4 * D per visible (query, key) pair per query head
    H, D = case.num_heads, case.head_dim
    pairs = 0
    for i, n_ctx in enumerate(case.context_lens.tolist()):
        ql = int(case.query_lens[i])
        prefix = n_ctx - ql
        pairs += ql * prefix + ql * (ql + 1) // 2
    flops = 4.0 * D * pairs * H
    tflops = flops / (t_ms * 1e-3) / 1e12
    # the matrix unit's peak scales with the clock, which drops under this load
    clk = measure_clock(run)
    at_clock = (tflops / (BF16_DENSE_PEAK_TFLOPS * clk["ghz"] / PEAK_CLOCK_GHZ)) if clk["ghz"] else None
    return dict(us=t_ms * 1e3, tflops=tflops, frac=tflops / BF16_DENSE_PEAK_TFLOPS, flops=flops, stats=stats_ms(each),
                tokens_per_s=int(case.query_start_loc[-1]) / (t_ms * 1e-3), clock=clk,
                frac_at_measured_clock=at_clock, src=source_hash("pa_prefill.hip", "pa_common.h"))


def host_info():
    """What the CPU baseline ran on: cores available to this process, the
    CPU model, numpy and its BLAS."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            blas.append({k: d.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")})
    except ImportError:  # pragma: no cover
        pass
    return {"cores": len(os.sched_getaffinity(0)), "cpu_model": model, "numpy": np.__version__, "blas": blas}


def bench_tiny(steps=200):
    """The tiny fp32 workload: kv_cache_write of its one new token, then
    decode (partition 16 tokens, so that split-K and the reduce run):
    launch-bound, a correctness workload rather than a roofline claim."""
    import torch
    import paged_attention_kv_cache_amd as P
    import workloads as W
    case = W.make_config("tiny_fp32_decode", poison=False)
    k, v = to_dev(case.k_cache, case.dtype), to_dev(case.v_cache, case.dtype)
    nk, nv = to_dev(case.new_key, case.dtype), to_dev(case.new_value, case.dtype)
    sm = torch.from_numpy(case.slot_mapping).cuda()
    q = to_dev(case.q, case.dtype)
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    out = torch.empty((1, q.shape[1], case.v_cache.shape[-1]), dtype=q.dtype, device="cuda")
    ws = torch.empty(max(P.pa_decode_workspace_bytes(1, q.shape[1], case.v_cache.shape[-1], case.max_context_len, 16), 1),
                     dtype=torch.uint8, device="cuda")

    def step(i):
        P.pa_kv_cache_write(nk, nv, k, v, sm)
        P.pa_decode(q, k, v, bt, cl, case.scale, case.max_context_len, 16, out=out, workspace=ws)

    for i in range(10):
        step(i)
    each = timed_each(step, steps)
    return {"workload": "tiny fp32 decode: 1 sequence, 8 q / 2 kv heads, head_dim 64, context 100, block_size 16; "
                        "write of 1 token + decode (partition 16) + reduce",
            "step": stats_ms(each), "kv_bytes": case.kv_bytes_logical()}


def run_only(args):
    """One workload alone, for counter runs: its timing dict as a JSON line."""
    import workloads as W
    name = args.only
    if name == "decode_bs32":
        r = bench_decode(args)
        r = {k: v for k, v in r.items() if k != "case"}
    elif name == "tiny_fp32_decode":
        r = bench_tiny()
    elif name == "stream_read":
        r = bench_stream_ceiling()
    elif name == "mfma_ceiling":
        r = bench_mfma_ceiling()
    elif name.startswith("chunked_prefill"):
        bs = int(name[len("chunked_prefill_bs"):]) if name != "chunked_prefill" else 32
        r = bench_prefill(args, block_size=bs)
    elif name == "long_context_decode":
        r = bench_decode_secondary(name, 512)
    elif name == "decode_batch_bs32_ctx4096":
        r = bench_decode_secondary(name, 1024, case=W.decode_batch(2000, poison=False, fixed_ctx=4096))
    elif name == "decode_batch_bs32_64q_8kv":
        r = bench_decode_secondary(name, 320, case=W.decode_batch(2000, poison=False, num_heads=64))
    elif name == "decode_batch_bs32_k128_v64":
        r = bench_decode_secondary(name, 192, case=W.decode_batch(2000, poison=False, v_head_dim=64))
    else:
        bs = 16 if name.endswith("16") else 8
        r = bench_decode_secondary(name, 512, groups=([0, 16, 32, 48, 64], [64 * bs] * 4), cascade_ps=640)
    print(json.dumps({"only": name, **{k: v for k, v in r.items() if isinstance(v, (int, float, str, dict, list))}}),
          flush=True)


def cpu_baseline(dec_case, pre_case, long_case, seconds):
    """The oracle as it stands (not tuned), in its fp32 mode, with BLAS on
    every host core this process may use, on the same inputs as the GPU
    lines: three legs, each the median of three runs.
      decode:  whole write + decode steps of the bs32 batch, repeated for
               about ``seconds`` per run;
      prefill: the 8 x 512-token chunk workload (the chunk's write, then
               every query row), once per run;
      long:    one sequence of the long-context batch (its blocks only).
    Reported in the GPU lines' units (tokens/s, and KV GB/s under the
    same byte formula)."""
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_limits
    info = host_info()
    threads = info["cores"]
    f32 = np.float32

    def runs3(fn):
        fn()  # first touch of the fresh host arrays, not timed
        vals = [fn() for _ in range(3)]
        return float(np.median(vals)), [round(v, 3) for v in vals]

    with threadpool_limits(threads):
        # decode leg
        q = W.storage_to_f32(dec_case.q, dec_case.dtype)
        kf = W.storage_to_f32(dec_case.k_cache, dec_case.dtype)
        vf = W.storage_to_f32(dec_case.v_cache, dec_case.dtype)
        nk = W.storage_to_f32(dec_case.new_key, dec_case.dtype)
        nv = W.storage_to_f32(dec_case.new_value, dec_case.dtype)

        def dec_run():
            steps, t0 = 0, time.perf_counter()
            while True:
                k2, v2 = oracle.kv_cache_write(kf, vf, nk, nv, dec_case.slot_mapping)
                oracle.paged_decode(q, k2, v2, dec_case.block_tables, dec_case.context_lens, dec_case.scale, f32)
                steps += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            return dec_case.num_seqs * steps / (time.perf_counter() - t0)

        dec_tps, dec_runs = runs3(dec_run)
        del kf, vf
        legs = [{"leg": "decode", "tokens_per_s": round(dec_tps, 1), "runs_tokens_per_s": dec_runs,
                 "kv_gbps": round(dec_tps / dec_case.num_seqs * dec_case.kv_bytes_logical() / 1e9, 3),
                 "sample": f"whole write + decode steps of the bs32 batch for ~{seconds:.0f} s per run"}]
        # prefill leg
        if pre_case is not None:
            pq = W.storage_to_f32(pre_case.q, pre_case.dtype)
            pk = W.storage_to_f32(pre_case.k_cache, pre_case.dtype)
            pv = W.storage_to_f32(pre_case.v_cache, pre_case.dtype)
            pnk = W.storage_to_f32(pre_case.new_key, pre_case.dtype)
            pnv = W.storage_to_f32(pre_case.new_value, pre_case.dtype)
            tq = int(pre_case.query_start_loc[-1])

            def pre_run():
                t0 = time.perf_counter()
                k2, v2 = oracle.kv_cache_write(pk, pv, pnk, pnv, pre_case.slot_mapping)
                oracle.paged_prefill(pq, pre_case.query_start_loc, k2, v2, pre_case.block_tables,
                                     pre_case.context_lens, pre_case.scale, f32)
                return tq / (time.perf_counter() - t0)

            pre_tps, pre_runs = runs3(pre_run)
            del pk, pv
            legs.append({"leg": "prefill", "tokens_per_s": round(pre_tps, 1), "runs_tokens_per_s": pre_runs,
                         "sample": "the whole 8 x 512-token chunk workload per run"})
        # long-context leg: sequence 0's blocks only
        if long_case is not None:
            n = int(long_case.context_lens[0])
            nb = -(-n // long_case.block_size)
            ids = long_case.block_tables[0, :nb]
            lk = W.storage_to_f32(long_case.k_cache[ids], long_case.dtype)
            lv = W.storage_to_f32(long_case.v_cache[ids], long_case.dtype)
            lq = W.storage_to_f32(long_case.q[:1], long_case.dtype)
            table = np.arange(nb, dtype=np.int32)[None, :]

            def long_run():
                t0 = time.perf_counter()
                oracle.paged_decode(lq, lk, lv, table, np.array([n], dtype=np.int32), long_case.scale, f32)
                return 1.0 / (time.perf_counter() - t0)

            long_tps, long_runs = runs3(long_run)
            row = long_case.num_kv_heads * (long_case.head_dim + long_case.v_head_dim) * 2
            legs.append({"leg": "long_context", "tokens_per_s": round(long_tps, 3), "runs_tokens_per_s": long_runs,
                         "kv_gbps": round(long_tps * n * row / 1e9, 3),
                         "sample": f"one decode token of sequence 0 ({n} context tokens, its {nb} blocks)"})
    return dict(value=round(dec_tps, 1), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"decode leg: whole write + decode steps of the bs32 batch ({dec_case.num_seqs} sequences), "
                       f"fp32 oracle, {threads} BLAS threads, median of 3 runs of ~{seconds:.0f} s",
                threads=threads, host=info, legs=legs)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode and prefill kernels "
                                   "are measured on a single MI355X (--gpus 1)"}))
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import paged_attention_kv_cache_amd as P
    import workloads as W
    P.load_library()

    if args.only:
        if args.copy_calibration:
            src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
            del src
        run_only(args)
        return
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)          # 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del src, dst
    clock_idle_before = measure_clock()
    dec = bench_decode(args)
    ceiling = bench_stream_ceiling()
    # the same read at the partition kernel's own byte count (launch ramp
    # and tail weigh as much as in the kernel)
    ceiling_same = bench_stream_ceiling(dec["part_bytes"])
    log(f"plain sequential read: {ceiling['gbps']:.0f} GB/s at 1 GiB, {ceiling_same['gbps']:.0f} GB/s at "
        f"{dec['part_bytes'] / 1e6:.0f} MB")
    pre = None if args.no_prefill else bench_prefill(args)
    mceil = None if args.no_prefill else bench_mfma_ceiling()
    case = dec["case"]
    tokens_per_s = dec["S"] / (dec["ms_step"] * 1e-3)
    traffic = traffic_from_profiles("decode_partition", dec["src"], dec["ps"])
    step_gbps = dec["kv_bytes"] / (dec["ms_step"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "bf16 paged decode batch: 32 sequences, context U[512,4096], 32 q / 8 kv heads, "
                        "head_dim 128, block_size 32, pool 1.25x; step = pa_decode_append (the 32 new "
                        "tokens' K/V rows written into the cache by the partition kernel that attends to "
                        "them) + reduce",
            "num_seqs": dec["S"],
            "context_tokens": int(case.context_lens.sum()),
            "block_size": case.block_size,
            "partition_size": dec["ps"],
            "kv_pool_rotations": dec["R"],
        },
        # KV bytes of the step over the step time (what tokens/s describes)
        "kv_gbps": round(step_gbps, 1),
        "kv_hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        # the same bytes over the partition kernel's own launch time
        "kv_gbps_partition_kernel": round(dec["achieved"], 1),
        "kv_hbm_frac_partition_kernel": round(dec["achieved"] / HBM_PEAK_GBPS, 4),
        "stream_read_ceiling": ceiling,
        "partition_kernel_frac_of_stream_ceiling": round(dec["achieved"] / ceiling["gbps"], 4),
        "stream_read_ceiling_same_bytes": ceiling_same,
        "partition_kernel_frac_of_same_bytes_ceiling": round(dec["achieved"] / ceiling_same["gbps"], 4),
        "timing": {
            "step_cold": dec["step_stats"],
            "step_warm_ms": round(dec["ms_step_warm"], 5),
            "step_warm_tokens_per_s": round(dec["S"] / (dec["ms_step_warm"] * 1e-3), 1),
            "partition_kernel": dec["part_stats"],
        },
        "roofline": {
            "kernel": "decode_partition_mfma_kernel<128, 128, 4>",
            "bound": "hbm",
            "achieved": round(dec["achieved"], 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec["achieved"] / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dec["part_bytes"],
            "avg_launch_us": round(dec["t_part_b2b"] * 1e3, 2),
        },
        # the same step as three launches: kv_cache_write, partition, reduce
        "step_three_launches": {
            "api": "pa_kv_cache_write + pa_decode_partition + pa_decode_reduce",
            "ms_per_step": round(dec["ms_step_three"], 5),
            "tokens_per_s": round(dec["S"] / (dec["ms_step_three"] * 1e-3), 1),
            "kernel_us": {"kv_cache_write": round(dec["t_write"] * 1e3, 2),
                          "decode_partition": round(dec["t_part"] * 1e3, 2),
                          "decode_reduce": round(dec["t_red"] * 1e3, 2)},
        },
    }
    if pre is not None:
        line["prefill_chunk"] = {
            "workload": "8 sequences x 512-token chunk over prefix U[0,3584], 32q/8kv, D128, BS32, bf16",
            "us": round(pre["us"], 2), "tokens_per_s": round(pre["tokens_per_s"], 1), "timing": pre["stats"],
            "roofline": {"kernel": "prefill_chunk_kernel<128, 128, 4>", "bound": "mfma", "achieved": round(pre["tflops"], 1), "peak": BF16_DENSE_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(pre["frac"], 4),
                         "traffic": traffic_from_profiles("prefill_chunk", pre["src"]),
                         "algorithmic_flops_per_launch": pre["flops"]},
            "mfma_ceiling": mceil,
            "frac_of_mfma_ceiling": round(pre["tflops"] / mceil["tflops"], 4),
            "clock_during_launches": pre["clock"],
            "mfma_frac_at_measured_clock": round(pre["frac_at_measured_clock"], 4) if pre["frac_at_measured_clock"] else None,
        }
    if not args.quick and pre is not None:
        line["prefill_other_block_sizes"] = []
        for bs in (16, 8):
            p2 = bench_prefill(args, block_size=bs)
            line["prefill_other_block_sizes"].append({
                "block_size": bs, "us": round(p2["us"], 2), "tokens_per_s": round(p2["tokens_per_s"], 1),
                "tflops": round(p2["tflops"], 1), "mfma_frac": round(p2["frac"], 4)})
    line["tiny_fp32_decode"] = bench_tiny()
    long_case = None if args.quick else W.make_config("long_context_decode", poison=False)
    if not args.quick:
        line["decode_other_workloads"] = [
            bench_decode_secondary("long_context_decode", 512, case=long_case),
            # the metric's literal shape: 32 sequences of exactly 4096 tokens
            bench_decode_secondary("decode_batch_bs32_ctx4096", 1024,
                                   case=W.decode_batch(2000, poison=False, fixed_ctx=4096)),
            # eight query heads per kv head: 64 q over the same 8 kv heads and K/V bytes
            bench_decode_secondary("decode_batch_bs32_64q_8kv", 320,
                                   case=W.decode_batch(2000, poison=False, num_heads=64)),
            # a value head dim of its own: 128-wide keys, 64-wide values
            bench_decode_secondary("decode_batch_bs32_k128_v64", 192,
                                   case=W.decode_batch(2000, poison=False, v_head_dim=64)),
            bench_decode_secondary("prefix_shared_decode_bs16", 512, groups=([0, 16, 32, 48, 64], [64 * 16] * 4),
                                   cascade_ps=640),
            bench_decode_secondary("prefix_shared_decode_bs8", 512, groups=([0, 16, 32, 48, 64], [64 * 8] * 4),
                                   cascade_ps=640),
        ]
        bench_serving(num_requests=8)  # untimed: the first pass on a device pays one-time costs
        line["serving_loop"] = bench_serving()
        line["serving_loop_mixed"] = bench_serving(mixed=True)
        line["serving_loop_python_driver"] = bench_serving(native=False)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (decode, prefill and long-context legs, median of 3 each)")
        pre_case = None if args.no_prefill else W.chunked_prefill(poison=False)
        line["cpu_baseline"] = cpu_baseline(case, pre_case, long_case, args.cpu_seconds)
    line["clock_idle_ghz"] = {"before": clock_idle_before["ghz"], "after": measure_clock()["ghz"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
