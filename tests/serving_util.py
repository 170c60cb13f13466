"""The serving loop shared by the CPU and GPU serving tests: the host block
manager and step scheduler plan each step, a backend writes the new tokens'
K/V through the step's slot mapping and runs prefill or decode over the
step's block tables, and every output row is checked against the oracle's
attention over the request's dense K/V (which never goes through a block
table)."""

import numpy as np

import oracle
import workloads as W

from gpu_util import assert_close, log


class DenseKV:
    """Per-request K/V of positions computed so far, extended incrementally."""

    def __init__(self, trace):
        self.trace = trace
        self.k, self.v, self.state = {}, {}, {}

    def get(self, rid, tokens, n):
        have = 0 if rid not in self.k else self.k[rid].shape[0]
        if n > have:
            k, v, st = self.trace.kv(tokens[:n], start=have, state=self.state.get(rid))
            self.k[rid] = k if have == 0 else np.concatenate([self.k[rid], k])
            self.v[rid] = v if have == 0 else np.concatenate([self.v[rid], v])
            self.state[rid] = st
        return self.k[rid][:n], self.v[rid][:n]


class OracleBackend:
    """The oracle's paged functions over a host pool (CPU)."""

    def __init__(self, trace):
        shape = (trace.num_blocks, trace.block_size, trace.num_kv_heads, trace.head_dim)
        self.kc = np.zeros(shape, np.float64)
        self.vc = np.zeros(shape, np.float64)

    def grow(self, kvm, new_num_blocks):
        pad = lambda c: np.concatenate([c, np.zeros((new_num_blocks - c.shape[0],) + c.shape[1:], c.dtype)])
        self.kc, self.vc = pad(self.kc), pad(self.vc)
        kvm.grow(new_num_blocks)

    def step(self, st, keys, vals, qs, scale, partition_size):
        f = lambda x: W.storage_to_f32(x, W.BF16).astype(np.float64)
        self.kc, self.vc = oracle.kv_cache_write(self.kc, self.vc, f(keys), f(vals), st.slot_mapping)
        if st.kind in (1, 3):  # prompt or mixed: decode rows are chunks of one token
            return oracle.paged_prefill(f(qs), st.query_start_loc, self.kc, self.vc, st.block_tables,
                                        st.context_lens, scale)
        return oracle.paged_decode(f(qs), self.kc, self.vc, st.block_tables, st.context_lens, scale)


class LibraryBackend:
    """The library's kernels over a device pool (GPU)."""

    def __init__(self, trace):
        from gpu_util import torch
        t = torch()
        self.t = t
        shape = (trace.num_blocks, trace.block_size, trace.num_kv_heads, trace.head_dim)
        self.kc = t.zeros(shape, dtype=t.bfloat16, device="cuda")
        self.vc = t.zeros_like(self.kc)

    def grow(self, kvm, new_num_blocks):
        import paged_attention_kv_cache_amd as P
        self.kc, self.vc = P.grow_pool(kvm, self.kc, self.vc, new_num_blocks)

    def step(self, st, keys, vals, qs, scale, partition_size):
        import paged_attention_kv_cache_amd as P
        from gpu_util import to_dev, to_host_f32
        t = self.t
        dev_k, dev_v, dev_q = to_dev(keys, W.BF16), to_dev(vals, W.BF16), to_dev(qs, W.BF16)
        slots = t.from_numpy(st.slot_mapping.copy()).cuda()
        tables = t.from_numpy(st.block_tables.copy()).cuda()
        lens = t.from_numpy(st.context_lens.copy()).cuda()
        P.pa_kv_cache_write(dev_k, dev_v, self.kc, self.vc, slots)
        if st.kind in (P.KIND_PROMPT, P.KIND_MIXED):  # mixed: decode rows are chunks of one token
            qstart = t.from_numpy(st.query_start_loc.copy()).cuda()
            out = P.pa_prefill_chunk(dev_q, qstart, self.kc, self.vc, tables, lens, scale, st.max_query_len,
                                     st.max_context_len)
        else:
            out = P.pa_decode(dev_q, self.kc, self.vc, tables, lens, scale, st.max_context_len, partition_size)
        t.cuda.synchronize()
        return to_host_f32(out, W.BF16)


class NativeBackend(LibraryBackend):
    # decode-row context from which a mixed step splits its decode rows off
    # to split-K decode (small here, so that the short test contexts take
    # that path too; 0 keeps every mixed step in one prefill launch)
    mixed_split_context = 1

    """The library's native serving step (pa_serve_plan / pa_serve_attend /
    pa_serve_complete of include/pagedattn_serve.h): the scheduler plans into
    pinned memory, one copy moves the step's arrays to the device, and the
    library launches the write and the attention."""

    def attach(self, sched, trace, max_seqs, max_blocks_per_seq, max_tokens, partition_size):
        import paged_attention_kv_cache_amd as P
        t = self.t
        self.server = P.Server(sched, trace.num_heads, trace.scale, partition_size, max_seqs, max_blocks_per_seq,
                               max_tokens, mixed_split_context=self.mixed_split_context)
        self.shape = (trace.num_heads, trace.head_dim)
        self.ws = None
        if partition_size:
            need = P.pa_decode_workspace_bytes(max_seqs, trace.num_heads, trace.head_dim,
                                               max_blocks_per_seq * trace.block_size, partition_size)
            self.ws = t.empty(max(need, 1), dtype=t.uint8, device="cuda")

    def plan(self):
        return self.server.plan()

    def step(self, st, keys, vals, qs, scale, partition_size):
        from gpu_util import to_dev, to_host_f32
        t = self.t
        dev_k, dev_v, dev_q = to_dev(keys, W.BF16), to_dev(vals, W.BF16), to_dev(qs, W.BF16)
        out = t.empty((st.num_tokens,) + self.shape, dtype=t.bfloat16, device="cuda")
        self.server.attend(self.kc, self.vc, dev_k, dev_v, dev_q, out, workspace=self.ws)
        t.cuda.synchronize()
        return to_host_f32(out, W.BF16)

    def complete(self, sampled):
        self.server.complete(sampled)

    def close(self):
        self.server.close()


def serve_and_check(trace, backend, partition_size=0, max_batched_tokens=256, max_chunk_tokens=128,
                    max_seqs=8, max_blocks_per_seq=32, tag="", grow_at=None, mixed=False):
    """Runs the trace to completion; returns a summary dict.  ``grow_at``
    maps a step index to a larger pool size: before that step the backend's
    pool is moved into the larger allocation and the manager extended."""
    import paged_attention_kv_cache_amd as P

    m = P.KvManager(trace.num_blocks, trace.block_size)
    s = P.StepScheduler(m, max_batched_tokens=max_batched_tokens, max_chunk_tokens=max_chunk_tokens,
                        max_seqs=max_seqs, max_blocks_per_seq=max_blocks_per_seq, mixed=mixed)
    for rid, prompt in trace.prompts.items():
        s.add_request(rid, prompt, trace.max_new[rid])
    native = hasattr(backend, "plan")
    if native:
        backend.attach(s, trace, max_seqs, max_blocks_per_seq, max(max_batched_tokens, max_seqs), partition_size)
    H, Hkv, D = trace.num_heads, trace.num_kv_heads, trace.head_dim
    expected = {rid: list(p) for rid, p in trace.prompts.items()}
    gen = {rid: 0 for rid in trace.prompts}
    dense = DenseKV(trace)
    recomputed, kinds, worst = set(), [], 0.0
    reached = {rid: 0 for rid in trace.prompts}  # K/V positions computed before (a restart goes back)
    for step in range(5000):
        w, a, _ = s.counts()
        if w == 0 and a == 0:
            break
        if grow_at and step in grow_at:
            log(f"serving{tag}: pool grows to {grow_at[step]} blocks before step {step}")
            backend.grow(m, grow_at[step])
        st = backend.plan() if native else s.next_step()
        assert st.kind in ((P.KIND_PROMPT, P.KIND_DECODE, P.KIND_MIXED) if mixed else (P.KIND_PROMPT, P.KIND_DECODE))
        kinds.append(st.kind)
        ids = st.request_ids.tolist()
        qsl = st.query_start_loc.astype(np.int64)
        ctx = st.context_lens.astype(np.int64)
        T = st.num_tokens
        keys = np.empty((T, Hkv, D), np.uint16)
        vals = np.empty_like(keys)
        qs = np.empty((T, H, D), np.uint16)
        firsts = []
        for i, rid in enumerate(ids):
            n = int(qsl[i + 1] - qsl[i])
            first = int(ctx[i]) - n
            firsts.append(first)
            k, v = dense.get(rid, expected[rid], int(ctx[i]))
            keys[qsl[i]:qsl[i + 1]] = k[first:]
            vals[qsl[i]:qsl[i + 1]] = v[first:]
            qs[qsl[i]:qsl[i + 1]] = trace.q(rid, first, n)
            if first < reached[rid]:
                recomputed.add(rid)
            reached[rid] = max(reached[rid], int(ctx[i]))
        log(f"serving{tag} ps={partition_size} step {step} kind {st.kind} seqs {st.num_seqs} tokens {T} "
            f"max_ctx {st.max_context_len}")
        got = backend.step(st, keys, vals, qs, trace.scale, partition_size)
        for i, rid in enumerate(ids):
            c = int(ctx[i])
            k, v = dense.get(rid, expected[rid], c)
            qf = W.storage_to_f32(qs[qsl[i]:qsl[i + 1]], W.BF16)
            ref = oracle.attention(qf, W.storage_to_f32(k, W.BF16), W.storage_to_f32(v, W.BF16), trace.scale,
                                   np.arange(firsts[i], c))
            err, _ = assert_close(got[qsl[i]:qsl[i + 1]], ref, W.BF16,
                                  f"step {step} request {rid} ctx {c} kind {st.kind}")
            worst = max(worst, err)
        sampled = [trace.sampled_token(rid, int(ctx[i])) for i, rid in enumerate(ids)]
        if native:
            backend.complete(sampled)
        else:
            s.complete_step(sampled)
        for i, rid in enumerate(ids):
            if int(ctx[i]) < len(expected[rid]):
                continue
            if gen[rid] < trace.max_new[rid]:
                expected[rid].append(sampled[i])
                gen[rid] += 1
    else:
        raise AssertionError("serving did not finish")
    stats = m.stats()
    assert s.counts() == (0, 0, len(trace.prompts))
    assert all(gen[r] == trace.max_new[r] for r in gen)
    if native:
        backend.close()
    s.close()
    m.close()
    return {"steps": len(kinds), "kinds": kinds, "worst": worst, "recomputed": len(recomputed), "stats": stats}
