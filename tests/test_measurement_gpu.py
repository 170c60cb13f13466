"""The measurement helpers of include/pagedattn_bench.h on the GPU: the
shader-clock probe reports a clock the device can run at, over the interval
it was asked for, and the stream-read probe reads a buffer without writing
its sink."""

import pytest

from gpu_util import log, torch

pytestmark = pytest.mark.gpu


def test_clock_probe_idle_and_under_load():
    import paged_attention_kv_cache_amd as P
    t = torch()
    out = t.zeros(3, dtype=t.int64, device="cuda")
    log("clock probe: 1 ms idle")
    P.pa_clock_probe(out, 100_000)
    t.cuda.synchronize()
    cycles, ticks, steps = (int(x) for x in out.cpu().tolist())
    assert ticks >= 100_000 and steps < 100_000 * 16 + 1024
    ghz = cycles / ticks * 0.1
    print(f"idle: {cycles} cycles over {ticks} ticks: {ghz:.3f} GHz, {steps} sleep steps")
    assert 0.1 < ghz <= 2.5
    # beside a stream of reads on the current stream
    buf = t.ones(1 << 27, dtype=t.int16, device="cuda")
    sink = t.zeros(1, dtype=t.int32, device="cuda")
    side = t.cuda.Stream()
    out.zero_()
    t.cuda.synchronize()
    for i in range(40):
        P.pa_stream_read(buf, sink)
        if i == 1:
            ev = t.cuda.Event()
            ev.record()
            side.wait_event(ev)
            P.pa_clock_probe(out, 20_000, stream=side)
    t.cuda.synchronize()
    cycles, ticks, steps = (int(x) for x in out.cpu().tolist())
    ghz = cycles / ticks * 0.1
    print(f"under load: {ghz:.3f} GHz")
    assert ticks >= 20_000 and 0.1 < ghz <= 2.5
    assert int(sink.item()) == 0
