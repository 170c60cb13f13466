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


def test_mfma_ceiling_probe():
    """The matrix-unit ceiling kernel runs, writes nothing, and its rate is
    one the device can reach: above a fifth of the published dense bf16
    peak and not above it."""
    import paged_attention_kv_cache_amd as P
    t = torch()
    sink = t.zeros(1, dtype=t.float32, device="cuda")
    cus = t.cuda.get_device_properties(0).multi_processor_count
    iters = 1024
    P.pa_mfma_peak(sink, iters)
    t.cuda.synchronize()
    e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        P.pa_mfma_peak(sink, iters)
    e1.record()
    t.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    tflops = cus * 4 * 4 * iters * 4 * 32768.0 / (ms * 1e-3) / 1e12
    log(f"mfma ceiling: {tflops:.0f} TFLOP/s over {cus} CUs")
    print(f"mfma ceiling: {tflops:.0f} TFLOP/s ({ms * 1e3:.1f} us per launch)")
    assert 500.0 < tflops <= 2500.0 * 1.02
    assert float(sink.item()) == 0.0
