/*
 * pagedattn_bench.h - measurement helpers of the paged-attention library
 * (MI355X, gfx950).  Not attention operations: they exist so that a
 * benchmark can measure, on the same device and in the same run as the
 * kernels, the HBM read rate that a plain sequential read reaches (the
 * practical ceiling of the bandwidth-bound decode), the dense bf16 rate
 * the matrix units sustain (that of the matrix-bound prefill) and the
 * shader clock (the matrix unit's peak scales with it).
 */
#ifndef PAGEDATTN_BENCH_H
#define PAGEDATTN_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of the device buffer `buf` (a multiple of 16) once,
 * sequentially, one 16-byte load per thread per step of a grid-stride loop
 * over 4 work-groups of 256 threads per compute unit, on `stream` (a
 * hipStream_t; NULL for the null stream).
 * `sink` is a device pointer to 4 writable bytes that the kernel writes
 * only in the rare case that the loaded data folds to one fixed word.
 * Returns PA_OK, or PA_ERR_NULL / PA_ERR_SHAPE / PA_ERR_HIP with the
 * message set (pa_last_error_message). */
int pa_stream_read(const void *buf, size_t bytes, void *sink, void *stream);

/* Most rounds pa_mfma_peak runs per wave. */
#define PA_MFMA_PEAK_MAX_ITERS 65536

/* Enqueues the matrix-unit ceiling kernel on `stream`: 4 work-groups of 4
 * waves per compute unit, every wave running `iters` rounds (1 ..
 * PA_MFMA_PEAK_MAX_ITERS) of four independent chains of
 * v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic.
 * One launch performs (compute units x 4) x 4 x iters x 4 x 32768 FLOP; its
 * time gives the dense bf16 rate the device sustains (at the clock that
 * load runs it at).  `sink` is a device pointer to 4 writable bytes that
 * the kernel writes only if the folded accumulators equal one fixed value.
 * Returns PA_OK, or PA_ERR_NULL / PA_ERR_SHAPE / PA_ERR_HIP with the
 * message set. */
int pa_mfma_peak(void *sink, int32_t iters, void *stream);

/* Longest interval pa_clock_probe measures: 10 ms of the 100 MHz reference. */
#define PA_CLOCK_PROBE_MAX_TICKS 1000000

/* Enqueues one wave on `stream` that measures the shader clock over `ticks`
 * ticks (1 .. PA_CLOCK_PROBE_MAX_TICKS) of the GPU's constant 100 MHz
 * reference counter and writes three uint64 values to the device buffer
 * `out` (24 bytes, caller-owned): shader cycles elapsed (s_memtime), reference
 * ticks elapsed (s_memrealtime) and the number of sleep steps taken; the
 * clock in Hz is cycles / ticks x 1e8.  Enqueued on a second stream while
 * other kernels run, it measures the clock they run at (one wave on one
 * CU).  Its loop also stops after ticks x 16 + 1024 sleep steps, so it ends
 * even if a counter does not advance (then the ticks value falls short).
 * Returns PA_OK, or PA_ERR_NULL / PA_ERR_SHAPE / PA_ERR_HIP with the
 * message set. */
int pa_clock_probe(void *out, int64_t ticks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_BENCH_H */
