/*
 * pagedattn_bench.h - measurement helper of the paged-attention library
 * (MI355X, gfx950).  Not an attention operation: it exists so that a
 * benchmark can measure, on the same device and in the same run as the
 * decode kernels, the HBM read rate that a plain sequential read reaches,
 * the practical ceiling of the bandwidth-bound decode.
 */
#ifndef PAGEDATTN_BENCH_H
#define PAGEDATTN_BENCH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of the device buffer `buf` (a multiple of 16) once,
 * sequentially, with 16-byte non-temporal loads from 8 work-groups per
 * compute unit, on `stream` (a hipStream_t; NULL for the null stream).
 * `sink` is a device pointer to 4 writable bytes that the kernel writes
 * only in the rare case that the loaded data folds to one fixed word.
 * Returns PA_OK, or PA_ERR_NULL / PA_ERR_SHAPE / PA_ERR_HIP with the
 * message set (pa_last_error_message). */
int pa_stream_read(const void *buf, size_t bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_BENCH_H */
