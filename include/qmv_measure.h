/*
 * qmv_measure.h -- C ABI of libqmv_measure.so, the two reference kernels the
 * benchmark measures the quantized matvec against on the same GPU:
 *
 *  - a plain streaming read (16-byte loads, every byte read once), whose rate
 *    is the clean-stream ceiling that effective bandwidth is audited against
 *    ("raw-Metal loop playbook", the audit of effective GB/s against what
 *    clean streams reach on the same silicon; "Gemma4 raw-Metal loop on A19 --
 *    findings + the remaining (parked) levers", "Traps": only streams of
 *    about 100 MB and more give true DRAM numbers);
 *  - an empty kernel, whose back-to-back rate is the dispatch floor that
 *    bounds the short calls ("Gemma4 raw-Metal loop on A19", "What moved the
 *    needle": per-dispatch overhead).
 *
 * Neither computes anything of the method; they exist only to be timed.
 * Pointers are device memory owned by the caller; calls are asynchronous on
 * `stream` (a hipStream_t, NULL = the null stream) and allocate nothing.
 */
#ifndef QMV_MEASURE_H
#define QMV_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at `src` (16-byte aligned, bytes a multiple of 16) once
 * with 16-byte non-temporal loads, grid-stride over `grid` workgroups of 256
 * lanes (grid <= 0: 2048), and write one word per workgroup (an XOR of what
 * it read, so the loads cannot be dropped) to sink[0 .. grid).
 * Returns 0, 1 for an invalid argument (null pointer, misalignment, zero or
 * ragged size), 5 if the launch failed. */
int qmv_measure_stream_read(const void *src, size_t bytes, uint32_t *sink, int grid, void *stream);

/* Launch one empty kernel (one workgroup of 64 lanes).  Returns 0, or 5 if
 * the launch failed. */
int qmv_measure_empty(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_MEASURE_H */
