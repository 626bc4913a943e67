/*
 * bi_measure.h -- measured ceilings of the GPU, for benchmarking only.
 *
 * The benchmark reports each kernel's throughput against the datasheet peak
 * and against what this GPU measurably sustains: a plain streaming read of
 * HBM (every byte once) and a loop of independent bf16 matrix-core
 * instructions with no memory traffic.  Flops count two per multiply-add,
 * the convention of the page "Исследование производительности Laya MLX"
 * (its arithmetic model of a matrix product).  These calls are not part of
 * the batch-invariant compute path and no other entry point uses them.
 *
 * Both enqueue one kernel on `stream` (a hipStream_t, NULL = legacy default
 * stream) and return without synchronising; time them with events.
 */
#ifndef BI_MEASURE_H
#define BI_MEASURE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at device pointer `src` exactly once (16-byte aligned,
 * bytes a multiple of 16) with `workgroups` workgroups of 256 threads.
 * `sink` is a device buffer of at least workgroups * 256 * 4 bytes that the
 * kernel may write (in practice it writes nothing).  Returns 0 when the
 * kernel was enqueued, 1 for bad arguments, 4 for a launch error. */
int bi_measure_stream_read(const void *src, size_t bytes, void *sink, int workgroups, void *stream);

/* Runs `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16 chains in
 * every wavefront of `workgroups` workgroups of 4 wavefronts.  `sink` is as
 * above.  Returns the flops the launch performs (2 per multiply-add), or a
 * negative value for bad arguments or a launch error. */
double bi_measure_mfma(void *sink, int workgroups, int iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_MEASURE_H */
