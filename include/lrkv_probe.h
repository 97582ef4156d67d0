/*
 * lrkv_probe.h - measurement kernels that frame the decode's numbers on one
 * MI355X (gfx950): a plain HBM read stream (the practical bandwidth ceiling a
 * kernel reading the same bytes can reach) and a bounded spin that keeps the GPU
 * busy while a host loop enqueues the launches to be timed.  They compute
 * nothing of the method; the benchmark loads them from liblrkv_probe.so.
 *
 * Conventions as in lrkv.h: device pointers are plain HIP device addresses,
 * every argument is checked on the host before any HIP call, work is enqueued on
 * `stream` and returns at once.  Return values are lrkv_status codes
 * (0 = ok, 1 = null pointer, 2 = a size out of range, 5 = misaligned,
 * 8 = launch failure).
 */
#ifndef LRKV_PROBE_H
#define LRKV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *lrkv_stream_t; /* same object as hipStream_t */

/*
 * Reads `bytes` bytes from `src` once with 16-byte vector loads: `grid`
 * workgroups of 256 threads sweep the buffer in chunks of 256 * unroll 16-byte
 * pieces (chunk k of the sweep goes to workgroup k mod grid), each thread keeping
 * `unroll` loads in flight; `nontemporal` != 0 marks the loads as streaming.
 * The loaded words are folded together and stored to sink[blockIdx] only for
 * one particular value, so the loads cannot be dropped and (in practice) nothing
 * is written.
 *   src:  device, 16-byte aligned; bytes: > 0, a multiple of 16.
 *   sink: device uint32 [grid], caller-owned.
 *   grid: 1 .. 65535; unroll: 1, 2, 4 or 8.
 */
int32_t lrkv_probe_read(const void *src, int64_t bytes, uint32_t *sink, int32_t grid, int32_t unroll,
                        int32_t nontemporal, lrkv_stream_t stream);

/*
 * One wave waits until `ticks` ticks of the GPU's constant-rate wall clock have
 * passed since it started (sleeping between reads of the clock), then ends.  The
 * wait always ends: the clock only moves forward.  sink: device uint32 [1],
 * written only in the impossible case of a negative tick count having been seen.
 *   ticks: 0 .. 2^32 (lrkv_probe_wall_clock_khz gives the clock's rate).
 */
int32_t lrkv_probe_spin(int64_t ticks, uint32_t *sink, lrkv_stream_t stream);

/* The rate of the wall clock used by lrkv_probe_spin, in kHz, for the current
 * device (0 if it cannot be read). */
int32_t lrkv_probe_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* LRKV_PROBE_H */
