/*
 * libsq_probe.so: measured ceilings for the benchmark, not part of the layer's
 * API.  Each call only queues one kernel on the given stream (a hipStream_t as
 * void*; NULL is the default stream); the caller times it with events.
 * Return: 0 queued; 1 bad argument (nothing queued); 7 the launch failed.
 */
#ifndef SQ_PROBE_H
#define SQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The int8 matrix cores' sustained rate with the product kernel's register
 * pattern: `blocks` workgroups of 8 waves (two per SIMD at one workgroup per
 * CU); each wave loads 8 weight operands of 16 bytes per lane from `a` and 2
 * activation operands from `b`, once, then issues iters x 16
 * v_mfma_i32_16x16x64_i8.  Work = blocks * 8 * iters * 16 * 2 * 16 * 16 * 64
 * int8 ops.
 *   a    device, at least 8 KiB per wave slot: 8 * 8 * 1024 = 64 KiB
 *   b    device, at least 2 * 8 * 1024 = 16 KiB
 *   out  device int32 [blocks * 512], written (sums, so no work is dead)
 */
int sqp_mfma_rate(const int8_t *a, const int8_t *b, int iters, int blocks, int *out,
                  void *stream);

/*
 * A streaming read of `bytes` (a multiple of 16) from `buf` with 16-byte
 * non-temporal loads, grid-stride over `blocks` workgroups of 256 threads.
 *   out  device int32 [blocks * 256], written
 */
int sqp_stream_read(const void *buf, int64_t bytes, int blocks, int *out, void *stream);

/* The constant rate of the device's real-time counter (s_memrealtime), kHz. */
int sqp_wall_clock_khz(int *khz);

/*
 * One wave on one CU reads the shader cycle counter and the real-time counter,
 * sleeps until `ticks` real-time ticks have passed (at most `max_iter` sleeps
 * of 8 x 64 cycles), and reads both again:
 *   out  device uint64 [5], written: real-time start and end, cycles start
 *        and end, sleeps taken.
 * Queued on a second stream just before other work, it measures the shader
 * clock that work runs at: (cycles end - start) / (real-time span).
 */
int sqp_clock_watch(uint64_t ticks, uint64_t max_iter, uint64_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif
