/*
 * attn_probe.h - HBM read-bandwidth probe for AMD MI355X (gfx950).
 *
 * Not part of the attention path: the benchmark uses it to measure the
 * practical read ceiling of the device, against which the split-KV decode pass
 * is reported.  Flash-attention issue #1248 ("where is flash decoding second
 * stage (reduce) code?") notes that decoding runs close to the speed of a
 * memory copy, since it only streams the K/V cache once; this probe is that
 * copy's read half, measured on the same bytes.
 *
 * attn_probe_read reads `bytes` bytes of device memory starting at `buf`, in
 * chunks of `chunk` bytes whose starts lie `stride` bytes apart (chunk ==
 * stride: one contiguous range; the buffer must hold (bytes / chunk - 1) *
 * stride + chunk bytes), with 16-byte nontemporal loads, and writes one
 * 32-bit word per work-group to `sink` (device memory, `grid` words): the
 * wrapping sum of every 32-bit word the work-group read, so the loads cannot be
 * optimised away and the result can be checked.  `bytes` counts the bytes read
 * (a whole number of chunks).  grid = 0 picks four work-groups of 256 threads
 * per compute unit.  The call only enqueues the kernel on `stream` (a
 * hipStream_t; NULL = default).
 *
 * Returns 0 on success, -1 for a NULL pointer, -3 for sizes that are not
 * positive multiples of 16 (or chunk > stride, or bytes not a multiple of
 * chunk, or grid < 0), -5 for a pointer that is not 16-byte aligned, -8 for no
 * device, -9 when the launch fails.
 */
#ifndef EXACT_ATTN_PROBE_H
#define EXACT_ATTN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t attn_probe_read(const void *buf, int64_t bytes, int64_t chunk, int64_t stride,
                        uint32_t *sink, int32_t grid, void *stream);

/* MFMA throughput probe: every compute unit runs one work-group of 8 waves (two
 * per SIMD, as the prefill kernel does) that issues `iters` x 16
 * v_mfma_f32_32x32x16_bf16 in four accumulator chains on registers only.  With
 * random_operands != 0 the A and B operands are random bf16 values (random
 * sign, exponent and mantissa bits, magnitudes in [1/8, 2)) that change
 * from one instruction to the next (the switching of real attention data; the
 * device's power limit then lowers its clock); with 0 they are constant.  Writes
 * one float per thread to `out` (8 * 64 * compute units floats) so nothing is
 * optimised away, and to `ticks` (two uint64) the cycle-counter and steady-counter
 * deltas of wave 0 over its loop (which it may finish early: of two waves on a
 * SIMD the older one tends to be served first).  Flops per call: iters * 16 * 32768 * 8 *
 * compute units.  Returns 0, -1 (NULL), -3 (iters < 1), -8 (no device) or -9. */
int32_t attn_probe_mfma(float *out, int32_t iters, int32_t random_operands, uint64_t *ticks,
                        void *stream);

/* Clock probe: one wave that reads the cycle counter (clock64(): shader
 * cycles) and the steady counter (wall_clock64(), at a constant rate that
 * hipDeviceAttributeWallClockRate reports) when it starts and again once the steady
 * counter has advanced by `wall_ticks` (at most 2^31 of them; the wave sleeps
 * between reads), and writes the four values to `out` (four uint64).  Launched on
 * a second stream beside a long kernel it samples the shader clock while that
 * kernel runs (one wave of few registers fits next to it on a compute unit).
 * Returns 0, -1 (NULL), -3 (wall_ticks outside [1, 2^31]) or -9. */
int32_t attn_probe_clock(uint64_t *out, int64_t wall_ticks, void *stream);

/* The current device's steady-counter rate and peak shader clock, in kHz
 * (hipDeviceAttributeWallClockRate and hipDeviceAttributeClockRate).  Returns 0,
 * -1 (NULL) or -8 (no device). */
int32_t attn_probe_rates(int64_t *wall_khz, int64_t *peak_sclk_khz);

/* Work-groups attn_probe_read launches for `grid` (the count `sink` must hold):
 * grid itself when > 0, else four per compute unit of the current device
 * (negative on error, as above). */
int32_t attn_probe_grid(int32_t grid);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_PROBE_H */
