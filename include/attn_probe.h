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

/* Work-groups attn_probe_read launches for `grid` (the count `sink` must hold):
 * grid itself when > 0, else four per compute unit of the current device
 * (negative on error, as above). */
int32_t attn_probe_grid(int32_t grid);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_PROBE_H */
