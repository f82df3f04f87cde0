/*
 * bitlinear_probe.h -- measurement probes built into libbitlinear.so.  They
 * compute nothing of the BitLinear path; they give the floors its kernels are
 * compared against on the running GPU (what reading a buffer of a given size
 * once costs, and what a launch of an empty kernel costs).
 */
#ifndef BITLINEAR_PROBE_H
#define BITLINEAR_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bl_probe_read -- one kernel that reads `bytes` bytes of device memory at
 * `buf` once (16-byte non-temporal loads; a 256-thread block covers
 * per_lane x 4 KiB contiguous bytes, every lane issuing all of its loads
 * before it waits, the decode GEMV's pattern).  Nothing is written except,
 * in principle, one word of `sink` (device, >= 4096 bytes) if the XOR of the
 * data equals a fixed constant.  bytes: a multiple of 16; per_lane: 1, 2, 4
 * or 8.  Returns 0, 1 for a bad argument, 5 for a launch error.
 */
int bl_probe_read(const void *buf, size_t bytes, int per_lane, uint32_t *sink, void *stream);

/* bl_probe_empty -- one launch of an empty kernel (1 block of 64 threads).
 * Returns 0 or 5 for a launch error. */
int bl_probe_empty(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_PROBE_H */
