/*
 * pagedattn_probe.h - a measurement probe exported by libpagedattn.so.  It is
 * not part of the attention path: the benchmark uses it to measure the read
 * rate this GPU's memory system delivers for a buffer of a given size, the
 * reference against which the decode kernels' achieved bandwidth is read.
 */
#ifndef PAGEDATTN_PROBE_H
#define PAGEDATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` of device memory at `buf` once, in 16-byte vectors, with
 * num_workgroups workgroups of 256 threads striding over the buffer, and
 * writes one 32-bit XOR of what each wave read to sink[4 * wg + wave]
 * (uint32 [4 * num_workgroups], device memory) so that the reads are kept.
 * Enqueued on `stream` (hipStream_t, NULL = default); nothing is allocated.
 * Returns 0 (PA_OK), -1 (PA_ERR_NULL) for a NULL pointer, -2 (PA_ERR_SHAPE)
 * when bytes is 0 or not a multiple of 16 or num_workgroups < 1, and -6
 * (PA_ERR_HIP) when the launch fails.
 */
int pa_read_probe(const void *buf, size_t bytes, uint32_t *sink, int num_workgroups,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif
