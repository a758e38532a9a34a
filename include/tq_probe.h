/* Measurement helper of libtq.so, not part of the compression method.
 *
 * tq_probe_stream_read: one launch of a plain grid-stride read of `bytes` bytes at `buf`
 * (256 workgroups x 512 threads, 16-byte loads), timed by the caller with HIP events on
 * `hip_stream`.  bytes / time is the streaming-read bandwidth of the device, the measured
 * ceiling that a memory-bound kernel's achieved bandwidth is set against, next to the
 * HBM specification.
 *   buf    device, 16-byte aligned, bytes a positive multiple of 16; only read
 *   sink   device unsigned[1], 4-byte aligned; written only for one improbable data
 *          value (it keeps the loads alive), so its contents are meaningless
 * Errors: TQ_ERR_INVALID_ARG (null or misaligned pointers, bad size), TQ_ERR_HIP. */
#ifndef TQ_PROBE_H
#define TQ_PROBE_H

#include <stddef.h>

#include "tq.h" /* status codes */

#ifdef __cplusplus
extern "C" {
#endif

int tq_probe_stream_read(const void *buf, size_t bytes, unsigned *sink, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif
