/* qkv_measure.h -- measurement helper of libqkv.so (not part of the attention
 * path).
 *
 * The decode streams its packed K/V cache from HBM once per call, so its
 * speed is compared with what a plain streaming read achieves on the same
 * machine with the same byte count.  This entry point provides that read.
 */
#ifndef QKV_MEASURE_H
#define QKV_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "qkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest workgroup count of a call; the sink holds 4 words per workgroup. */
#define QKV_MEASURE_MAX_WORKGROUPS 8192

/* Reads the 'bytes' bytes at device pointer 'buf' once with 'workgroups'
 * workgroups of 256 threads: workgroup w reads the w-th of 'workgroups'
 * contiguous, equal ranges (the last one shorter) with 16-byte loads, four in
 * flight per thread.  Each wave writes the XOR of the words it read to one
 * word of 'sink' (device memory of at least 4 * workgroups uint32), so the
 * loads cannot be dropped.  Enqueued on 'stream' (a hipStream_t, NULL = the
 * default stream); nothing is allocated or synchronised.
 * Errors: EINVAL for null pointers, 'bytes' = 0 or not a multiple of 16,
 * 'buf' not 16-byte aligned, or 'workgroups' outside
 * [1, QKV_MEASURE_MAX_WORKGROUPS]; EHIP if the launch fails. */
qkv_status qkv_measure_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                            void* stream);

/* The same plain read with its shape chosen by the caller, to sweep the
 * read rate over load shapes: 'threads' per workgroup (64, 128, ..., 1024),
 * 'in_flight' loads per thread issued before any is used (1, 2, 4, 8 or 16),
 * each 'width' bytes wide (4, 8 or 16); workgroup w reads the w-th of
 * 'workgroups' contiguous, equal ranges.  'sink' must hold
 * workgroups * threads / 64 words.  Errors: EINVAL for null pointers, bytes
 * = 0 or not a multiple of 'width', 'buf' not 'width'-aligned, or any
 * parameter outside the sets above (workgroups in [1,
 * QKV_MEASURE_MAX_WORKGROUPS]); EHIP if the launch fails. */
qkv_status qkv_measure_read_config(const void* buf, size_t bytes, int32_t workgroups, int32_t threads,
                                   int32_t in_flight, int32_t width, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QKV_MEASURE_H */
