/*
 * hswd_measure.h -- C ABI of libhswd_measure.so, the measurement library
 * beside libhswd.so.  Nothing here is a step of the decode path; the
 * benchmark uses it to find the streaming-read ceiling of the GPU it runs
 * on, against which the attention kernels' bandwidth is compared.
 *
 * Status codes are those of hswd.h (HSWD_OK, HSWD_ERR_INVALID,
 * HSWD_ERR_ALIGN, HSWD_ERR_HIP).  Streams are hipStream_t passed as void*
 * (NULL: the default stream); calls are asynchronous on the stream.
 */
#ifndef HSWD_MEASURE_H
#define HSWD_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) of device memory at `buf` (DEVICE,
 * 16-byte aligned) once: `workgroups` workgroups of 256 threads, each
 * streaming one contiguous range with the 128-bit non-temporal loads the
 * attention kernels read their K/V tiles with, eight in flight per thread.
 * Its duration over a buffer much larger than the 256 MB last-level cache
 * gives the streaming-read ceiling.  `sink` (DEVICE, 16-byte aligned, at
 * least 4 * workgroups bytes) keeps the loads from being optimised away:
 * word w is written only if the loads of workgroup w fold to a fixed
 * 32-bit pattern, so in practice never.  The caller owns both buffers.
 * Errors: HSWD_ERR_INVALID (null pointer, bytes 0 or not a multiple of 16,
 * workgroups outside [1, 65536]), HSWD_ERR_ALIGN; nothing is launched
 * then.  HSWD_ERR_HIP if the launch fails. */
int32_t hswd_measure_stream_read(const void* buf, size_t bytes, void* sink,
                                 int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSWD_MEASURE_H */
