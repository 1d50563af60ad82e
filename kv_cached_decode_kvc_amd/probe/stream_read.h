/* stream_read.h -- streaming-read probe of HBM bandwidth (libkvc_probe.so).
 *
 * Not part of the decode path or of libkvc.so's interface.  It measures the
 * read rate a plain kernel reaches on this device, the ceiling beside which
 * the attention kernels' bandwidth is reported.
 */
#ifndef KVC_PROBE_STREAM_READ_H
#define KVC_PROBE_STREAM_READ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16) of device memory at `src` (16-byte
 * aligned) once, with `workgroups` workgroups of 256 threads, each streaming
 * one contiguous share 16 KiB at a time with four 16-byte loads in flight
 * per thread; ordinary loads, or non-temporal ones when `nontemporal` != 0.  `sink` (device, 4 bytes) is
 * written only in the improbable case that the combined data equals a fixed
 * constant.  Asynchronous on `stream` (a hipStream_t, NULL = default).
 * Returns 0, -1 for a bad argument, -7 for a failed launch. */
int kvc_probe_stream_read(const void* src, size_t bytes, int nontemporal, int workgroups,
                          uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_PROBE_STREAM_READ_H */
