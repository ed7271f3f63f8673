/*
 * mxfp4_probe.h - measurement helper exported by libmxfp4.so.  Not part of
 * the dequantize-and-multiply path: it exists so that a benchmark can time,
 * in the same process and on the same cold buffers, the plain read rate a
 * single kernel launch of a given size reaches, and report the GEMM and
 * expert-bank kernels against that ceiling as well as against the HBM peak.
 */
#ifndef MXFP4_PROBE_H
#define MXFP4_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at device pointer `buf` once, 16 bytes per lane per
 * load, `loads_per_thread` (4, 8 or 16) loads per thread issued before any
 * is used, 256 threads per workgroup, one workgroup per
 * 256 * loads_per_thread * 16 bytes.  The data is only read: `sink`, a
 * device pointer to 4 bytes, receives a thread's XOR of its loads only when
 * that XOR equals a fixed word, a store that keeps the loads from being
 * removed.  buf 16-byte aligned, bytes a positive multiple of
 * 16, sink 4-byte aligned.  Stream-ordered on `stream` (a hipStream_t).
 * Returns 0, -1 for bad arguments (nothing launched), -4 if the launch
 * failed. */
int mxfp4_probe_read(const void *buf, int64_t bytes, int loads_per_thread, void *sink,
                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_PROBE_H */
