/*
 * wqbmm_probe.h -- measurement helper exported by libwqbmm.so beside the
 * operator (include/wqbmm.h).  Not part of the operator.
 *
 * The weight-streaming (decode) kernels of the operator are bound by HBM
 * bandwidth.  Besides the published peak, they are compared with what a
 * plain read of the same number of bytes achieves on the same device; this
 * entry point is that plain read.
 */
#ifndef WQBMM_PROBE_H
#define WQBMM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of the read kernel at most, and so the uint32 words of `sink`. */
#define WQBMM_PROBE_SINK_WORDS 2048

/*
 * Reads `bytes` bytes at `src` once, with 16-byte nontemporal loads, and
 * stores one XOR of the words read per workgroup into `sink` (uint32
 * [WQBMM_PROBE_SINK_WORDS], device memory; only the first words are written).
 * src: device memory, 16-byte aligned; bytes > 0 and a multiple of 16.
 * Asynchronous on `stream` (a hipStream_t; NULL = the legacy default stream).
 * Returns 0 on success, 1 if a pointer is NULL, 2 if `bytes` or the alignment
 * breaks the rules (nothing launched), 4 if the launch failed.
 */
int wqbmm_probe_stream_read(const void* src, int64_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* WQBMM_PROBE_H */
