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

/* Workgroups of the read kernel at most (it loops over larger ranges). */
#define WQBMM_PROBE_MAX_GRID 2048

/*
 * Reads `bytes` bytes at `src` once, with 16-byte nontemporal loads.  Each
 * lane folds its words by XOR and stores the result to `sink` (one uint32 of
 * device memory) only if it equals 0x9E3779B9, which keeps the loads alive;
 * with data whose words cancel (e.g. a byte pattern repeated over aligned
 * 64-byte runs, such as a constant fill) nothing is written.
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
