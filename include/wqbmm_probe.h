/*
 * wqbmm_probe.h -- measurement helpers exported by libwqbmm.so beside the
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

/* Floats `wqbmm_probe_mfma_valu` may write to `out`: one per thread of its
 * (up to) 512 workgroups of 512 threads. */
#define WQBMM_PROBE_MFMA_VALU_OUT 262144

/*
 * Whether MFMA and VALU work overlap on a SIMD (the prefill GEMMs issue
 * both: FP6 MFMAs for step 9, fp32 FMAs for the combine of step 10).  Runs
 * 256 workgroups of 8 waves (two per SIMD), `iters` rounds each, a round
 * being per wave, by `mode`:
 *   0  a block of 12 independent v_mfma_scale_f32_16x16x128_f8f6f4 (FP6)
 *   1  a block of 64 fp32 FMAs (16 independent chains)
 *   2  both blocks, one after the other
 *   3  waves 0-3 the MFMA block only, waves 4-7 the FMA block only (one wave
 *      of each kind per SIMD)
 *   4  as 2, with a workgroup barrier after every round
 *   5, 6, 7  as 2, 0 and 1 with waves 4-7 idle (one wave per SIMD)
 *   8, 9, 10 as 2, 0 and 1 with 512 workgroups (two per CU: four waves per
 *            SIMD)
 * No memory traffic inside the loop.  out: WQBMM_PROBE_MFMA_VALU_OUT floats
 * of device memory, written (values of no meaning).  Asynchronous on
 * `stream`.  Returns 0 on success, 1 if out is NULL, 2 if mode is not 0-10 or
 * iters not in [1, 2^20] (nothing launched), 4 if the launch failed.
 */
int wqbmm_probe_mfma_valu(int mode, int iters, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* WQBMM_PROBE_H */
