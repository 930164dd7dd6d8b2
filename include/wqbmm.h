/*
 * wqbmm.h -- C ABI of the MI355X (gfx950) A16W4 per-group MSD matmul.
 *
 *     y = MSD(x, dequant(w))        x: fp16 [M][K], w: int4 [K][N], y: fp16 [M][N]
 *
 * The operation is the one specified on the page "WeightQuantBatchMatmulExperiment
 * 算子深度解析：A16W4 PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计"
 * (lpnh.cn/news/2294145, "the WQBMM-Exp page"):
 *   - §4.2 (算子规格): x1 M x K fp16 ND, x2 K x N int4 ND, antiquant_scale
 *     GroupNum x N fp16 ND, y M x N fp16 ND; only these dtypes are accepted.
 *   - §4.1 (MSD 伪量化算法): per (row, K-group) A_max = max|x|; three rounds of
 *     round(7.49*x/A_max), round(residual*14.98), round(residual*14.98) give
 *     int4-range matrices A1, A2, A3; each is contracted with the group's int4
 *     weights in integer arithmetic; the three results are combined as
 *     (Y1/7.49 + Y2/(7.49*14.98) + Y3/(7.49*14.98^2)) * A_max * scale and
 *     accumulated over groups.
 *   - §4.3: int4 weights are stored two per byte.
 *
 * Weights are static, so they are converted ONCE, on the device, from the
 * page's ND layout into the tiled layout every kernel reads
 * (wqbmm_a16w4_tiled_weight_bytes + wqbmm_a16w4_tile_weights), the way the
 * call example (section 调用示例) of the page "CANN ops-math：
 * aclnnCalculateMatmulWeightSizeV2 接口详解" (zskr.cn/news/2299903) queries the
 * converted size, converts the ND weight once and then passes the converted
 * weight to the quantized matmul.  The matmul entry points take w_tiled.
 *
 * Conventions for every entry point:
 *   - Array pointers are DEVICE pointers (HIP device memory of the current
 *     device) owned by the caller; the library never retains or frees them.
 *     Row-major ("ND") layouts, no padding between rows.
 *   - fp16 arrays hold IEEE binary16 values.
 *   - w_nd (the ND weight) is uint8 [K][N/2]: byte (k, j) holds column 2j in
 *     bits 0-3 and column 2j+1 in bits 4-7, each a 4-bit two's-complement value
 *     in [-8, 7].
 *   - w_tiled is the output of wqbmm_a16w4_tile_weights for the same K and N,
 *     wqbmm_a16w4_tiled_weight_bytes(K, N) bytes.  Its layout is internal to the
 *     library (int4, 16-column x 128-row tiles of 1 KB shaped after the MFMA
 *     operands; rows are padded to a multiple of 128 with zeros) and is only
 *     produced and consumed by it.
 *   - stream is a hipStream_t (NULL = the legacy default stream).  All work is
 *     enqueued asynchronously on it; nothing synchronizes the host.  Faults in
 *     device code surface at the caller's next synchronization, as with any
 *     stream API.
 *   - Arguments are validated on the host before any device work, in the
 *     order: null pointers -> shapes -> support.  On error nothing is launched
 *     and outputs are untouched.
 *   - Shape rules: M >= 0 (M == 0 is a no-op returning WQBMM_OK; the arrays
 *     with an M extent -- x, y, a_int, a_max, y_int -- may then be NULL), K >= 1,
 *     N >= 1, K % group_size == 0, N % 32 == 0, M <= 2^24, K <= 2^20,
 *     N <= 2^20, every pointer 16-byte aligned.
 *   - group_size must be 64 or 128 (other positive values: WQBMM_ERR_UNSUPPORTED).
 *   - Workspace.  The two-kernel paths (decode at 4 < M <= 96, prefill) pass
 *     operands between their kernels through device memory, and the fused
 *     decode kernel (M <= 4) with K > 4096 sums its K-splits in accumulators.
 *     The library keeps that memory per (device, stream): allocated on first
 *     need and grown on demand with hipMalloc.  Growth never synchronizes and
 *     never frees: a replaced buffer stays allocated until the process ends
 *     (a graph captured earlier may still use it), and sizes at least double,
 *     so the retired buffers of a stream take less than its current one.
 *     Growth is refused while the stream is being captured into a graph:
 *     the call returns WQBMM_ERR_CAPTURE and launches nothing.  Make one
 *     eager call of the largest shape on a stream before capturing on it.
 *     Calls on different streams never share workspace.  Calls captured on a
 *     stream use that stream's workspace when their graph is replayed, so a
 *     replay must not run concurrently with other calls that use the same
 *     stream's workspace (replay on that stream, or synchronize in between).
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Only gfx950 (MI355X) is supported: other devices give WQBMM_ERR_UNSUPPORTED.
 *   - Finite inputs are assumed; Inf/NaN inputs give unspecified outputs.
 */
#ifndef WQBMM_H
#define WQBMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wqbmm_status {
  WQBMM_OK = 0,
  WQBMM_ERR_NULLPTR = 1,     /* a required pointer is NULL                       */
  WQBMM_ERR_INVALID = 2,     /* a shape / alignment rule above is violated       */
  WQBMM_ERR_UNSUPPORTED = 3, /* group_size not 64/128, or the device is not gfx950 */
  WQBMM_ERR_LAUNCH = 4,      /* a HIP call or kernel launch failed               */
  WQBMM_ERR_ALLOC = 5,       /* workspace allocation failed                      */
  WQBMM_ERR_CAPTURE = 6,     /* the workspace would have to grow during graph capture */
  WQBMM_ERR_TOO_LARGE = 7    /* the shape exceeds wqbmm_a16w4_msd_noalloc's fixed scratch */
} wqbmm_status;

/* Kernel path selector for the *_path / *_yint entry points. */
typedef enum wqbmm_path {
  WQBMM_PATH_AUTO = 0,     /* what wqbmm_a16w4_msd picks (wqbmm_select_path)      */
  WQBMM_PATH_DECODE = 1,   /* weight-streaming kernels; valid for M <= 96        */
  WQBMM_PATH_PREFILL = 2   /* operand preparation + MFMA GEMM; any M            */
} wqbmm_path;

/*
 * Size in bytes of the tiled weights for K x N (K*N/2 when K % 128 == 0), or
 * -1 if K or N breaks the shape rules (K in [1, 2^20], N in [32, 2^20],
 * N % 32 == 0).  Pure host function.
 */
int64_t wqbmm_a16w4_tiled_weight_bytes(int64_t K, int64_t N);

/*
 * One-time conversion of the ND int4 weights into the tiled layout.
 *   w_nd     uint8 [K][N/2]   (format above)
 *   w_tiled  wqbmm_a16w4_tiled_weight_bytes(K, N) bytes, caller-allocated,
 *            written completely (padding rows included)
 * Shape rules as for wqbmm_a16w4_tiled_weight_bytes; both pointers 16-byte
 * aligned; w_nd and w_tiled must not overlap.
 */
wqbmm_status wqbmm_a16w4_tile_weights(const void* w_nd, int64_t K, int64_t N, void* w_tiled,
                                      void* stream);

/*
 * The operator (WQBMM-Exp page §4.1 steps 1-11, §4.2).
 *   x               fp16  [M][K]
 *   w_tiled         int4 weights K x N, tiled (wqbmm_a16w4_tile_weights)
 *   antiquant_scale fp16  [K/group_size][N]   (per group of K, per column)
 *   y               fp16  [M][N]              (write-only, fully overwritten)
 * y[m][n] is the round-to-nearest-even fp16 of the fp32 sum over groups.
 */
wqbmm_status wqbmm_a16w4_msd(const void* x, const void* w_tiled,
                             const void* antiquant_scale, int64_t group_size,
                             int64_t M, int64_t K, int64_t N, void* y,
                             void* stream);

/* Same operation with an explicit kernel path (WQBMM_PATH_*).  The decode
 * path with M > 96 returns WQBMM_ERR_INVALID. */
wqbmm_status wqbmm_a16w4_msd_path(const void* x, const void* w_tiled,
                                  const void* antiquant_scale, int64_t group_size,
                                  int64_t M, int64_t K, int64_t N, void* y,
                                  int path, void* stream);

/*
 * The weights' operand form: the FP6 (e2m3) MFMA operand tiles that the
 * group-size-128 prefill GEMM contracts (each int4 weight halved, 6 bits;
 * columns padded with zeros to a multiple of 256), converted ONCE from the
 * tiled weights, like the tiled weights from the ND ones (the convert-once
 * pattern of the aclnnCalculateMatmulWeightSizeV2 page's call example,
 * section 调用示例).  Without it the prefill path's operand kernel converts
 * the tiled weights again on every call (WQBMM-Exp page §6.1, UnfoldA); with
 * it that kernel only decomposes x.  It costs 0.75 byte per weight (plus
 * padding) beside the tiled weights' 0.5 and is optional: only the prefill
 * path at group size 128 reads it.
 * wqbmm_a16w4_operand_weight_bytes: its size in bytes,
 *   (ceil(N/256)*256 / 32) * ceil(K/128) * 3072, or -1 if K or N breaks the
 *   rules of wqbmm_a16w4_tiled_weight_bytes.  Pure host function.
 * wqbmm_a16w4_operand_weights:
 *   w_tiled    tiled weights for K x N (wqbmm_a16w4_tile_weights)
 *   w_operand  wqbmm_a16w4_operand_weight_bytes(K, N) bytes, caller-allocated,
 *              written completely
 * Both pointers 16-byte aligned, not overlapping.
 */
int64_t wqbmm_a16w4_operand_weight_bytes(int64_t K, int64_t N);
wqbmm_status wqbmm_a16w4_operand_weights(const void* w_tiled, int64_t K, int64_t N,
                                         void* w_operand, void* stream);

/*
 * wqbmm_a16w4_msd_path with the weights' operand form as well.  w_operand is
 * NULL (then this is wqbmm_a16w4_msd_path) or the output of
 * wqbmm_a16w4_operand_weights for the same weights, K and N, 16-byte aligned
 * (else WQBMM_ERR_INVALID); it is read only by the prefill path at group size
 * 128, and the result is bit-identical to the call without it.  w_tiled is
 * still required (the decode path and group size 64 read it).
 */
wqbmm_status wqbmm_a16w4_msd_ex(const void* x, const void* w_tiled, const void* w_operand,
                                const void* antiquant_scale, int64_t group_size,
                                int64_t M, int64_t K, int64_t N, void* y,
                                int path, void* stream);

/*
 * wqbmm_a16w4_msd without any device allocation, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same operation, arguments, rules and
 * kernels as wqbmm_a16w4_msd, and bit-identical results.  It calls no
 * hipMalloc, hipFree or other allocating routine: the memory its kernels
 * pass between them is one fixed 64 MiB array per device, a static device
 * variable of the library that the device holds from loading until the
 * process ends (2 MiB of split-K accumulators for M <= 4 with K > 4096, which
 * allows M * N up to 262144 there; 62 MiB of operands for the two-kernel
 * paths, enough for M = 4096 at K = N = 4096 with group size 128).  A shape
 * that needs more returns WQBMM_ERR_TOO_LARGE before any launch.
 *   - The first call on a device sets the array up (its device address, and a
 *     kernel on `stream` that zeroes the accumulators); that first call must
 *     not be made while `stream` is being captured (WQBMM_ERR_CAPTURE).
 *   - Every call on a device shares that device's array and leaves the last
 *     call's operands in it: calls that overlap in time on one device race
 *     and give wrong results.  Order them (one stream, or synchronize in
 *     between); a graph holding such calls must not replay concurrently with
 *     other calls of this entry point on the same device.
 */
wqbmm_status wqbmm_a16w4_msd_noalloc(const void* x, const void* w_tiled,
                                     const void* antiquant_scale, int64_t group_size,
                                     int64_t M, int64_t K, int64_t N, void* y,
                                     void* stream);

/*
 * Steps 1-8 alone (WQBMM-Exp page §4.1: A_max, tmp1..tmp3, A1..A3, A_int),
 * computed by the same device routine every path uses.
 *   x      fp16 [M][K]
 *   a_int  int8 [3][M][K]   level-major: A1 rows, then A2 rows, then A3 rows
 *   a_max  fp32 [M][K/group_size]
 * Each level value lies in [-7, 7].  A group whose A_max is 0 gives zeros.
 */
wqbmm_status wqbmm_a16w4_msd_prepass(const void* x, int64_t group_size,
                                     int64_t M, int64_t K, int8_t* a_int,
                                     float* a_max, void* stream);

/*
 * Steps 1-9 for the groups [g_begin, g_end) (WQBMM-Exp page §4.1 step 9:
 * Y_int = A_int . Weight_group), through the same kernels as the chosen path,
 * stopping before the fp32 combine.
 *   y_int  int32 [g_end-g_begin][3][M][N]
 *          y_int[g-g_begin][l][m][n] = sum over k in group g of A_l[m][k]*w[k][n]
 * Requires 0 <= g_begin < g_end <= K/group_size (else WQBMM_ERR_INVALID).
 */
wqbmm_status wqbmm_a16w4_msd_yint(const void* x, const void* w_tiled,
                                  int64_t group_size, int64_t M, int64_t K,
                                  int64_t N, int64_t g_begin, int64_t g_end,
                                  int32_t* y_int, int path, void* stream);

/*
 * Profiling support: run ONE stage of a kernel path (WQBMM_PATH_* as in
 * wqbmm_a16w4_msd_path), so that its kernels can be timed separately.
 *   stage 1: the operand kernel only (WQBMM-Exp page §6.1 UnfoldA: x -> the
 *            three levels of §4.1 steps 1-8 and the rows' step-10 level
 *            weights; on the prefill path without w_operand also w -> MFMA
 *            operand tiles), into this stream's workspace; y is not
 *            written.  The decode path at
 *            M <= 4 is one fused kernel: nothing is launched.
 *   stage 2: the contraction kernel only (§4.1 steps 9-11) on the operands
 *            that the most recent call of the same path on the SAME stream
 *            prepared; y is written.  Returns WQBMM_ERR_INVALID if that call
 *            had another path, shape or group size, or used w_operand where
 *            this one does not or the other way round (or none happened).
 *            x is not re-read in this stage.  The decode path at M <= 4 runs
 *            its fused kernel (all of steps 1-11).
 * Arguments and rules as for wqbmm_a16w4_msd_ex; other stage values give
 * WQBMM_ERR_INVALID.
 */
wqbmm_status wqbmm_a16w4_msd_profile_stage(const void* x, const void* w_tiled,
                                           const void* w_operand,
                                           const void* antiquant_scale, int64_t group_size,
                                           int64_t M, int64_t K, int64_t N, void* y,
                                           int path, int stage, void* stream);

/* The path wqbmm_a16w4_msd takes for this shape (WQBMM_PATH_DECODE or
 * WQBMM_PATH_PREFILL): decode for M <= 48; at group size 128 also for
 * M <= 96 when K*N <= 2^24 and for M <= 64 when K*N <= 3*2^24; prefill
 * otherwise (set from measured sweeps of both paths over M and shape).
 * Pure host function. */
int wqbmm_select_path(int64_t M, int64_t K, int64_t N, int64_t group_size);

/* Static, human-readable name of a status code (never NULL). */
const char* wqbmm_status_string(int status);

/* Library ABI version: major*10000 + minor*100 + patch. */
int wqbmm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* WQBMM_H */
