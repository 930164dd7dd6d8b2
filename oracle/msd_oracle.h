/*
 * msd_oracle.h -- plain CPU oracle of the A16W4 per-group MSD matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The HIP product path
 * never links, loads or calls it, and the two share no source.
 *
 * Source of the method: the page "WeightQuantBatchMatmulExperiment 算子深度解析：
 * A16W4 PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计" (lpnh.cn/news/2294145),
 * called "the WQBMM-Exp page" below.
 *
 * All arrays are host memory owned by the caller, row-major.
 * fp16 values are passed as their IEEE binary16 bit patterns (uint16_t).
 */
#ifndef MSD_ORACLE_H
#define MSD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 <-> binary32, from the format definition (exact / RNE). */
float    msd_oracle_half_to_float(uint16_t h);
uint16_t msd_oracle_float_to_half(float f);

/* WQBMM-Exp page §4.1 steps 1-8: per (row, K-group) A_max and the
 * three-level decomposition.  x: fp16 bits [M][K].  a_int: int8 [3][M][K]
 * (level-major: A1 rows, then A2 rows, then A3 rows).  a_max: fp32 [M][K/gs].
 * Returns 0, or -1 if gs does not divide K or sizes are not positive. */
int msd_oracle_decompose(const uint16_t* x, int64_t M, int64_t K, int64_t gs,
                         int8_t* a_int, float* a_max);

/* WQBMM-Exp page §4.3: two int4 per byte.  Byte (k, j) holds column 2j in
 * the low nibble and column 2j+1 in the high nibble, two's complement.
 * w_packed: uint8 [K][N/2] -> w: int8 [K][N]. */
int msd_oracle_unpack_w(const uint8_t* w_packed, int64_t K, int64_t N, int8_t* w);

/* WQBMM-Exp page §4.1 step 9, restricted to groups [g_begin, g_end):
 * y_int[g - g_begin][l][m][n] = sum over k in group g of A_l[m][k] * w[k][n].
 * a_int: int8 [3][M][K]; w: int8 [K][N]; y_int: int32 [g_end-g_begin][3][M][N]. */
int msd_oracle_yint(const int8_t* a_int, const int8_t* w, int64_t M, int64_t K,
                    int64_t N, int64_t gs, int64_t g_begin, int64_t g_end,
                    int32_t* y_int);

/* The whole operator (WQBMM-Exp page §4.1 steps 1-11) for a subset of rows.
 * rows: n_rows row indices into x (NULL = all M rows in order, n_rows = M).
 * y32: fp32 [n_rows][N] (the step-11 accumulator), y16: fp16 bits
 * [n_rows][N] (round-to-nearest-even of y32).  Either output may be NULL. */
int msd_oracle_matmul(const uint16_t* x, const uint8_t* w_packed,
                      const uint16_t* scale, int64_t gs, int64_t M, int64_t K,
                      int64_t N, const int64_t* rows, int64_t n_rows,
                      float* y32, uint16_t* y16);

/* Number of OpenMP threads the oracle's parallel loops use (1 if built
 * without OpenMP). */
int msd_oracle_num_threads(void);

/* Sets the number of OpenMP threads for later calls (n > 0; ignored without
 * OpenMP).  Used to time the oracle at one thread and at all cores. */
void msd_oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
