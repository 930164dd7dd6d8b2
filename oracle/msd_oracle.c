/*
 * msd_oracle.c -- plain, slow, obviously-correct CPU oracle of the A16W4
 * per-group MSD (multi-step decomposition) weight-quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, __graft_entry__.smoke() and
 * bench.py's cpu_baseline leg, never by the HIP product path.  It shares no
 * code with the HIP kernels.
 *
 * What it follows: the page "WeightQuantBatchMatmulExperiment 算子深度解析：
 * A16W4 PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计" (lpnh.cn/news/2294145,
 * "the WQBMM-Exp page"), §4.1 (MSD 伪量化算法, the eleven formulas),
 * §4.2 (operator spec) and §4.3 (int4 storage).  The page states the kernel
 * keeps the expansion factors as the fp32 literals 7.49f, 14.98f, 14.98f, so
 * every floating-point step here is IEEE binary32, one rounding per written
 * operation, in the order the formulas write them.  Build with
 * -O2 -ffp-contract=off and without -ffast-math so no operation is fused or
 * reordered.
 *
 * Readings taken where the page is silent or its formulas lost operators
 * in extraction (each is listed in the design notes):
 *   - round() is round-half-to-even (rintf in the default rounding mode);
 *   - step 2 multiplies by 7.49 first, then divides by A_max;
 *   - A_max is per (row, K-group);
 *   - a group whose A_max is 0 decomposes to all-zero levels;
 *   - step 10 is  [(Y1/7.49 + Y2/(7.49*14.98) + Y3/(7.49*14.98*14.98)) * A_max] * scale,
 *     the constant denominators formed left to right in fp32;
 *   - step 11 is  Y^i = Y_group + Y^(i-1), Y^0 = 0, in fp32, groups ascending;
 *     the fp16 output is the round-to-nearest-even of that fp32 sum;
 *   - int4 byte (k, j): low nibble = column 2j, high nibble = column 2j+1.
 *
 * Parity pins (tests/test_oracle_pins.py): invariants |A_l| <= 7, the
 * residual bound of the three-level expansion, group locality, sign symmetry,
 * exact-tie vectors, an exact-rational brute force on tiny shapes, an int64
 * library matmul for step 9, closed forms for steps 10-11 (one-hot X, zero W,
 * zero scale) and the fp64 direct-dequant GEMM within the MSD truncation bound.
 */
#include "msd_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- IEEE binary16 (1 sign, 5 exponent bits, bias 15, 10 fraction bits) ---- */

float msd_oracle_half_to_float(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float v;
    if (e == 0) {
        v = ldexpf((float)f, -24);                 /* zero / subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexpf((float)(1024 + f), e - 25);     /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

uint16_t msd_oracle_float_to_half(float x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return 0x7e00;
    /* Largest finite half is 65504; values at or above the midpoint 65520
     * to the next (nonexistent) step round to infinity. */
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: count of 2^-24 units, rounded half-to-even */
        double q = rint(a * ldexp(1.0, 24));       /* exact scaling, RNE */
        return sign | (uint16_t)q;                 /* q == 1024 gives the min normal */
    }
    int e;
    frexp(a, &e);                                  /* a = m * 2^e, m in [0.5,1) */
    e -= 1;                                        /* a in [2^e, 2^(e+1)) */
    double m = rint(a * ldexp(1.0, 10 - e));       /* in [1024, 2048], RNE */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e > 15) return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* ---- WQBMM-Exp page §4.1, steps 1-8 ---- */

static const float F1 = 7.49f;    /* multiFactors_[0] */
static const float F2 = 14.98f;   /* multiFactors_[1] == multiFactors_[2] */

/* Decompose one group of one row.  a: gs fp32 values (exact widenings of the
 * fp16 inputs).  Writes the three levels and returns A_max. */
static float decompose_group(const float* a, int64_t gs,
                             int8_t* l1, int8_t* l2, int8_t* l3) {
    /* step 1: A_max = rowMax(|A_group|) */
    float amax = 0.0f;
    for (int64_t k = 0; k < gs; ++k) {
        float v = fabsf(a[k]);
        if (v > amax) amax = v;
    }
    for (int64_t k = 0; k < gs; ++k) {
        if (amax == 0.0f) {            /* all-zero group: nothing to expand */
            l1[k] = l2[k] = l3[k] = 0;
            continue;
        }
        float prod = F1 * a[k];        /* step 2: tmp1 = 7.49 * A / A_max */
        float tmp1 = prod / amax;
        float A1 = rintf(tmp1);        /* step 3: round half to even */
        float d1 = tmp1 - A1;          /* step 4: tmp2 = (tmp1 - A1) * 14.98 */
        float tmp2 = d1 * F2;
        float A2 = rintf(tmp2);        /* step 5 */
        float d2 = tmp2 - A2;          /* step 6: tmp3 = (tmp2 - A2) * 14.98 */
        float tmp3 = d2 * F2;
        float A3 = rintf(tmp3);        /* step 7 */
        l1[k] = (int8_t)(int)A1;       /* step 8: A_int = [A1; A2; A3] */
        l2[k] = (int8_t)(int)A2;
        l3[k] = (int8_t)(int)A3;
    }
    return amax;
}

int msd_oracle_decompose(const uint16_t* x, int64_t M, int64_t K, int64_t gs,
                         int8_t* a_int, float* a_max) {
    if (M < 0 || K <= 0 || gs <= 0 || K % gs) return -1;
    const int64_t G = K / gs;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float* a = (float*)malloc(sizeof(float) * (size_t)gs);
        for (int64_t g = 0; g < G; ++g) {
            for (int64_t k = 0; k < gs; ++k)
                a[k] = msd_oracle_half_to_float(x[m * K + g * gs + k]);
            int64_t off = m * K + g * gs;
            a_max[m * G + g] = decompose_group(a, gs, a_int + 0 * M * K + off,
                                               a_int + 1 * M * K + off,
                                               a_int + 2 * M * K + off);
        }
        free(a);
    }
    return 0;
}

/* ---- WQBMM-Exp page §4.3: int4 storage, two per byte ---- */

static int8_t nibble_to_int(unsigned v) {       /* 4-bit two's complement */
    v &= 0xF;
    return (int8_t)(v >= 8 ? (int)v - 16 : (int)v);
}

int msd_oracle_unpack_w(const uint8_t* w_packed, int64_t K, int64_t N, int8_t* w) {
    if (K <= 0 || N <= 0 || N % 2) return -1;
    const int64_t NB = N / 2;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t j = 0; j < NB; ++j) {
            uint8_t b = w_packed[k * NB + j];
            w[k * N + 2 * j] = nibble_to_int(b);
            w[k * N + 2 * j + 1] = nibble_to_int(b >> 4);
        }
    }
    return 0;
}

/* ---- WQBMM-Exp page §4.1 step 9: Y_int = A_int . Weight_group ---- */

int msd_oracle_yint(const int8_t* a_int, const int8_t* w, int64_t M, int64_t K,
                    int64_t N, int64_t gs, int64_t g_begin, int64_t g_end,
                    int32_t* y_int) {
    if (M < 0 || K <= 0 || N <= 0 || gs <= 0 || K % gs) return -1;
    if (g_begin < 0 || g_end > K / gs || g_begin > g_end) return -1;
    const int64_t NG = g_end - g_begin;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t gi = 0; gi < NG; ++gi) {
        for (int64_t m = 0; m < M; ++m) {
            const int64_t g = g_begin + gi;
            for (int l = 0; l < 3; ++l) {
                int32_t* out = y_int + ((gi * 3 + l) * M + m) * N;
                const int8_t* arow = a_int + (int64_t)l * M * K + m * K;
                for (int64_t n = 0; n < N; ++n) out[n] = 0;
                for (int64_t k = g * gs; k < (g + 1) * gs; ++k) {
                    int32_t av = arow[k];
                    const int8_t* wrow = w + k * N;
                    for (int64_t n = 0; n < N; ++n) out[n] += av * (int32_t)wrow[n];
                }
            }
        }
    }
    return 0;
}

/* ---- WQBMM-Exp page §4.1 steps 1-11 for a subset of rows ---- */

int msd_oracle_matmul(const uint16_t* x, const uint8_t* w_packed,
                      const uint16_t* scale, int64_t gs, int64_t M, int64_t K,
                      int64_t N, const int64_t* rows, int64_t n_rows,
                      float* y32, uint16_t* y16) {
    if (M < 0 || K <= 0 || N <= 0 || gs <= 0 || K % gs || N % 2) return -1;
    if (rows == NULL) n_rows = M;
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    const int64_t G = K / gs;

    int8_t* w = (int8_t*)malloc((size_t)K * (size_t)N);
    if (!w) return -2;
    msd_oracle_unpack_w(w_packed, K, N, w);

    /* step 10 constants: 7.49, 7.49*14.98, 7.49*14.98*14.98, left to right */
    const float D1 = F1;
    const float D2 = F1 * F2;
    const float D3 = D2 * F2;

    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t m = rows ? rows[r] : r;
        float* a = (float*)malloc(sizeof(float) * (size_t)gs);
        int8_t* lev = (int8_t*)malloc((size_t)(3 * gs));
        int32_t* yl = (int32_t*)malloc(sizeof(int32_t) * (size_t)(3 * N));
        float* acc = (float*)malloc(sizeof(float) * (size_t)N);
        if (!a || !lev || !yl || !acc) {
#pragma omp atomic write
            err = -2;
        } else {
            for (int64_t n = 0; n < N; ++n) acc[n] = 0.0f;           /* Y^0 = 0 */
            for (int64_t g = 0; g < G; ++g) {
                for (int64_t k = 0; k < gs; ++k)
                    a[k] = msd_oracle_half_to_float(x[m * K + g * gs + k]);
                float amax = decompose_group(a, gs, lev, lev + gs, lev + 2 * gs);
                /* step 9: the three integer products for this group */
                for (int64_t i = 0; i < 3 * N; ++i) yl[i] = 0;
                for (int l = 0; l < 3; ++l) {
                    for (int64_t k = 0; k < gs; ++k) {
                        int32_t av = lev[l * gs + k];
                        const int8_t* wrow = w + (g * gs + k) * N;
                        for (int64_t n = 0; n < N; ++n) yl[l * N + n] += av * (int32_t)wrow[n];
                    }
                }
                /* step 10: Y_group; step 11: Y^i = Y_group + Y^(i-1) */
                for (int64_t n = 0; n < N; ++n) {
                    float s1 = (float)yl[n] / D1;
                    float s2 = (float)yl[N + n] / D2;
                    float s3 = (float)yl[2 * N + n] / D3;
                    float sum = (s1 + s2) + s3;
                    float yg = (sum * amax) * msd_oracle_half_to_float(scale[g * N + n]);
                    acc[n] = yg + acc[n];
                }
            }
            for (int64_t n = 0; n < N; ++n) {
                if (y32) y32[r * N + n] = acc[n];
                if (y16) y16[r * N + n] = msd_oracle_float_to_half(acc[n]);
            }
        }
        free(a); free(lev); free(yl); free(acc);
    }
    free(w);
    return err;
}

int msd_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void msd_oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
