// msd_decode.hip -- fused MSD kernel for the smallest M (decode, M <= 4).
//
// WQBMM-Exp page (the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4
// PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145):
// all of §4.1 (steps 1-11) in one launch.  The page's BASIC_MSD template runs
// pre-process (UnfoldA), Cube matmul and post-process (MergeY) as serial
// stages with full-core syncs (§6.1), and its PRELOAD_MSD template overlaps
// them across loop rounds with double/triple buffers (§6.2).  At small M the
// cost is streaming the int4 weights, so here every wave issues all of its
// weight loads first and the workgroup decomposes its slice of x while they
// are in flight; the three stages then run back to back in registers and LDS.
//
// Work split (the intra-device form of the page's N split across cores, §8.1
// nGmOffset = baseN * blockIdx, plus a split of K):
//   wave      = one 16-column tile x KBW 128-row blocks of the tiled weights
//               (KBW contiguous 1 KB runs, one 16-byte load per lane each);
//   workgroup = WC column tiles x WK waves along K, all sharing one decomposed
//               slice of x (R = WK*KBW*128 rows) in LDS;
//   grid      = (column blocks) x (K-splits).
// The decomposition is recomputed by every column block, M*R elements per
// workgroup; at M <= 4 that is cheap, so a workgroup is 1 column tile x 16
// waves x 2 blocks: R = 4096, and K <= 4096 needs no split and no hand-off.
// (For 4 < M <= 16 the repeated decomposition would cost more than the
// weight stream; that range decomposes x once in a kernel of its own, see
// msd_decode_gemv.hip.)
// The tiled layout makes each 16-byte chunk exactly a lane's B operand of
// v_mfma_i32_16x16x64_i8 for two 64-row steps (16*w per byte after masking the
// nibbles), so the weights need no transposition.
// Rows of the MFMA A operand ("slots"): slot 4*m + level, one 16-row tile;
// the levels of a row land in elements 0..2 of one lane's accumulator.
//
// Split-K: the WK waves of a column tile are summed in LDS; when K is split
// over several workgroups (K > 4096), each adds its partial, as a 2^-24 fixed-point
// integer, into a per-output int64 accumulator whose low 6 bits count the
// adds (one device-scope atomic with return per output).  The add that
// completes the count finishes that output: fp16 y, accumulator back to 0.
// One memory round trip after the contraction, no workgroup waits for
// another, no device-scope fence (on gfx950 such a fence writes back and
// invalidates the whole L2 of the XCD), and integer addition makes the
// result independent of arrival order.  An earlier hand-off (fp32 partials
// published with atomic stores, a per-block counter, a gather by the last
// workgroup) took three dependent round trips.
#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {
namespace dc {
constexpr int PAD = 16;                       // LDS row padding (bank spread)
}  // namespace dc

// Split-K partial of one output -> fixed point with 2^-24 resolution (the
// spacing of the smallest fp16 subnormals), saturated at +-2^27 so that 63
// of them cannot overflow the accumulator's 58-bit sum field.
constexpr float kPartialMax = 134217728.0f;   // 2^27

__device__ __forceinline__ int64_t fixed_partial(float v) {
  const float c = fminf(fmaxf(v, -kPartialMax), kPartialMax);
  return (int64_t)__builtin_rint((double)c * 16777216.0);
}

template <int GS, int WC, int WK, int KBW, bool YINT>
__global__ __launch_bounds__(64 * WC * WK) void msd_decode_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wt,
    const uint16_t* __restrict__ scale, int M, int K, int N, int g_begin, int g_end,
    int kb_begin, int splits, int nch, uint16_t* __restrict__ y, int32_t* __restrict__ y_int,
    uint64_t* __restrict__ accum) {
  constexpr int THREADS = 64 * WC * WK;
  constexpr int COLS = WC * kTileCols;          // columns per workgroup
  constexpr int PAD = dc::PAD;
  constexpr int R = WK * KBW * kTileRows;       // K rows per chunk
  constexpr int ROWA = R + PAD;                 // LDS bytes per A slot row
  constexpr int RT = 1;                         // 16-row A tiles
  constexpr int MT = 4;                         // rows of x covered by the slots
  constexpr int GPB = R / GS;                   // groups per chunk
  constexpr int GPW = KBW * kTileRows / GS;     // groups per wave and chunk
  constexpr int MROWS = 1;                      // output rows per lane

  __shared__ __attribute__((aligned(16))) int8_t sA[16 * RT * ROWA];
  __shared__ float sAmax[MT][GPB];
  __shared__ float sRed[WK > 1 ? WK - 1 : 1][WC][MROWS][64];   // lane fastest: conflict-free

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wc = wave % WC;                      // column tile within the workgroup
  const int wk = wave / WC;                      // K slice of this wave
  const int cb = blockIdx.x;
  const int s = blockIdx.y;
  const int NT = N / kTileCols;
  const int KB = (K + kTileRows - 1) / kTileRows;
  const int G = K / GS;
  const int nt = cb * WC + wc;
  const bool nt_ok = nt < NT;                    // N % 32 == 0: whole tiles only
  const int n = nt * kTileCols + (lane & 15);    // this lane's column
  const int mrows = M < MT ? M : MT;             // rows of x that exist

  float yacc[MROWS];
#pragma unroll
  for (int i = 0; i < MROWS; ++i) yacc[i] = 0.0f;

  // A split covers nch consecutive chunks of R rows (nch > 1 only for very
  // large K); groups are summed in ascending order across chunks.
  for (int c = 0; c < nch; ++c) {
    const int kb0 = kb_begin + (s * nch + c) * (WK * KBW);   // first 128-row block of the chunk
    const int kbase = kb0 * kTileRows;                      // first row of the chunk
    const int kreal = K - kbase < R ? (K - kbase > 0 ? K - kbase : 0) : R;   // rows < K
    const int kch = kreal / 8;                              // 8-element chunks per row
    const int items = mrows * kch;
    if (c > 0) __syncthreads();                             // the previous chunk's LDS is free

    // ---- 1. this thread's x chunks first (so waiting for them does not wait
    //         for the weights), the per-group scales, then every W load of the
    //         wave.  Loads are unconditional: an out-of-range one reads a valid
    //         address.  Its weights and scale are used as loaded, since they
    //         only reach groups >= G, which step 3 skips; zeroing them would
    //         be a select on the load result, and the compiler would wait for
    //         the load right there, i.e. before the barrier below.  (A load
    //         under a branch makes it wait for every outstanding load at the
    //         join.)  Out-of-range x chunks are zeroed: they are decomposed.
    // Only the M real rows and the rows below K are decomposed.  The other LDS
    // rows and A_max entries are left as they are: they only meet zero
    // weights (rows >= K of the tiled format are zero), feed groups >= G, or
    // feed accumulator rows that are never stored; integer MFMAs cannot trap.
    constexpr int ROUNDS = (MT * (R / 8) + THREADS - 1) / THREADS;
    // row of item `it` (it / kch for it < items <= MT * kch), by comparisons:
    // a division by the runtime kch costs about 25 VALU per lane, and it sits
    // in front of every load of the wave
    auto row_of = [&](int it) __attribute__((always_inline)) {
      int r = 0;
#pragma unroll
      for (int i = 1; i < MT; ++i) r += it >= i * kch ? 1 : 0;
      return r;
    };
    uint4 xv[ROUNDS];
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      const int it = rd * THREADS + tid;
      const bool ok = it < items;
      const int m = ok ? row_of(it) : 0;
      const int k = ok ? kbase + (it - m * kch) * 8 : 0;
      const uint4 v = *reinterpret_cast<const uint4*>(x + (ok ? (int64_t)m * K + k : 0));
      xv[rd] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
    const int gw0 = (kbase + wk * KBW * kTileRows) / GS;   // first group of this wave
    uint32_t sraw[GPW];
#pragma unroll
    for (int gl = 0; gl < GPW; ++gl) {
      if constexpr (YINT) {
        sraw[gl] = 0u;
      } else {
        const int g = gw0 + gl;
        const bool ok = nt_ok && g < G;
        sraw[gl] = scale[ok ? (int64_t)g * N + n : 0];
      }
    }
    v4i wv[KBW];
    {
      const uint8_t* wb = wt + (int64_t)(nt_ok ? nt : 0) * KB * 1024 + lane * 16;
#pragma unroll
      for (int j = 0; j < KBW; ++j) {
        const int kb = kb0 + wk * KBW + j;
        const bool ok = nt_ok && kb < KB;
        wv[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wb + (int64_t)(ok ? kb : 0) * 1024));
      }
    }

    // ---- 2. steps 1-8 for x[0:M][kbase : kbase+kreal] into LDS (A operand
    // layout).  Every lane of a wave runs the same rounds (the group maximum is
    // a cross-lane reduction over aligned lanes; kch is a multiple of GS/8);
    // items past the end decompose zeros and are dropped.
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      if (rd * THREADS >= items) break;              // workgroup-uniform
      // wave-uniform: a wave with no item in this round skips it (at M = 1 half
      // of the waves), leaving its SIMD to the waves that have items
      if (rd * THREADS + wave * 64 >= items) continue;
      const int it = rd * THREADS + tid;
      const int m = it < items ? row_of(it) : 0;
      const int ch = it - m * kch;
      uint32_t lv[3][2];
      float amax;
      msd_decompose8<GS>(xv[rd], lv, amax);
      if (it < items) {
#pragma unroll
        for (int l = 0; l < 3; ++l) {
          const int slot = 4 * m + l;
          *reinterpret_cast<uint2*>(sA + slot * ROWA + ch * 8) = make_uint2(lv[l][0], lv[l][1]);
        }
        if ((ch & (GS / 8 - 1)) == 0) sAmax[m][(ch * 8) / GS] = amax;
      }
    }
    __syncthreads();

    // ---- 3. per 64-row step: step 9 on MFMA; per completed group, steps 10-11
    //         (or the Y_int export)
    v4i acc[RT];
#pragma unroll
    for (int j = 0; j < KBW; ++j) {
      const uint32_t d[4] = {(uint32_t)wv[j][0], (uint32_t)wv[j][1], (uint32_t)wv[j][2], (uint32_t)wv[j][3]};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int krel = (wk * KBW + j) * kTileRows + 64 * st;   // row offset in the chunk
        if (krel % GS == 0) {
#pragma unroll
          for (int t = 0; t < RT; ++t) acc[t] = v4i{0, 0, 0, 0};
        }
        const v4i b = v4i{(int)lo16(d[2 * st]), (int)hi16(d[2 * st]), (int)lo16(d[2 * st + 1]),
                          (int)hi16(d[2 * st + 1])};
        const int kofs = krel + 16 * (lane >> 4);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const v4i af = *reinterpret_cast<const v4i*>(sA + (t * 16 + (lane & 15)) * ROWA + kofs);
          acc[t] = mfma_i8(af, b, acc[t]);
        }
        if ((krel + 64) % GS != 0) continue;                 // group not complete yet
        const int gloc = krel / GS;                           // group within the chunk
        const int gl = gloc - wk * GPW;                       // group within the wave
        const int g = kbase / GS + gloc;                      // absolute group
        if (g < g_begin || g >= g_end) continue;              // wave-uniform

        if constexpr (YINT) {
          const int64_t gi = g - g_begin;
#pragma unroll
          for (int i = 0; i < MROWS; ++i) {
            const int m = (lane >> 4) + i;
            if (m >= M || !nt_ok) continue;
#pragma unroll
            for (int l = 0; l < 3; ++l)
              y_int[((gi * 3 + l) * M + m) * (int64_t)N + n] = acc[0][l] >> 4;
          }
        } else {
          const float sc = half_bits_to_float(sraw[gl]);
#pragma unroll
          for (int i = 0; i < MROWS; ++i) {
            const int m = (lane >> 4) + i;
            const float am = sAmax[m][gloc];
            const float q1 = am * kC1, q2 = am * kC2, q3 = am * kC3;
            const int y1 = acc[0][0];
            const int y2 = acc[0][1];
            const int y3 = acc[0][2];
            float tt = (float)y1 * q1;
            tt = __builtin_fmaf((float)y2, q2, tt);
            tt = __builtin_fmaf((float)y3, q3, tt);
            yacc[i] = __builtin_fmaf(tt, sc, yacc[i]);
          }
        }
      }
    }
  }
  if constexpr (YINT) return;

  // ---- 4. sum the WK waves of each column tile (fixed order 0, 1, ...)
  if constexpr (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int i = 0; i < MROWS; ++i) sRed[wk - 1][wc][i][lane] = yacc[i];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int v = 0; v < WK - 1; ++v)
#pragma unroll
        for (int i = 0; i < MROWS; ++i) yacc[i] += sRed[v][wc][i][lane];
    }
  }
  if (wk != 0 || !nt_ok) return;

  // ---- 5. one split: store y.  Several: add the fixed-point partial into
  // the element's accumulator, whose low 6 bits count the adds; the add that
  // brings the count to `splits` completes the element: that lane converts
  // the sum, stores y and re-arms the accumulator.  Integer addition is
  // associative, so the result does not depend on the order of arrival.
#pragma unroll
  for (int i = 0; i < MROWS; ++i) {
    const int m = (lane >> 4) + i;
    if (m >= M) continue;
    uint16_t* out = y + (int64_t)m * N + n;
    if (splits == 1) {
      *out = float_to_half_bits(yacc[i]);
      continue;
    }
    uint64_t* a = accum + (int64_t)m * ((int64_t)gridDim.x * COLS) + n;
    const uint64_t add = (uint64_t)fixed_partial(yacc[i]) * 64u + 1u;
    const uint64_t old = __hip_atomic_fetch_add(a, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int)(old & 63u) == splits - 1) {
      const int64_t total = (int64_t)(old + add) >> 6;
      *out = float_to_half_bits((float)((double)total * 0x1p-24));
      __hip_atomic_store(a, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Zero the split-K accumulators once, when a workspace is (re)allocated.  A
// fill kernel rather than a memset, so that it is an ordinary kernel node if
// the caller happens to be capturing a graph.
__global__ void msd_zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(msd_zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// The workgroup shape (see the top of this file).
namespace dc {
constexpr int S0_WC = 1, S0_WK = 16, S0_KBW = 2;
constexpr int64_t kMaxSplits = 32;                 // < 64: the accumulators' count field
}  // namespace dc

DecodePlan decode_plan(int gs, int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end) {
  (void)K;
  DecodePlan p;
  (void)M;
  p.shape = 0;
  const int wc = dc::S0_WC;
  const int64_t per = dc::S0_WK * dc::S0_KBW;   // blocks per chunk
  p.cols = wc * kTileCols;
  p.col_blocks = (N + p.cols - 1) / p.cols;
  p.kb_begin = g_begin * gs / kTileRows;
  const int64_t kb_end = (g_end * gs + kTileRows - 1) / kTileRows;
  const int64_t chunks = (kb_end - p.kb_begin + per - 1) / per;
  p.splits = chunks < dc::kMaxSplits ? chunks : dc::kMaxSplits;
  p.nch = (chunks + p.splits - 1) / p.splits;
  p.splits = (chunks + p.nch - 1) / p.nch;
  return p;
}

size_t decode_accum_bytes(const DecodePlan& p, int64_t M, int64_t N) {
  (void)N;
  if (p.splits <= 1) return 0;
  return (size_t)M * (size_t)(p.col_blocks * p.cols) * sizeof(uint64_t);
}

hipError_t launch_decode(const void* x, const void* w, const void* scale, int gs, int64_t M,
                         int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                         int32_t* y_int, uint64_t* accum, const DecodePlan& plan, hipStream_t stream) {
  const dim3 grid((unsigned)plan.col_blocks, (unsigned)plan.splits);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint16_t* sp = static_cast<const uint16_t*>(scale);
  uint16_t* yp = static_cast<uint16_t*>(y);
  const int m = (int)M, k = (int)K, n = (int)N, gb = (int)g_begin, ge = (int)g_end;
  const int kb0 = (int)plan.kb_begin, S = (int)plan.splits, nch = (int)plan.nch;
  if (M > 4 || S > dc::kMaxSplits) return hipErrorInvalidValue;
  if (S > 1 && !y_int && !accum) return hipErrorInvalidValue;
#define WQBMM_DECODE_SHAPE(GS_, Y_)                                                                      \
  hipLaunchKernelGGL((msd_decode_kernel<GS_, dc::S0_WC, dc::S0_WK, dc::S0_KBW, Y_>), grid,             \
                     dim3(64 * dc::S0_WC * dc::S0_WK), 0, stream, xp, wp, sp, m, k, n, gb, ge, kb0, S, nch, \
                     yp, y_int, accum)
  if (gs == 64) {
    if (y_int) WQBMM_DECODE_SHAPE(64, true); else WQBMM_DECODE_SHAPE(64, false);
  } else {
    if (y_int) WQBMM_DECODE_SHAPE(128, true); else WQBMM_DECODE_SHAPE(128, false);
  }
#undef WQBMM_DECODE_SHAPE
  return hipGetLastError();
}

}  // namespace wqbmm
