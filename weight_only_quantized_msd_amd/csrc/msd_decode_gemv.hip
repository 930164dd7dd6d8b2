// msd_decode_gemv.hip -- the MSD matmul for 4 < M <= 96 as two kernels: x is
// decomposed ONCE into int4-packed MFMA operands, then a GEMV-shaped
// contraction streams the weights with every workgroup covering whole K.
//
// WQBMM-Exp page (the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4
// PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145):
// §4.1 steps 1-8 in the operand kernel (the page's pre-processing stage,
// UnfoldA, §6.1), steps 9-11 in the contraction kernel (its Cube matmul and
// MergeY stages).
//
// Why two kernels at this M.  A fused kernel whose workgroups each decompose
// the slice of x they contract repeats the decomposition once per column
// block (about 20 VALU operations per element of x); to keep that slice short
// it has to split K over workgroups and hand partial sums between them, and
// at 16 rows those hand-offs (device-scope atomics, executed past the L2) cost
// more than the weight stream itself.  Decomposing x once costs one short
// launch; the contraction then needs no hand-off at all:
//   workgroup = one 16-column tile of the tiled weights x all of K,
//   wave      = a contiguous run of 128-row blocks (WK waves split K),
//   reduction = the WK waves' fp32 sums added in LDS in a fixed order.
//
// Rows of x come in slices of 16 (R = ceil(M/16) <= 6 slices): each weight
// chunk a wave loads is the MFMA operand of all R slices, so the weights are
// streamed once whatever M is, while the level operands (every row of x, for
// every column tile) grow with R.
//
// Level operands.  Every level value lies in [-7, 7] (7.49 < 7.5 and a
// residual is at most 1/2), so the levels are stored as 4-bit two's
// complement in exactly the nibble arrangement of the tiled weights: chunk
// (128-row block kb, slice r, level l, lane) is 16 bytes at
// (((kb*R + r)*3 + l)*64 + lane)*16; the lane holds row m = 16r + lane%16 at
// k = 128kb + 64s + 16(lane/16) + 8d + j (low nibble of byte 4d + j of step
// s's 8 bytes) and k + 4 (high nibble).
// The same two masks that turn a weight chunk into the i8 MFMA's B operand
// (16*w per byte) turn a level chunk into its A operand (16*a per byte), so
// each product is 256*a*w, exact in int32 (|sum| <= 256*7*8*128 < 2^21).
// Rows m >= M and rows k >= K hold 0.  Beside them the operand kernel stores
// each group's step-10 level weights A_max * w_l as fp32 [G][slice][level][16
// rows] (rows >= M: 0), so that the contraction does not form them once per
// column tile.
#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {

// Step-10 weights of the three levels with the 1/256 that undoes the two
// nibble unpacks (16*a times 16*w).  kC1..kC3 carry 1/16; a further 1/16 is
// an exact power-of-two scaling.
constexpr float kD1 = kC1 * 0.0625f;
constexpr float kD2 = kC2 * 0.0625f;
constexpr float kD3 = kC3 * 0.0625f;

// ---- steps 1-8: x fp16 [M][K] -> level chunks + group maxima ---------------
// One workgroup per (128-row block kb, slice r); thread t = 16m + 8s + 2q + d
// decomposes the 8 elements of row 16r + m at k = 128kb + 64s + 16q + 8d +
// (0..7), which is one dword of each level chunk (lane m + 16q, step s, dword
// d).  A group is GS/8 consecutive, aligned threads (16 at GS = 128: all (s,
// q, d) of a row; 8 at GS = 64: all (q, d) of a row and step), as
// msd_decompose8 requires.
template <int GS>
__global__ __launch_bounds__(256) void msd_decode_operands_kernel(
    const uint16_t* __restrict__ x, int M, int K, int R, uint32_t* __restrict__ lvl,
    float* __restrict__ qt) {
  const int kb = blockIdx.x;
  const int r = blockIdx.y;
  const int t = threadIdx.x;
  const int m = t >> 4, s = (t >> 3) & 1, q = (t >> 1) & 3, d = t & 1;
  const int row = 16 * r + m;
  const int k = kb * kTileRows + 64 * s + 16 * q + 8 * d;
  const bool ok = row < M && k < K;
  const uint4 v = *reinterpret_cast<const uint4*>(x + (ok ? (int64_t)row * K + k : 0));
  const uint4 xv = ok ? v : make_uint4(0u, 0u, 0u, 0u);
  uint32_t lv[3][2];
  float amax;
  msd_decompose8<GS>(xv, lv, amax);
  const int64_t base = (((int64_t)kb * R + r) * 3 * 64 + m + 16 * q) * 4 + 2 * s + d;   // level 0
#pragma unroll
  for (int l = 0; l < 3; ++l)   // byte j: element j (low nibble), element j + 4 (high nibble)
    lvl[base + (int64_t)l * 64 * 4] = (lv[l][0] & 0x0F0F0F0Fu) | ((lv[l][1] & 0x0F0F0F0Fu) << 4);
  if ((t & (GS / 8 - 1)) == 0 && k < K) {   // the group's level weights A_max * w_l (step 10)
    float* qq = qt + ((int64_t)((kb * kTileRows + 64 * s) / GS) * R + r) * 48 + m;
    qq[0] = amax * kD1;
    qq[16] = amax * kD2;
    qq[32] = amax * kD3;
  }
}

// ---- steps 9-11: contraction, combine, accumulate -----------------------------
// Grid: one workgroup per 16-column tile; WK waves, wave w owning the 128-row
// blocks [kb_lo + w*kbw, kb_lo + (w+1)*kbw) of the group range, in rounds of
// KBW blocks.  Per round a wave
//   - loads the round's level weights (contiguous, a few floats per lane) and
//     scales (16 columns x KBW*GS/128 groups, 2-4 bytes per lane) with one or
//     two loads and keeps them in its own LDS slice: per block, per lane
//     loads of them would cost three 4-byte and one 8-byte access of 64 lanes
//     for 48 and 32 distinct bytes;
//   - keeps D blocks of weight and level chunks in flight: the loads of
//     block j+D are issued after the compute of block j;
//   - per 64-row step runs one v_mfma_i32_16x16x64_i8 per slice and level
//     with the weight chunk as the A operand (MFMA row = output column) and
//     the level chunk as the B operand (MFMA column = row of x): D^T = W^T .
//     A_l^T.
// Every load is unconditional and its result unmodified (a block past the
// wave's range reads the round's first block again and its groups are
// dropped by a zero scale; a load under a branch, or a select on its result,
// makes the compiler wait for it right there).  Lane l holds row 16r + l%16
// of x (slice r) for the four consecutive columns 16nt + 4(l/16) + c
// (element c).  Per completed group the three level sums combine with
// A_max*w_l and the scale (step 10) into the lane's fp32 sums (step 11,
// groups ascending within the wave).  The waves' sums are then added in LDS,
// wave 0 first, and wave 0 stores y, 8 bytes per lane and slice.
template <int GS, int WK, int KBW, int R, bool YINT>
__global__ __launch_bounds__(64 * WK) void msd_decode_gemv_kernel(
    const uint8_t* __restrict__ lvl, const float* __restrict__ qt,
    const uint8_t* __restrict__ wt, const uint16_t* __restrict__ scale, int M, int K, int N,
    int g_begin, int g_end, int kb_lo, int kb_hi, int kbw, uint16_t* __restrict__ y,
    int32_t* __restrict__ y_int) {
  constexpr int GPB = kTileRows / GS;            // groups per block
  constexpr int RG = KBW * GPB;                  // groups per round
  constexpr int QG = 48 * R;                     // level weights per group: [slice][level][16 rows]
  constexpr int QF = RG * QG / 64;               // staged level weights per lane
  constexpr int SV = RG * 16 / 64;               // staged scales per lane
  // blocks in flight: at one slice all of a round's (an 8-wave workgroup at
  // K = 4096: its whole share; M = 8-16, K = N = 4096 step about 1% faster than
  // two), at two slices two, beyond that one (registers)
  constexpr int D = R == 1 ? KBW : (R == 2 ? 2 : 1);
  static_assert(QF * 64 == RG * QG && SV * 64 == RG * 16 && (SV == 1 || SV == 2), "round shape");
  static_assert(QG % QF == 0, "a lane's staged level weights lie in one group");
  __shared__ float4 sRed[WK > 1 ? WK - 1 : 1][R][64];
  __shared__ float sQ[YINT ? 1 : WK][YINT ? 1 : RG * QG];                // [group][slice][level][row]
  __shared__ __attribute__((aligned(8))) uint16_t sS[YINT ? 1 : WK][YINT ? 4 : RG * 16];   // [group][col]

  const int lane = threadIdx.x & 63;
  const int wk = threadIdx.x >> 6;
  const int nt = blockIdx.x;
  const int KB = (K + kTileRows - 1) / kTileRows;
  const int G = K / GS;
  const int m = lane & 15;                       // this lane's row of x within its slice
  const int n0 = nt * kTileCols + 4 * (lane >> 4);   // first of its 4 columns
  const int wb_lo = kb_lo + wk * kbw;
  const int wb_hi = min(wb_lo + kbw, kb_hi);

  float yacc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) yacc[r][c] = 0.0f;
  const uint8_t* wcol = wt + (int64_t)nt * KB * 1024 + lane * 16;
  // staging: lane covers level weights [QF*lane, QF*lane + QF) of the round
  // and scales of group sgi, columns sc0 .. sc0 + SV - 1
  const int sgi = lane / (16 / SV);
  const int sc0 = SV * (lane % (16 / SV));

  for (int kb0 = wb_lo; kb0 < wb_hi; kb0 += KBW) {
    v4i av[KBW][R][3], wv[KBW];
    float qst[QF];
    uint32_t sst = 0;
    if constexpr (!YINT) {
      const int g0 = kb0 * GPB;
      const int qo = min(g0 * QG + QF * lane, G * QG - QF);   // past G: any valid floats
#pragma unroll
      for (int i = 0; i < QF; ++i) qst[i] = qt[qo + i];
      const int gc = min(g0 + sgi, G - 1);
      const uint16_t* sp = scale + (int64_t)gc * N + nt * kTileCols + sc0;
      if constexpr (SV == 1) sst = *sp;
      else sst = *reinterpret_cast<const uint32_t*>(sp);
    }
    auto load_block = [&](int j) __attribute__((always_inline)) {
      const int kb = kb0 + j;
      const int kbc = kb < wb_hi ? kb : kb0;
      wv[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wcol + (int64_t)kbc * 1024));
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int l = 0; l < 3; ++l)
          av[j][r][l] = *reinterpret_cast<const v4i*>(lvl + ((((int64_t)kbc * R + r) * 3 + l) * 64 + lane) * 16);
    };
    auto stage = [&]() __attribute__((always_inline)) {
      if constexpr (!YINT) {
#pragma unroll
        for (int i = 0; i < QF; ++i) sQ[wk][QF * lane + i] = qst[i];
        const int g = kb0 * GPB + sgi;
        const bool gok = kb0 + sgi / GPB < wb_hi && g >= g_begin && g < g_end;
        const uint32_t v = gok ? sst : 0u;       // a zero scale drops the group
        if constexpr (SV == 1) sS[wk][lane] = (uint16_t)v;
        else *reinterpret_cast<uint32_t*>(&sS[wk][2 * lane]) = v;
      }
    };
    auto compute_block = [&](int j) __attribute__((always_inline)) {
      v4i acc[R][3];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if ((64 * st) % GS == 0) {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int l = 0; l < 3; ++l) acc[r][l] = v4i{0, 0, 0, 0};
        }
        const uint32_t w0 = (uint32_t)wv[j][2 * st], w1 = (uint32_t)wv[j][2 * st + 1];
        const v4i b = v4i{(int)lo16(w0), (int)hi16(w0), (int)lo16(w1), (int)hi16(w1)};
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int l = 0; l < 3; ++l) {
            const uint32_t a0 = (uint32_t)av[j][r][l][2 * st], a1 = (uint32_t)av[j][r][l][2 * st + 1];
            const v4i a = v4i{(int)lo16(a0), (int)hi16(a0), (int)lo16(a1), (int)hi16(a1)};
            acc[r][l] = mfma_i8(b, a, acc[r][l]);
          }
        if ((64 * st + 64) % GS != 0) continue;                      // group not complete
        const int gl = (64 * st) / GS;
        if constexpr (YINT) {
          const int g = (kb0 + j) * GPB + gl;
          if (kb0 + j >= wb_hi || g < g_begin || g >= g_end) continue;
          const int64_t gi = g - g_begin;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int row = 16 * r + m;
            if (row >= M) continue;
#pragma unroll
            for (int l = 0; l < 3; ++l)
              *reinterpret_cast<v4i*>(y_int + ((gi * 3 + l) * M + row) * (int64_t)N + n0) = acc[r][l] >> 8;
          }
        } else {
          const int gi = j * GPB + gl;
          const uint2 sv = *reinterpret_cast<const uint2*>(&sS[wk][gi * 16 + 4 * (lane >> 4)]);
          const float sc[4] = {half_bits_to_float(sv.x & 0xffffu), half_bits_to_float(sv.x >> 16),
                               half_bits_to_float(sv.y & 0xffffu), half_bits_to_float(sv.y >> 16)};
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float* qg = &sQ[wk][gi * QG + r * 48];
            const float q0 = qg[m], q1 = qg[16 + m], q2 = qg[32 + m];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              float tt = (float)acc[r][0][c] * q0;
              tt = __builtin_fmaf((float)acc[r][1][c], q1, tt);
              tt = __builtin_fmaf((float)acc[r][2][c], q2, tt);
              yacc[r][c] = __builtin_fmaf(tt, sc[c], yacc[r][c]);
            }
          }
        }
      }
    };
    // the scheduling barriers keep each stage's loads where they are written:
    // without them the scheduler moves waits into the loads to save registers
#pragma unroll
    for (int j = 0; j < (D < KBW ? D : KBW); ++j) load_block(j);
    __builtin_amdgcn_sched_barrier(0);
    stage();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < KBW; ++j) {
      compute_block(j);
      __builtin_amdgcn_sched_barrier(0);
      if (j + D < KBW) {
        load_block(j + D);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (YINT) return;

  // ---- the WK waves' sums, added in wave order; wave 0 stores y
  if constexpr (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) sRed[wk - 1][r][lane] = make_float4(yacc[r][0], yacc[r][1], yacc[r][2], yacc[r][3]);
    }
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int v = 0; v < WK - 1; ++v)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float4 p = sRed[v][r][lane];
        yacc[r][0] += p.x; yacc[r][1] += p.y; yacc[r][2] += p.z; yacc[r][3] += p.w;
      }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = 16 * r + m;
    if (row < M) {
      const uint32_t lo = (uint32_t)float_to_half_bits(yacc[r][0]) | ((uint32_t)float_to_half_bits(yacc[r][1]) << 16);
      const uint32_t hi = (uint32_t)float_to_half_bits(yacc[r][2]) | ((uint32_t)float_to_half_bits(yacc[r][3]) << 16);
      *reinterpret_cast<uint2*>(y + (int64_t)row * N + n0) = make_uint2(lo, hi);
    }
  }
}

// ---- steps 9-11 for more column tiles than CUs: level operands read once ---
// With N/16 column tiles beyond the CU count, a workgroup of the kernel above
// would read all of x's level chunks once per column tile (three times the
// bytes of the tile's weights at one slice).  Here a workgroup covers `tpb`
// consecutive column tiles: wave w loads the level chunks of its run of at
// most KBR 128-row blocks ONCE into registers (and its level weights into its
// LDS slice), then streams the weights of one column tile after the other
// through them.  The weights (and scales) of the next two tiles are in
// flight while a tile is computed; per tile the waves' sums are added in LDS
// in wave order and wave 0 stores y, as above.  Same arithmetic and order
// as the kernel above per output, so the two give the same bits.
template <int GS, int WK, int KBR, int R>
__global__ __launch_bounds__(64 * WK) void msd_decode_gemv_multi_kernel(
    const uint8_t* __restrict__ lvl, const float* __restrict__ qt,
    const uint8_t* __restrict__ wt, const uint16_t* __restrict__ scale, int M, int K, int N,
    int g_begin, int g_end, int kb_lo, int kb_hi, int kbw, int tpb, uint16_t* __restrict__ y) {
  constexpr int GPB = kTileRows / GS;            // groups per block
  constexpr int RG = KBR * GPB;                  // groups per wave
  constexpr int QG = 48 * R;                     // level weights per group: [slice][level][16 rows]
  constexpr int QF = RG * QG / 64;               // staged level weights per lane
  constexpr int SV = RG * 16 / 64;               // staged scales per lane
  static_assert(QF * 64 == RG * QG && SV * 64 == RG * 16 && (SV == 1 || SV == 2 || SV == 4), "shape");
  static_assert(QG % QF == 0, "a lane's staged level weights lie in one group");
  __shared__ float4 sRed[WK > 1 ? WK - 1 : 1][R][64];
  __shared__ float sQ[WK][RG * QG];                              // [group][slice][level][row]
  __shared__ __attribute__((aligned(8))) uint16_t sS[2][WK][RG * 16];   // [tile parity][group][col]

  const int lane = threadIdx.x & 63;
  const int wk = threadIdx.x >> 6;
  const int NT = N / kTileCols;
  const int t_lo = blockIdx.x * tpb;
  const int t_hi = min(t_lo + tpb, NT);
  const int KB = (K + kTileRows - 1) / kTileRows;
  const int G = K / GS;
  const int m = lane & 15;
  const int wb_lo = kb_lo + wk * kbw;
  const int wb_hi = min(wb_lo + kbw, kb_hi);
  const bool has = wb_lo < wb_hi;                // wave-uniform: the wave owns blocks
  const int kb_any = has ? wb_lo : 0;            // a valid block for the loads past the run
  const int sgi = lane / (16 / SV);
  const int sc0 = SV * (lane % (16 / SV));

  // the wave's level chunks (all its blocks) and level weights, once
  v4i av[KBR][R][3];
#pragma unroll
  for (int j = 0; j < KBR; ++j) {
    const int kb = wb_lo + j < wb_hi ? wb_lo + j : kb_any;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int l = 0; l < 3; ++l)
        av[j][r][l] = *reinterpret_cast<const v4i*>(lvl + ((((int64_t)kb * R + r) * 3 + l) * 64 + lane) * 16);
  }
  {
    const int g0 = kb_any * GPB;
    const int qo = min(g0 * QG + QF * lane, G * QG - QF);
#pragma unroll
    for (int i = 0; i < QF; ++i) sQ[wk][QF * lane + i] = qt[qo + i];
  }

  // weights and scales of column tile nt (loads only).  The loads are issued
  // whether or not the run has tile nt: past its end every lane reads the
  // first 16 bytes of the weights and the first scales (one line, results
  // unused), so that every path issues the same loads and each tile waits
  // only for its own (a load under a branch leaves the compiler no count to
  // wait for but zero, which also waits for the next tile's loads).
  auto load_tile = [&](int nt, v4i (&wv)[KBR], uint32_t (&sst)[SV == 4 ? 2 : 1]) __attribute__((always_inline)) {
    const bool real = nt < t_hi;                 // uniform
    const uint8_t* wcol = real ? wt + (int64_t)nt * KB * 1024 + lane * 16 : wt;
#pragma unroll
    for (int j = 0; j < KBR; ++j) {
      const int kb = wb_lo + j < wb_hi ? wb_lo + j : kb_any;
      wv[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wcol + (real ? (int64_t)kb * 1024 : 0)));
    }
    const int gc = min(kb_any * GPB + sgi, G - 1);
    const uint16_t* sp = real ? scale + (int64_t)gc * N + nt * kTileCols + sc0 : scale;
    if constexpr (SV == 1) sst[0] = *sp;
    else if constexpr (SV == 2) sst[0] = *reinterpret_cast<const uint32_t*>(sp);
    else {
      const uint2 v = *reinterpret_cast<const uint2*>(sp);
      sst[0] = v.x;
      sst[1] = v.y;
    }
  };
  // stage tile nt's scales (a zero scale drops a group outside the range),
  // contract, reduce over the waves and store y
  auto do_tile = [&](int nt, int par, const v4i (&wv)[KBR], const uint32_t (&sst)[SV == 4 ? 2 : 1]) __attribute__((always_inline)) {
    {
      const int g = kb_any * GPB + sgi;
      const bool gok = has && kb_any + sgi / GPB < wb_hi && g >= g_begin && g < g_end;
      if constexpr (SV == 1) sS[par][wk][lane] = gok ? (uint16_t)sst[0] : (uint16_t)0;
      else if constexpr (SV == 2) *reinterpret_cast<uint32_t*>(&sS[par][wk][2 * lane]) = gok ? sst[0] : 0u;
      else *reinterpret_cast<uint2*>(&sS[par][wk][4 * lane]) = gok ? make_uint2(sst[0], sst[1]) : make_uint2(0u, 0u);
    }
    float yacc[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) yacc[r][c] = 0.0f;
    // Beyond 4 blocks of one slice the level chunks count as redefined per
    // tile, so that their unpacked MFMA operands (twice the registers) are
    // formed per tile; at 4 blocks and one slice they fit, and the compiler
    // keeps them unpacked across the tiles.
    if constexpr (KBR > 4 || R > 1) {
#pragma unroll
      for (int j = 0; j < KBR; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int l = 0; l < 3; ++l) asm volatile("" : "+v"(av[j][r][l]));
    }
    if (has) {
#pragma unroll
      for (int j = 0; j < KBR; ++j) {
        v4i acc[R][3];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          if ((64 * st) % GS == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
              for (int l = 0; l < 3; ++l) acc[r][l] = v4i{0, 0, 0, 0};
          }
          const uint32_t w0 = (uint32_t)wv[j][2 * st], w1 = (uint32_t)wv[j][2 * st + 1];
          const v4i b = v4i{(int)lo16(w0), (int)hi16(w0), (int)lo16(w1), (int)hi16(w1)};
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int l = 0; l < 3; ++l) {
              const uint32_t a0 = (uint32_t)av[j][r][l][2 * st], a1 = (uint32_t)av[j][r][l][2 * st + 1];
              const v4i a = v4i{(int)lo16(a0), (int)hi16(a0), (int)lo16(a1), (int)hi16(a1)};
              acc[r][l] = mfma_i8(b, a, acc[r][l]);
            }
          if ((64 * st + 64) % GS != 0) continue;                    // group not complete
          const int gi = j * GPB + (64 * st) / GS;
          const uint2 sv = *reinterpret_cast<const uint2*>(&sS[par][wk][gi * 16 + 4 * (lane >> 4)]);
          const float sc[4] = {half_bits_to_float(sv.x & 0xffffu), half_bits_to_float(sv.x >> 16),
                               half_bits_to_float(sv.y & 0xffffu), half_bits_to_float(sv.y >> 16)};
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float* qg = &sQ[wk][gi * QG + r * 48];
            const float q0 = qg[m], q1 = qg[16 + m], q2 = qg[32 + m];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              float tt = (float)acc[r][0][c] * q0;
              tt = __builtin_fmaf((float)acc[r][1][c], q1, tt);
              tt = __builtin_fmaf((float)acc[r][2][c], q2, tt);
              yacc[r][c] = __builtin_fmaf(tt, sc[c], yacc[r][c]);
            }
          }
        }
      }
    }
    // the WK waves' sums, added in wave order; wave 0 stores y
    if constexpr (WK > 1) {
      if (wk > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          sRed[wk - 1][r][lane] = make_float4(yacc[r][0], yacc[r][1], yacc[r][2], yacc[r][3]);
      }
      __syncthreads();
      if (wk == 0) {
#pragma unroll
        for (int v = 0; v < WK - 1; ++v)
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float4 p = sRed[v][r][lane];
            yacc[r][0] += p.x; yacc[r][1] += p.y; yacc[r][2] += p.z; yacc[r][3] += p.w;
          }
      }
    }
    if (wk == 0) {
      const int n0 = nt * kTileCols + 4 * (lane >> 4);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = 16 * r + m;
        if (row < M) {
          const uint32_t lo = (uint32_t)float_to_half_bits(yacc[r][0]) | ((uint32_t)float_to_half_bits(yacc[r][1]) << 16);
          const uint32_t hi = (uint32_t)float_to_half_bits(yacc[r][2]) | ((uint32_t)float_to_half_bits(yacc[r][3]) << 16);
          *reinterpret_cast<uint2*>(y + (int64_t)row * N + n0) = make_uint2(lo, hi);
        }
      }
    }
    __syncthreads();   // sRed and this parity's scales are free again
  };

  // a ring of D register sets: the loads of tile t + D are issued as soon as
  // tile t is computed (a third set measured slower: M = 16, K = 4096,
  // N = 11008 contraction 9.1 against 8.3 us; K = 8192, N = 28672, group
  // size 64 42.3 against 35.3 us, where it also spills)
  constexpr int D = 2;
  v4i wr[D][KBR];
  uint32_t sr[D][SV == 4 ? 2 : 1];
#pragma unroll
  for (int i = 0; i < D; ++i) load_tile(t_lo + i, wr[i], sr[i]);
  for (int nt = t_lo; nt < t_hi; nt += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int t = nt + i;
      // uniform; the run's last tile is done (a return, not a break, so that
      // no path reaches the loop head without the loads of the pass before)
      if (t >= t_hi) return;
      do_tile(t, i & 1, wr[i], sr[i]);
      load_tile(t + D, wr[i], sr[i]);
    }
  }
}

namespace dg {
constexpr int WK = 8;    // waves per workgroup (K split within the workgroup)
constexpr int KBW = 4;   // 128-row blocks per wave and load round
constexpr int kMaxSlices = 6;
constexpr int kCUs = 256;   // column tiles beyond this: the multi-tile contraction
}  // namespace dg

int decode_gemv_slices(int64_t M) { return (int)((M + 15) / 16); }

size_t decode_gemv_workspace_bytes(int gs, int64_t M, int64_t K) {
  const int64_t KB = (K + kTileRows - 1) / kTileRows;
  const int64_t R = decode_gemv_slices(M);
  return (size_t)(KB * R) * 3 * 1024 + (size_t)(K / gs) * (size_t)R * 48 * sizeof(float);
}

hipError_t launch_decode_gemv(const void* x, const void* w, const void* scale, int gs, int64_t M,
                              int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                              int32_t* y_int, uint8_t* ws, int stage, hipStream_t stream) {
  const int R = decode_gemv_slices(M);
  if (M < 1 || R > dg::kMaxSlices || N % kTileCols != 0 || stage < 0 || stage > 2)
    return hipErrorInvalidValue;
  const int KB = (int)((K + kTileRows - 1) / kTileRows);
  uint32_t* lvl = reinterpret_cast<uint32_t*>(ws);
  float* qt = reinterpret_cast<float*>(ws + (size_t)KB * R * 3 * 1024);
  if (stage != 2) {
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const dim3 og((unsigned)KB, (unsigned)R);
    if (gs == 64)
      hipLaunchKernelGGL(msd_decode_operands_kernel<64>, og, dim3(256), 0, stream, xp, (int)M, (int)K, R, lvl, qt);
    else
      hipLaunchKernelGGL(msd_decode_operands_kernel<128>, og, dim3(256), 0, stream, xp, (int)M, (int)K, R, lvl, qt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || stage == 1) return e;
  }

  const int kb_lo = (int)(g_begin * gs / kTileRows);
  const int kb_hi = (int)((g_end * gs + kTileRows - 1) / kTileRows);
  const int kbw = (kb_hi - kb_lo + dg::WK - 1) / dg::WK;
  const dim3 grid((unsigned)(N / kTileCols));
  const uint8_t* lp = ws;
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint16_t* sp = static_cast<const uint16_t*>(scale);
  uint16_t* yp = static_cast<uint16_t*>(y);
  const int m = (int)M, k = (int)K, n = (int)N, gb = (int)g_begin, ge = (int)g_end;

  // More column tiles than CUs: a workgroup per run of tpb tiles with the
  // level chunks held in registers (one slice at up to 8 blocks per wave, two
  // slices at up to 4), y only.
  const int64_t NT = N / kTileCols;
  if (!y_int && NT > dg::kCUs && ((R == 1 && kbw <= 8) || (R == 2 && kbw <= 4))) {
    const int tpb = (int)((NT + dg::kCUs - 1) / dg::kCUs);
    const dim3 mgrid((unsigned)((NT + tpb - 1) / tpb));
#define WQBMM_MULTI(GS_, KBR_, R_)                                                                  \
  hipLaunchKernelGGL((msd_decode_gemv_multi_kernel<GS_, dg::WK, KBR_, R_>), mgrid, dim3(64 * dg::WK),  \
                     0, stream, lp, qt, wp, sp, m, k, n, gb, ge, kb_lo, kb_hi, kbw, tpb, yp)
    if (gs == 64) {
      if (R == 2) WQBMM_MULTI(64, 4, 2);
      else if (kbw <= 4) WQBMM_MULTI(64, 4, 1);
      else WQBMM_MULTI(64, 8, 1);
    } else {
      if (R == 2) WQBMM_MULTI(128, 4, 2);
      else if (kbw <= 4) WQBMM_MULTI(128, 4, 1);
      else WQBMM_MULTI(128, 8, 1);
    }
#undef WQBMM_MULTI
    return hipGetLastError();
  }
#define WQBMM_GEMV_LAUNCH(GS_, R_, Y_)                                                              \
  hipLaunchKernelGGL((msd_decode_gemv_kernel<GS_, dg::WK, dg::KBW, R_, Y_>), grid, dim3(64 * dg::WK), 0,   \
                     stream, lp, qt, wp, sp, m, k, n, gb, ge, kb_lo, kb_hi, kbw, yp, y_int)
#define WQBMM_GEMV_R(GS_, Y_)                                                                       \
  do {                                                                                              \
    switch (R) {                                                                                    \
      case 1: WQBMM_GEMV_LAUNCH(GS_, 1, Y_); break;                                                 \
      case 2: WQBMM_GEMV_LAUNCH(GS_, 2, Y_); break;                                                 \
      case 3: WQBMM_GEMV_LAUNCH(GS_, 3, Y_); break;                                                 \
      case 4: WQBMM_GEMV_LAUNCH(GS_, 4, Y_); break;                                                 \
      case 5: WQBMM_GEMV_LAUNCH(GS_, 5, Y_); break;                                                 \
      default: WQBMM_GEMV_LAUNCH(GS_, 6, Y_); break;                                                \
    }                                                                                               \
  } while (0)
  if (gs == 64) {
    if (y_int) WQBMM_GEMV_R(64, true); else WQBMM_GEMV_R(64, false);
  } else {
    if (y_int) WQBMM_GEMV_R(128, true); else WQBMM_GEMV_R(128, false);
  }
#undef WQBMM_GEMV_R
#undef WQBMM_GEMV_LAUNCH
  return hipGetLastError();
}

}  // namespace wqbmm
