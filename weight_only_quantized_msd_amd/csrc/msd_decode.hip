// msd_decode.hip -- fused MSD kernel for small M (decode, M <= 16).
//
// WQBMM-Exp page (the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4
// PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145):
// all of §4.1 (steps 1-11) in ONE launch.  The page's BASIC_MSD template runs
// pre-process (UnfoldA), Cube matmul and post-process (MergeY) as serial
// stages with full-core syncs (§6.1), and its PRELOAD_MSD template overlaps
// them across loop rounds with double/triple buffers (§6.2).  At small M the
// cost is streaming the int4 weights, so here every workgroup issues all of
// its weight loads first and decomposes its slice of x while they are in
// flight; the three stages then run back to back in registers and LDS.
//
// Work split (one GPU, intra-device version of the page's N-split across
// cores, §8.1 nGmOffset = baseN * blockIdx):
//   workgroup = 128 columns (64 bytes of each W row) x 512 rows of K,
//   4 waves, one per 128-row slice (one group at GS=128, two at GS=64).
//   Lane l reads the dword of 8 columns at chunk (l%16) from the 16 rows
//   16*(l/16) .. 16*(l/16)+15 of each 64-row MFMA step; transpose4x4 turns
//   them into eight B operands (one per column) of v_mfma_i32_16x16x64_i8.
// Rows of the MFMA A operand ("slots"):
//   LAYOUT 0 (M <= 4):  slot 4*m + level, one 16-row tile, levels of a row
//                       land in elements 0..2 of the same lane's accumulator;
//   LAYOUT 1 (M <= 16): tile = level, slot = m, three tiles.
// Split-K: each workgroup writes an fp32 partial; the last workgroup of a
// column block (atomic counter) sums the partials in split order (fixed, so
// the result is deterministic) and stores fp16 y, then re-arms the counter.
#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {
namespace dc {
constexpr int THREADS = 256;
constexpr int COLS = 128;        // columns per workgroup
constexpr int WAVE_ROWS = 128;   // K rows per wave
constexpr int KW = 4 * WAVE_ROWS;  // K rows per workgroup
constexpr int PAD = 16;
constexpr int ROWA = KW + PAD;   // LDS bytes per A slot row
}  // namespace dc

template <int GS, int LAYOUT, bool YINT>
__global__ __launch_bounds__(256) void msd_decode_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int M, int K, int N, int g_begin, int g_end,
    int splits, uint16_t* __restrict__ y, int32_t* __restrict__ y_int,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
  using namespace dc;
  constexpr int RT = LAYOUT == 0 ? 1 : 3;      // 16-row A tiles
  constexpr int MT = LAYOUT == 0 ? 4 : 16;     // rows of x covered by the slots
  constexpr int GPW = WAVE_ROWS / GS;          // groups per wave
  constexpr int GPB = KW / GS;                 // groups per workgroup
  constexpr int NACC = LAYOUT == 0 ? 8 : 32;   // fp32 partial outputs per lane

  __shared__ __attribute__((aligned(16))) int8_t sA[16 * RT * ROWA];
  __shared__ float sAmax[MT][GPB];
  __shared__ float sRed[3][64][NACC];
  __shared__ int sLast;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nb = blockIdx.x;
  const int s = blockIdx.y;
  const int NB2 = N / 2;
  const int kend = g_end * GS;                           // exclusive row bound
  const int kblk = g_begin * GS + s * KW;                // first row of this workgroup
  const int kwave = kblk + wave * WAVE_ROWS;             // first row of this wave
  const int col_lane = nb * COLS + 8 * (lane & 15);      // first of the lane's 8 columns
  const bool col_ok = col_lane < N;                      // N % 32 == 0: chunks all-in or all-out

  // ---- 1. issue every W load of this wave (2 MFMA steps x 16 rows, 1 dword each)
  uint32_t raw[2][16];
  {
    const uint8_t* wl = w + col_lane / 2;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k = kwave + ks * 64 + 16 * (lane >> 4) + r;
        raw[ks][r] = (col_ok && k < kend) ? __builtin_nontemporal_load(
                                                reinterpret_cast<const uint32_t*>(wl + (int64_t)k * NB2))
                                          : 0u;
      }
  }

  // ---- 2. steps 1-8 for x[0:MT][kblk : kblk+KW] into LDS (A operand layout)
  constexpr int ITEMS = MT * (KW / 8);
  for (int it = tid; it < ITEMS; it += THREADS) {   // ITEMS % 256 == 0: uniform trip count
    const int m = it / (KW / 8);
    const int ch = it % (KW / 8);
    const int k = kblk + ch * 8;
    uint4 xv = make_uint4(0u, 0u, 0u, 0u);
    if (m < M && k < kend) xv = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + k);
    uint32_t lv[3][2];
    float amax;
    msd_decompose8<GS>(xv, lv, amax);
#pragma unroll
    for (int l = 0; l < 3; ++l) {
      const int slot = LAYOUT == 0 ? (4 * m + l) : (l * 16 + m);
      *reinterpret_cast<uint2*>(sA + slot * ROWA + ch * 8) = make_uint2(lv[l][0], lv[l][1]);
    }
    if (LAYOUT == 0) *reinterpret_cast<uint2*>(sA + (4 * m + 3) * ROWA + ch * 8) = make_uint2(0u, 0u);
    if ((ch & (GS / 8 - 1)) == 0) sAmax[m][(ch * 8) / GS] = amax;
  }
  __syncthreads();

  // ---- 3. per group: step 9 on MFMA, then steps 10-11 (or the Y_int export)
  float yacc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) yacc[j] = 0.0f;

#pragma unroll
  for (int gl = 0; gl < GPW; ++gl) {
    v4i acc[RT][8];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[t][c] = v4i{0, 0, 0, 0};

#pragma unroll
    for (int kk = 0; kk < GS / 64; ++kk) {
      const int ks = gl * (GS / 64) + kk;
      v4i bf[8];
      {
        uint32_t e[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          transpose4x4(raw[ks][4 * q], raw[ks][4 * q + 1], raw[ks][4 * q + 2], raw[ks][4 * q + 3],
                       e[q][0], e[q][1], e[q][2], e[q][3]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          bf[2 * b] = v4i{(int)lo16(e[0][b]), (int)lo16(e[1][b]), (int)lo16(e[2][b]), (int)lo16(e[3][b])};
          bf[2 * b + 1] = v4i{(int)hi16(e[0][b]), (int)hi16(e[1][b]), (int)hi16(e[2][b]), (int)hi16(e[3][b])};
        }
      }
      const int kofs = wave * WAVE_ROWS + ks * 64 + 16 * (lane >> 4);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const v4i af = *reinterpret_cast<const v4i*>(sA + (t * 16 + (lane & 15)) * ROWA + kofs);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[t][c] = mfma_i8(af, bf[c], acc[t][c]);
      }
    }

    const int gloc = wave * GPW + gl;          // group index within the workgroup
    const int g = kblk / GS + gloc;            // absolute group index
    if (g >= g_end) continue;                  // wave-uniform

    if constexpr (YINT) {
      const int64_t gi = g - g_begin;
#pragma unroll
      for (int i = 0; i < (LAYOUT == 0 ? 1 : 4); ++i) {
        const int m = LAYOUT == 0 ? (lane >> 4) : 4 * (lane >> 4) + i;
        if (m >= M || !col_ok) continue;
#pragma unroll
        for (int l = 0; l < 3; ++l) {
          int32_t* out = y_int + ((gi * 3 + l) * M + m) * (int64_t)N + col_lane;
          int v[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) v[c] = (LAYOUT == 0 ? acc[0][c][l] : acc[l][c][i]) >> 4;
          *reinterpret_cast<int4*>(out) = make_int4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<int4*>(out + 4) = make_int4(v[4], v[5], v[6], v[7]);
        }
      }
    } else {
      float sc[8];
      {
        uint4 sv = make_uint4(0u, 0u, 0u, 0u);
        if (col_ok) sv = *reinterpret_cast<const uint4*>(scale + (int64_t)g * N + col_lane);
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[2 * i] = half_bits_to_float(sw[i] & 0xffffu);
          sc[2 * i + 1] = half_bits_to_float(sw[i] >> 16);
        }
      }
      if constexpr (LAYOUT == 0) {
        const int m = lane >> 4;
        const float am = sAmax[m][gloc];
        const float q1 = am * kC1, q2 = am * kC2, q3 = am * kC3;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float t = (float)acc[0][c][0] * q1;
          t = __builtin_fmaf((float)acc[0][c][1], q2, t);
          t = __builtin_fmaf((float)acc[0][c][2], q3, t);
          yacc[c] = __builtin_fmaf(t, sc[c], yacc[c]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float am = sAmax[4 * (lane >> 4) + i][gloc];
          const float q1 = am * kC1, q2 = am * kC2, q3 = am * kC3;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            float t = (float)acc[0][c][i] * q1;
            t = __builtin_fmaf((float)acc[1][c][i], q2, t);
            t = __builtin_fmaf((float)acc[2][c][i], q3, t);
            yacc[i * 8 + c] = __builtin_fmaf(t, sc[c], yacc[i * 8 + c]);
          }
        }
      }
    }
  }
  if constexpr (YINT) return;

  // ---- 4. reduce the four waves (fixed order: wave 0 + 1 + 2 + 3)
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < NACC; ++j) sRed[wave - 1][lane][j] = yacc[j];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int v = 0; v < 3; ++v)
#pragma unroll
      for (int j = 0; j < NACC; ++j) yacc[j] += sRed[v][lane][j];
  }

  // ---- 5. split-K: direct store, or partial + last-workgroup reduction
  constexpr int MROWS = LAYOUT == 0 ? 1 : 4;
  if (splits == 1) {
    if (wave == 0 && col_ok) {
#pragma unroll
      for (int i = 0; i < MROWS; ++i) {
        const int m = LAYOUT == 0 ? (lane >> 4) : 4 * (lane >> 4) + i;
        if (m >= M) continue;
        uint32_t h[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          h[c] = (uint32_t)float_to_half_bits(yacc[i * 8 + 2 * c]) |
                 ((uint32_t)float_to_half_bits(yacc[i * 8 + 2 * c + 1]) << 16);
        *reinterpret_cast<uint4*>(y + (int64_t)m * N + col_lane) = make_uint4(h[0], h[1], h[2], h[3]);
      }
    }
    return;
  }

  const int64_t npad = (int64_t)gridDim.x * COLS;
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < MROWS; ++i) {
      const int m = LAYOUT == 0 ? (lane >> 4) : 4 * (lane >> 4) + i;
      if (m >= M) continue;
      float* p = partials + ((int64_t)s * M + m) * npad + col_lane;
      *reinterpret_cast<float4*>(p) = make_float4(yacc[i * 8 + 0], yacc[i * 8 + 1], yacc[i * 8 + 2], yacc[i * 8 + 3]);
      *reinterpret_cast<float4*>(p + 4) = make_float4(yacc[i * 8 + 4], yacc[i * 8 + 5], yacc[i * 8 + 6], yacc[i * 8 + 7]);
    }
  }
  __threadfence();   // release this workgroup's partial at device scope
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&counters[nb], 1u);
    sLast = (prev == (uint32_t)(splits - 1));
  }
  __syncthreads();
  if (!sLast) return;
  __threadfence();   // acquire: every partial of this column block is visible
  for (int e = tid; e < M * COLS; e += THREADS) {
    const int m = e / COLS, c = e % COLS;
    const int n = nb * COLS + c;
    float sum = 0.0f;
    for (int sp = 0; sp < splits; ++sp) sum += partials[((int64_t)sp * M + m) * npad + n];
    if (n < N) y[(int64_t)m * N + n] = float_to_half_bits(sum);
  }
  if (tid == 0) atomicExch(&counters[nb], 0u);   // re-arm for the next launch
}

DecodePlan decode_plan(int gs, int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end) {
  (void)M; (void)K;
  DecodePlan p;
  p.col_blocks = (N + dc::COLS - 1) / dc::COLS;
  p.splits = ((g_end - g_begin) * gs + dc::KW - 1) / dc::KW;
  return p;
}

size_t decode_partials_bytes(const DecodePlan& p, int64_t M, int64_t N) {
  (void)N;
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * (size_t)M * (size_t)(p.col_blocks * dc::COLS) * sizeof(float);
}

size_t decode_counter_bytes(const DecodePlan& p) { return (size_t)p.col_blocks * sizeof(uint32_t); }

hipError_t launch_decode(const void* x, const void* w, const void* scale, int gs, int64_t M,
                         int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                         int32_t* y_int, float* partials, uint32_t* counters,
                         const DecodePlan& plan, hipStream_t stream) {
  const dim3 grid((unsigned)plan.col_blocks, (unsigned)plan.splits);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint16_t* sp = static_cast<const uint16_t*>(scale);
  uint16_t* yp = static_cast<uint16_t*>(y);
  const int m = (int)M, k = (int)K, n = (int)N, gb = (int)g_begin, ge = (int)g_end;
  const int S = (int)plan.splits;
#define WQBMM_DECODE_LAUNCH(GS_, L_, Y_)                                                          \
  hipLaunchKernelGGL((msd_decode_kernel<GS_, L_, Y_>), grid, dim3(dc::THREADS), 0, stream, xp, wp, \
                     sp, m, k, n, gb, ge, S, yp, y_int, partials, counters)
  const bool yint = y_int != nullptr;
  const int layout = M <= 4 ? 0 : 1;
  if (gs == 64) {
    if (layout == 0) { if (yint) WQBMM_DECODE_LAUNCH(64, 0, true); else WQBMM_DECODE_LAUNCH(64, 0, false); }
    else             { if (yint) WQBMM_DECODE_LAUNCH(64, 1, true); else WQBMM_DECODE_LAUNCH(64, 1, false); }
  } else {
    if (layout == 0) { if (yint) WQBMM_DECODE_LAUNCH(128, 0, true); else WQBMM_DECODE_LAUNCH(128, 0, false); }
    else             { if (yint) WQBMM_DECODE_LAUNCH(128, 1, true); else WQBMM_DECODE_LAUNCH(128, 1, false); }
  }
#undef WQBMM_DECODE_LAUNCH
  return hipGetLastError();
}

}  // namespace wqbmm
