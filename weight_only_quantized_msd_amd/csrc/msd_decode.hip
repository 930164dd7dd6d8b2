// msd_decode.hip -- fused MSD kernel for small M (decode, M <= 16).
//
// WQBMM-Exp page (the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4
// PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145):
// all of §4.1 (steps 1-11) in one launch.  The page's BASIC_MSD template runs
// pre-process (UnfoldA), Cube matmul and post-process (MergeY) as serial
// stages with full-core syncs (§6.1), and its PRELOAD_MSD template overlaps
// them across loop rounds with double/triple buffers (§6.2).  At small M the
// cost is streaming the int4 weights, so here every workgroup issues all of
// its weight loads first and decomposes its slice of x while they are in
// flight; the three stages then run back to back in registers and LDS.
//
// Work split (one GPU; the intra-device form of the page's N split across
// cores, §8.1 nGmOffset = baseN * blockIdx, plus a split of K):
//   wave      = 128 columns (64 bytes of each W row) x 128 rows of K
//               (one group at GS=128, two at GS=64);
//   workgroup = WN waves side by side in N x WK waves stacked in K.  With
//               WN = 2 a workgroup reads whole 128-byte lines of each row; a
//               tile that takes half lines (the other half going to another
//               workgroup, usually on another XCD) streamed about 1.45x
//               slower in a plain read test of the same 8 MiB.
//   Lane l reads the dword of 8 columns at chunk (l%16) from the 16 rows
//   16*(l/16) .. 16*(l/16)+15 of each 64-row MFMA step; transpose4x4 turns
//   them into eight B operands (one per column) of v_mfma_i32_16x16x64_i8.
// Rows of the MFMA A operand ("slots"):
//   LAYOUT 0 (M <= 4):  slot 4*m + level, one 16-row tile, the levels of a
//                       row land in elements 0..2 of one lane's accumulator;
//   LAYOUT 1 (M <= 16): tile = level, slot = m, three tiles.
//
// Split-K: each workgroup sums its WK waves in LDS; when K is split over
// several workgroups the partials are combined in split order (fixed, so the
// result is deterministic) in one of two ways:
//  * HANDOFF_LAST (M <= 4, small partials): each workgroup publishes its fp32
//    partial with device-scope atomic stores, waits until they are complete,
//    and bumps a per-column-block counter; the workgroup that bumps it last
//    reads every partial back with device-scope atomic loads, stores fp16 y
//    and re-arms the counter.  One launch; no workgroup waits for another and
//    no device-scope fence is issued (on gfx950 such a fence writes back and
//    invalidates the whole L2 of the XCD; one per workgroup dominated the run
//    time of an earlier version).
//  * HANDOFF_KERNEL (M > 4): partials are written with plain stores and a
//    second kernel, spread over the whole GPU, sums them.  At M = 16 the
//    partials are a large fraction of the weight bytes, and funnelling their
//    gather through one workgroup per column block was the slowest phase.
#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {
namespace dc {
constexpr int WAVE_COLS = 128;   // columns per wave
constexpr int WAVE_ROWS = 128;   // K rows per wave
constexpr int PAD = 16;
}  // namespace dc

enum Handoff { HANDOFF_STORE_Y = 0, HANDOFF_LAST = 1, HANDOFF_KERNEL = 2 };

template <int GS, int LAYOUT, int WN, int WK, bool YINT>
__global__ __launch_bounds__(64 * WN * WK) void msd_decode_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int M, int K, int N, int g_begin, int g_end,
    int splits, int handoff, uint16_t* __restrict__ y, int32_t* __restrict__ y_int,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
  using namespace dc;
  constexpr int THREADS = 64 * WN * WK;
  constexpr int COLS = WAVE_COLS * WN;          // columns per workgroup
  constexpr int KW = WAVE_ROWS * WK;            // K rows per workgroup
  constexpr int ROWA = KW + PAD;                // LDS bytes per A slot row
  constexpr int RT = LAYOUT == 0 ? 1 : 3;       // 16-row A tiles
  constexpr int MT = LAYOUT == 0 ? 4 : 16;      // rows of x covered by the slots
  constexpr int GPW = WAVE_ROWS / GS;           // groups per wave
  constexpr int GPB = KW / GS;                  // groups per workgroup
  constexpr int MROWS = LAYOUT == 0 ? 1 : 4;    // output rows per lane
  constexpr int NACC = 8 * MROWS;               // fp32 outputs per lane

  __shared__ __attribute__((aligned(16))) int8_t sA[16 * RT * ROWA];
  __shared__ float sAmax[MT][GPB];
  __shared__ float sRed[WK > 1 ? WK - 1 : 1][WN][NACC][64];   // lane fastest: conflict-free
  __shared__ int sLast;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % WN;                     // column stripe of this wave
  const int wk = wave / WN;                     // K slice of this wave
  const int nb = blockIdx.x;
  const int s = blockIdx.y;
  const int NB2 = N / 2;
  const int kend = g_end * GS;                             // exclusive row bound
  const int kblk = g_begin * GS + s * KW;                  // first row of this workgroup
  const int kwave = kblk + wk * WAVE_ROWS;                 // first row of this wave
  const int col_lane = nb * COLS + wn * WAVE_COLS + 8 * (lane & 15);
  const bool col_ok = col_lane < N;                        // N % 32 == 0: chunks all-in or all-out

  // ---- 1. this thread's x chunks first (so waiting for them does not wait
  //         for the weights), then every W load of this wave.  Loads are
  //         unconditional (out-of-range ones read a valid address and are
  //         zeroed afterwards): a load under a branch makes the compiler wait
  //         for every outstanding load at the join, which would stall the
  //         decomposition until all weights have arrived.
  constexpr int ITEMS = MT * (KW / 8);
  constexpr int ROUNDS = (ITEMS + THREADS - 1) / THREADS;
  uint4 xv[ROUNDS];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int it = rd * THREADS + tid;
    const int m = it / (KW / 8);
    const int k = kblk + (it % (KW / 8)) * 8;
    const bool ok = it < ITEMS && m < M && k < kend;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (ok ? (int64_t)m * K + k : 0));
    xv[rd] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
  }
  // per-group scales of this lane's 8 columns (step 10), prefetched now so
  // the epilogue does not wait for them
  uint4 sv[GPW];
#pragma unroll
  for (int gl = 0; gl < GPW; ++gl) {
    const int g = (kwave / GS) + gl;
    if constexpr (YINT) {
      sv[gl] = make_uint4(0u, 0u, 0u, 0u);
    } else {
      const bool ok = col_ok && g < g_end;
      const uint4 v = *reinterpret_cast<const uint4*>(scale + (ok ? (int64_t)g * N + col_lane : 0));
      sv[gl] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  uint32_t raw[2][16];
  {
    const uint8_t* wl = w + (col_ok ? col_lane / 2 : 0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k = kwave + ks * 64 + 16 * (lane >> 4) + r;
        const bool ok = col_ok && k < kend;
        const uint32_t v = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>(wl + (int64_t)(ok ? k : 0) * NB2));
        raw[ks][r] = ok ? v : 0u;
      }
  }

  // ---- 2. steps 1-8 for x[0:MT][kblk : kblk+KW] into LDS (A operand layout).
  // Every lane of a wave runs the same rounds (the group maximum is a
  // cross-lane reduction); items past the end decompose zeros and are dropped.
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int it = rd * THREADS + tid;
    const int m = it / (KW / 8);
    const int ch = it % (KW / 8);
    uint32_t lv[3][2];
    float amax;
    msd_decompose8<GS>(xv[rd], lv, amax);
    if (it < ITEMS) {
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        const int slot = LAYOUT == 0 ? (4 * m + l) : (l * 16 + m);
        *reinterpret_cast<uint2*>(sA + slot * ROWA + ch * 8) = make_uint2(lv[l][0], lv[l][1]);
      }
      if (LAYOUT == 0) *reinterpret_cast<uint2*>(sA + (4 * m + 3) * ROWA + ch * 8) = make_uint2(0u, 0u);
      if ((ch & (GS / 8 - 1)) == 0) sAmax[m][(ch * 8) / GS] = amax;
    }
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
      const int kofs = wk * WAVE_ROWS + ks * 64 + 16 * (lane >> 4);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const v4i af = *reinterpret_cast<const v4i*>(sA + (t * 16 + (lane & 15)) * ROWA + kofs);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[t][c] = mfma_i8(af, bf[c], acc[t][c]);
      }
    }

    const int gloc = wk * GPW + gl;            // group index within the workgroup
    const int g = kblk / GS + gloc;            // absolute group index
    if (g >= g_end) continue;                  // wave-uniform

    if constexpr (YINT) {
      const int64_t gi = g - g_begin;
#pragma unroll
      for (int i = 0; i < MROWS; ++i) {
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
        const uint32_t sw[4] = {sv[gl].x, sv[gl].y, sv[gl].z, sv[gl].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[2 * i] = half_bits_to_float(sw[i] & 0xffffu);
          sc[2 * i + 1] = half_bits_to_float(sw[i] >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < MROWS; ++i) {
        const int m = LAYOUT == 0 ? (lane >> 4) : 4 * (lane >> 4) + i;
        const float am = sAmax[m][gloc];
        const float q1 = am * kC1, q2 = am * kC2, q3 = am * kC3;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int y1 = LAYOUT == 0 ? acc[0][c][0] : acc[0][c][i];
          const int y2 = LAYOUT == 0 ? acc[0][c][1] : acc[1][c][i];
          const int y3 = LAYOUT == 0 ? acc[0][c][2] : acc[2][c][i];
          float t = (float)y1 * q1;
          t = __builtin_fmaf((float)y2, q2, t);
          t = __builtin_fmaf((float)y3, q3, t);
          yacc[i * 8 + c] = __builtin_fmaf(t, sc[c], yacc[i * 8 + c]);
        }
      }
    }
  }
  if constexpr (YINT) return;

  // ---- 4. sum the WK waves of each column stripe (fixed order 0, 1, ...)
  if constexpr (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int j = 0; j < NACC; ++j) sRed[wk - 1][wn][j][lane] = yacc[j];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int v = 0; v < WK - 1; ++v)
#pragma unroll
        for (int j = 0; j < NACC; ++j) yacc[j] += sRed[v][wn][j][lane];
    }
  }

  // ---- 5. one split: store y.  Several: hand the partial off.
  if (handoff == HANDOFF_STORE_Y) {
    if (wk == 0 && col_ok) {
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
  if (handoff == HANDOFF_KERNEL) {
    if (wk == 0) {
#pragma unroll
      for (int i = 0; i < MROWS; ++i) {
        const int m = LAYOUT == 0 ? (lane >> 4) : 4 * (lane >> 4) + i;
        if (m >= M) continue;
        float* p = partials + ((int64_t)s * M + m) * npad + col_lane;
        *reinterpret_cast<float4*>(p) = make_float4(yacc[i * 8 + 0], yacc[i * 8 + 1], yacc[i * 8 + 2], yacc[i * 8 + 3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(yacc[i * 8 + 4], yacc[i * 8 + 5], yacc[i * 8 + 6], yacc[i * 8 + 7]);
      }
    }
    return;
  }
  if (wk == 0) {
#pragma unroll
    for (int i = 0; i < MROWS; ++i) {
      const int m = LAYOUT == 0 ? (lane >> 4) : 4 * (lane >> 4) + i;
      if (m >= M) continue;
      uint64_t* p = reinterpret_cast<uint64_t*>(partials + ((int64_t)s * M + m) * npad + col_lane);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint64_t v = (uint64_t)__float_as_uint(yacc[i * 8 + 2 * c]) |
                           ((uint64_t)__float_as_uint(yacc[i * 8 + 2 * c + 1]) << 32);
        __hip_atomic_store(p + c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // every partial store of this thread has completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&counters[nb], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sLast = (prev == (uint32_t)(splits - 1));
  }
  __syncthreads();
  if (!sLast) return;
  // gather: one task = one row x 2 columns; the loads of 8 splits are issued
  // together before they are summed, in split order
  for (int e = tid; e < M * (COLS / 2); e += THREADS) {
    const int m = e / (COLS / 2);
    const int n = nb * COLS + (e % (COLS / 2)) * 2;
    if (n >= N) continue;
    const uint64_t* p = reinterpret_cast<const uint64_t*>(partials + (int64_t)m * npad + n);
    const int64_t sstride = (int64_t)M * npad / 2;   // uint64 words between splits
    float s0 = 0.0f, s1 = 0.0f;
    for (int sp0 = 0; sp0 < splits; sp0 += 8) {
      uint64_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = (sp0 + j < splits)
                   ? __hip_atomic_load(p + (int64_t)(sp0 + j) * sstride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : 0ull;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (sp0 + j < splits) {
          s0 += __uint_as_float((uint32_t)v[j]);
          s1 += __uint_as_float((uint32_t)(v[j] >> 32));
        }
      }
    }
    *reinterpret_cast<uint32_t*>(y + (int64_t)m * N + n) =
        (uint32_t)float_to_half_bits(s0) | ((uint32_t)float_to_half_bits(s1) << 16);
  }
  if (tid == 0) __hip_atomic_store(&counters[nb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// HANDOFF_KERNEL: sum of the split-K partials in split order, fp32, then one
// RNE cast to fp16.  One workgroup per (row, 64 columns): thread (sp, c) loads
// the 4 columns c of split sp (16 splits per pass, all loads in flight
// together), then 16 threads add the splits in order.
__global__ __launch_bounds__(256) void msd_splitk_reduce_kernel(const float* __restrict__ partials,
                                                                int splits, int M, int N, int64_t npad,
                                                                uint16_t* __restrict__ y) {
  __shared__ float4 sP[16][16];
  const int tid = threadIdx.x;
  const int c = tid & 15;             // float4 chunk within the 64 columns
  const int sp = tid >> 4;            // split within the pass
  const int64_t m = blockIdx.y;
  const int64_t n = (int64_t)blockIdx.x * 64 + 4 * c;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += 16) {
    const bool ok = s0 + sp < splits && n < N;
    const float4 v = *reinterpret_cast<const float4*>(
        partials + (ok ? ((int64_t)(s0 + sp) * M + m) * npad + n : 0));
    sP[sp][c] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
    if (tid < 16) {
      const int cnt = splits - s0 < 16 ? splits - s0 : 16;
      for (int j = 0; j < cnt; ++j) {
        const float4 t = sP[j][c];
        acc.x += t.x; acc.y += t.y; acc.z += t.z; acc.w += t.w;
      }
    }
    __syncthreads();
  }
  if (tid < 16 && n < N) {
    const uint32_t h0 = (uint32_t)float_to_half_bits(acc.x) | ((uint32_t)float_to_half_bits(acc.y) << 16);
    const uint32_t h1 = (uint32_t)float_to_half_bits(acc.z) | ((uint32_t)float_to_half_bits(acc.w) << 16);
    *reinterpret_cast<uint2*>(y + m * N + n) = make_uint2(h0, h1);
  }
}

// Zero the split-K counters once, when a workspace is (re)allocated.  A fill
// kernel rather than a memset, so that it is an ordinary kernel node if the
// caller happens to be capturing a graph.
__global__ void msd_zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_counters(uint32_t* counters, int64_t n, hipStream_t stream) {
  hipLaunchKernelGGL(msd_zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     counters, n);
  return hipGetLastError();
}

// Launch shape: WN = 2 waves across one 128-byte line of each W row; WK waves
// down K.  WK = 4 unless that leaves fewer than 192 workgroups (then 2).
DecodePlan decode_plan(int gs, int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end) {
  (void)K; (void)M;
  DecodePlan p;
  p.wn = 2;
  p.cols = dc::WAVE_COLS * p.wn;
  p.col_blocks = (N + p.cols - 1) / p.cols;
  const int64_t krows = (g_end - g_begin) * gs;
  p.wk = 4;
  if (p.col_blocks * ((krows + dc::WAVE_ROWS * 4 - 1) / (dc::WAVE_ROWS * 4)) < 192) p.wk = 2;
  p.splits = (krows + dc::WAVE_ROWS * p.wk - 1) / (dc::WAVE_ROWS * p.wk);
  return p;
}

size_t decode_partials_bytes(const DecodePlan& p, int64_t M, int64_t N) {
  (void)N;
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * (size_t)M * (size_t)(p.col_blocks * p.cols) * sizeof(float);
}

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
#define WQBMM_DECODE_LAUNCH(GS_, L_, WN_, WK_, Y_)                                              \
  hipLaunchKernelGGL((msd_decode_kernel<GS_, L_, WN_, WK_, Y_>), grid, dim3(64 * (WN_) * (WK_)), \
                     0, stream, xp, wp, sp, m, k, n, gb, ge, S, handoff, yp, y_int, partials, counters)
#define WQBMM_DECODE_WK(GS_, L_, Y_)                                  \
  do {                                                                \
    if (plan.wk == 4) WQBMM_DECODE_LAUNCH(GS_, L_, 2, 4, Y_);         \
    else WQBMM_DECODE_LAUNCH(GS_, L_, 2, 2, Y_);                      \
  } while (0)
  const bool yint = y_int != nullptr;
  const int layout = M <= 4 ? 0 : 1;
  const int handoff = (yint || S == 1) ? HANDOFF_STORE_Y : (layout == 0 ? HANDOFF_LAST : HANDOFF_KERNEL);
  if (plan.wn != 2 || (plan.wk != 2 && plan.wk != 4)) return hipErrorInvalidValue;
  if (gs == 64) {
    if (layout == 0) { if (yint) WQBMM_DECODE_WK(64, 0, true); else WQBMM_DECODE_WK(64, 0, false); }
    else             { if (yint) WQBMM_DECODE_WK(64, 1, true); else WQBMM_DECODE_WK(64, 1, false); }
  } else {
    if (layout == 0) { if (yint) WQBMM_DECODE_WK(128, 0, true); else WQBMM_DECODE_WK(128, 0, false); }
    else             { if (yint) WQBMM_DECODE_WK(128, 1, true); else WQBMM_DECODE_WK(128, 1, false); }
  }
#undef WQBMM_DECODE_WK
  if (handoff == HANDOFF_KERNEL) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(msd_splitk_reduce_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)M), dim3(256), 0,
                       stream, partials, S, m, n, (int64_t)plan.col_blocks * plan.cols, yp);
  }
#undef WQBMM_DECODE_LAUNCH
  return hipGetLastError();
}

}  // namespace wqbmm
