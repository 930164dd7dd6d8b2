// msd_prefill64.hip -- the prefill path for group size 64: an operand
// preparation kernel and an MFMA GEMM built on v_mfma_scale_f32_32x32x64_f8f6f4,
// whose K of 64 is exactly one group.
//
// WQBMM-Exp page (the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4
// PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145):
//   §4.1 steps 1-8   per (row, group) A_max and the three levels A1..A3
//   §4.1 step 9      Y_l = A_l . Weight_group, exact, on FP6 MFMAs
//   §4.1 steps 10-11 combine, scale and accumulate over groups in fp32
//   §6.2             PRELOAD_MSD: data movement ahead of the matmul
//
// Why a kernel of its own.  The 16x16x128 FP6 MFMA of the group-128 GEMM
// covers 128 k; a group of 64 would fill half of every operand with zeros
// (half the MFMA work and twice the operand bytes wasted).  The 32x32x64
// form contracts exactly one group.  The integer arithmetic is the same: both
// operands e2m3 (levels as they are, weights halved with the B... here the
// weight operand's E8M0 block scale 2^1), every product exact, a group's sum
// |Y_l| <= 7*8*64 = 3584 exact in the fp32 accumulator.
//
// Roles: the MFMA's A operand is the weights (its 32 "rows" are 32 output
// columns n) and its B operand is x (its 32 "columns" are 32 rows m of x), so
// D^T = W^T . X^T.  A lane then holds one row m of x in all 16 of its
// results, and the step-10 weights of that row (A_max * w_l, three values)
// are per lane; the scales vary with the result element (16 columns per
// lane, four runs of four consecutive columns).
//
// Operand tiles (1536 bytes: [lane][dwords 0-3] then [lane][dwords 4-5], as
// in the group-128 path): lane l holds row/column l%32 and the 32 values at
// group-relative k = 32*(l/32) + j, packed by v_cvt_scalef32_2xpk16_fp6_f32
// from u = values j = 0..15 and v = values j = 16..31 (the same packing for
// both operands, so the MFMA pairs equal k).
//   X_t: [row block of 128][group][level][row tile of 32: 0..3][tile]
//   W_t: [column block of BN][group][column tile of 32][tile]
//   Q_t: [group][row block][level][128 rows] fp32 (A_max * w_l)
//
// 32x32 result layout: lane l, element i -> MFMA row 8*(i/4) + 4*(l/32) + i%4
// (output column), MFMA column l%32 (row of x).
//
// GEMM: workgroup tile 128 rows x BN (256 or 128) columns; at BN = 256 8
// waves as 2 (rows: 64 = 2 row tiles of 32) x 4 (columns: 2 column tiles of
// 32), at BN = 128 16 waves as 4 x 4 (one 32x32 tile each).  A pipeline stage holds GPS consecutive groups (their operands are
// contiguous runs in X_t and W_t), double-buffered in LDS: the copies of
// stage s+1 (global_load_lds, no staging registers) run while stage s is
// computed, and one barrier per stage frees a buffer.  GPS groups per stage
// put GPS groups of compute between a copy and its use, which is what hides
// the copy latency when one group's compute is short (at M = 128 a group is
// about 0.2 us of work per workgroup).
#include <type_traits>

#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {
namespace p64 {
constexpr int BM = 128;
constexpr int WAVES_N = 4;                // waves along the columns
constexpr int RT = BM / 32;               // row tiles per block: 4
constexpr int TILE = 1536, TILE_LO = 1024;
constexpr int X_GROUP = 3 * RT * TILE;    // 18 KB
constexpr int Q_GROUP = 3 * BM * 4;       // 1.5 KB
constexpr int NXCD = 8;
constexpr int BAND = 4;
}  // namespace p64

typedef int v2i_ __attribute__((ext_vector_type(2)));
typedef int v6i_ __attribute__((ext_vector_type(6)));
typedef int v8i_ __attribute__((ext_vector_type(8)));
typedef float v16f_ __attribute__((ext_vector_type(16)));

namespace {
constexpr float kW1 = (float)(1.0 / (double)kF1);
constexpr float kW2 = (float)(1.0 / (double)(kF1 * kF2));
constexpr float kW3 = (float)(1.0 / (double)(kF1 * kF2 * kF2));
constexpr int kScaleX = 127;   // E8M0 2^0: levels as they are
constexpr int kScaleW = 128;   // E8M0 2^1: weights stored halved

typedef _Float16 v2h_ __attribute__((ext_vector_type(2)));
typedef _Float16 v32h_ __attribute__((ext_vector_type(32)));

// Operand slot order, the same for both operands: slot 8*i + t of lane l's
// 32 (i = 0..3, t = 0..7) holds group-relative k = 32*(l/32) + 8*i + kSlotK[t],
// the order in which weight_operand6 takes the nibbles of a tiled-weight dword.
// The MFMA pairs equal slots, so any order shared by both operands is exact.
constexpr int kSlotK[8] = {0, 2, 4, 6, 1, 3, 5, 7};

// 32 exactly representable fp16 values -> six dwords of e2m3 (value / div),
// slot e from element e.  An early-clobber destination: the instruction
// writes its result while it still reads its sources, and the builtin can be
// given a destination that overlaps them.
__device__ __forceinline__ v6i_ pack6h(const v32h_& v, float div) {
  v6i_ r;
  asm volatile("v_cvt_scalef32_pk32_fp6_f16 %0, %1, %2" : "=&v"(r) : "v"(v), "v"(div));
  return r;
}

// One weight-operand lane from its four tiled-int4 dwords (dword i: k-offsets
// 8i + j in the low nibble of byte j and 8i + 4 + j in its high nibble) -> the
// e2m3 operand of w/2.  Nibble n (4-bit two's complement) XOR 8 is u = w + 8;
// in the low mantissa bits of the fp16 number 1024 it reads 1024 + u (one
// nibble higher, 1024 + 16u), so one packed fp16 add (or fma by 1/16) per two
// values gives w exactly: 9 VALU per dword, no table.
__device__ __forceinline__ v6i_ weight_operand6(const uint32_t (&dw)[4]) {
  v32h_ h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = dw[i], hi = dw[i] >> 8;
    const v2h_ a = __builtin_bit_cast(v2h_, (lo & 0x000F000Fu) ^ 0x64086408u) - (_Float16)1032.0f;
    const v2h_ c = __builtin_bit_cast(v2h_, (hi & 0x000F000Fu) ^ 0x64086408u) - (_Float16)1032.0f;
    const v2h_ b = __builtin_elementwise_fma(__builtin_bit_cast(v2h_, (lo & 0x00F000F0u) ^ 0x64806480u),
                                             v2h_{(_Float16)0.0625f, (_Float16)0.0625f},
                                             v2h_{(_Float16)-72.0f, (_Float16)-72.0f});
    const v2h_ d = __builtin_elementwise_fma(__builtin_bit_cast(v2h_, (hi & 0x00F000F0u) ^ 0x64806480u),
                                             v2h_{(_Float16)0.0625f, (_Float16)0.0625f},
                                             v2h_{(_Float16)-72.0f, (_Float16)-72.0f});
    // k-offsets: a = (0, 2), b = (4, 6), c = (1, 3), d = (5, 7)
    h[8 * i + 0] = a[0]; h[8 * i + 1] = a[1];
    h[8 * i + 2] = b[0]; h[8 * i + 3] = b[1];
    h[8 * i + 4] = c[0]; h[8 * i + 5] = c[1];
    h[8 * i + 6] = d[0]; h[8 * i + 7] = d[1];
  }
  return pack6h(h, 2.0f);
}

__device__ __forceinline__ void store6(uint8_t* tile, int slot, const v6i_& p) {
  *reinterpret_cast<v4i*>(tile + slot * 16) = v4i{p[0], p[1], p[2], p[3]};
  *reinterpret_cast<v2i_*>(tile + p64::TILE_LO + slot * 8) = v2i_{p[4], p[5]};
}

// One operand lane (six dwords) as the MFMA's eight-dword argument; the FP6
// form reads six, the last two are left undefined.
__device__ __forceinline__ v8i_ operand6(const uint8_t* tile, int lane) {
  const v4i lo = *reinterpret_cast<const v4i*>(tile + lane * 16);
  const v2i_ hi = *reinterpret_cast<const v2i_*>(tile + p64::TILE_LO + lane * 8);
  return __builtin_shufflevector(lo, __builtin_shufflevector(hi, hi, 0, 1, -1, -1), 0, 1, 2, 3, 4, 5, -1, -1);
}
}  // namespace

// ---------------------------------------------------------------- preparation
// Waves [0, xwaves): one (row tile of 32, group) each.  Lane l takes row
// 32*tile + l%32 and the 32 elements k = 32*(l/32) + j of the group, so the
// group maximum is the maximum of lanes l and l^32; steps 1-8 (same
// arithmetic as every other kernel), then one packed operand lane per level
// and the row's level weights.
// Threads past that: lane l of (column tile of 32, 128-row block) takes
// column 32*tile + l%32 and the two tiled-int4 chunk lanes that hold its 32 k
// values of each 64-row step (k-quarters 2*(l/32) and 2*(l/32)+1), and writes
// its weight-operand lane of both groups of the block.
__global__ __launch_bounds__(256) void msd_prep64_kernel(const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ wt, int M,
                                                         int Mpad, int K, int N, int Npad,
                                                         int64_t xwaves, uint8_t* __restrict__ x_t,
                                                         float* __restrict__ q_t,
                                                         uint8_t* __restrict__ w_t, int BN) {
  using namespace p64;
  const int G = K / 64;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid < xwaves) {
    const int mt = (int)(wid / G), g = (int)(wid % G);
    const int h = lane >> 5;
    const int m = mt * 32 + (lane & 31);
    const bool real = m < M;
    const uint16_t* src = x + (real ? (int64_t)m * K + (int64_t)g * 64 + 32 * h : 0);
    uint4 xv[4];
    uint32_t mb = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      xv[c] = make_uint4(0u, 0u, 0u, 0u);
      if (real) xv[c] = *reinterpret_cast<const uint4*>(src + 8 * c);
      mb = max(mb, chunk_max_bits(xv[c]));
    }
    // steps 1-8 (msd_device.hpp): the group is lanes l and l^32
    float amax, rcp;
    msd_group_scale(max(mb, (uint32_t)__shfl_xor((int)mb, 32)), amax, rcp);
    float lv[3][32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t vw[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float u[3], rl[3];
        msd_levels(j & 1 ? vw[j >> 1] >> 16 : vw[j >> 1] & 0xffffu, amax, rcp, u, rl);
#pragma unroll
        for (int l = 0; l < 3; ++l) lv[l][8 * c + j] = rl[l];
      }
    }
    const int rb = mt / RT, rt = mt % RT;
#pragma unroll
    for (int l = 0; l < 3; ++l) {
      v32h_ hv;                                        // levels in slot order (exact in fp16)
#pragma unroll
      for (int e = 0; e < 32; ++e) hv[e] = (_Float16)lv[l][8 * (e / 8) + kSlotK[e % 8]];
      uint8_t* tile = x_t + ((((int64_t)rb * G + g) * 3 + l) * RT + rt) * TILE;
      store6(tile, lane, pack6h(hv, 1.0f));
    }
    if (h == 0) {
      float* q = q_t + (((int64_t)g * (Mpad / BM) + rb) * 3) * BM + (m % BM);
      q[0] = amax * kW1;
      q[BM] = amax * kW2;
      q[2 * BM] = amax * kW3;
    }
    return;
  }
  // weight operand lanes of both groups of a 128-row block: t = ((ct * KB) +
  // kb) * 64 + lane over Npad/32 column tiles.  The thread reads the two
  // 16-byte chunk lanes that hold its 32 k values of both 64-row steps and
  // writes one operand lane of group 2*kb (first half of each chunk lane)
  // and, if it exists, of group 2*kb + 1 (second half).
  const int KB = (K + kTileRows - 1) / kTileRows;
  const int64_t t = (wid - xwaves) * 64 + lane;
  const int64_t total = (int64_t)(Npad / 32) * KB * 64;
  if (t >= total) return;
  const int ct = (int)(t / ((int64_t)KB * 64));
  const int kb = (int)((t / 64) % KB);
  const int n = ct * 32 + (lane & 31);
  const int h = lane >> 5;
  uint4 c[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
  if (n < N) {
    const int nt = n / kTileCols;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int cl = (n % kTileCols) + 16 * (2 * h + half);       // chunk lane
      c[half] = *reinterpret_cast<const uint4*>(wt + (((int64_t)nt * KB + kb) * 64 + cl) * 16);
    }
  }
  const int CT = BN / 32;
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    const int g = 2 * kb + step;
    if (g >= G) break;                                   // K % 128 == 64: one group in the last block
    const uint32_t dw[4] = {step ? c[0].z : c[0].x, step ? c[0].w : c[0].y,
                            step ? c[1].z : c[1].x, step ? c[1].w : c[1].y};
    uint8_t* tile = w_t + (((int64_t)(ct / CT) * G + g) * CT + (ct % CT)) * TILE;
    store6(tile, lane, weight_operand6(dw));
  }
}

// ---------------------------------------------------------------- GEMM
template <int BN, int GPS, int WAVES_M, bool YINT>
__global__ __launch_bounds__(64 * WAVES_M * p64::WAVES_N, 1) void msd_gemm64_kernel(
    const uint8_t* __restrict__ x_t, const float* __restrict__ q_t,
    const uint8_t* __restrict__ w_t, const uint16_t* __restrict__ scale, int M, int Mpad, int K,
    int N, int g_begin, int g_end, int mblocks, int nblocks, uint16_t* __restrict__ y,
    int32_t* __restrict__ y_int) {
  using namespace p64;
  constexpr int WAVES = WAVES_M * WAVES_N;        // 8 or 16
  constexpr int XT = RT / WAVES_M;                // row tiles of 32 per wave: 2 or 1
  constexpr int CT = BN / 32;                     // column tiles per block: 8 or 4
  constexpr int WT = CT / WAVES_N;                // column tiles per wave: 2 or 1
  constexpr int WN = WT * 32;                     // columns per wave
  constexpr int W_GROUP = CT * TILE;              // 12 or 6 KB
  constexpr int X_KB = X_GROUP / 1024;            // 18 pieces of 1 KB
  constexpr int PIECES = GPS * (X_GROUP + W_GROUP) / 1024;
  constexpr int CPW = (PIECES + WAVES - 1) / WAVES;
  constexpr int QC = Q_GROUP / 256;               // 256-byte copies of level weights per group: 6
  constexpr int SC = BN * 2 / 256;                // of scales per group: 2 or 1
  constexpr int SMALL = GPS * (QC + (YINT ? 0 : SC));
  constexpr int SPW = (SMALL + WAVES - 1) / WAVES;
  static_assert((X_GROUP + W_GROUP) % 1024 == 0, "whole pieces");

  __shared__ __attribute__((aligned(16))) uint8_t sX[2][GPS * X_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sW[2][GPS * W_GROUP];
  __shared__ __attribute__((aligned(16))) float sQ[2][GPS * 3 * BM];
  __shared__ __attribute__((aligned(16))) uint16_t sS[2][GPS * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // tile order: as the group-128 GEMM (contiguous ranges per XCD, bands of
  // BAND row blocks, column-major within a band); speed only
  const int total = mblocks * nblocks;
  int t = blockIdx.x;
  if (total % NXCD == 0) t = (blockIdx.x % NXCD) * (total / NXCD) + blockIdx.x / NXCD;
  const int band_tiles = BAND * nblocks;
  const int band = t / band_tiles;
  const int in_band = t % band_tiles;
  const int band_rows = min(BAND, mblocks - band * BAND);
  const int rb = band * BAND + in_band % band_rows;
  const int cb = in_band / band_rows;
  const int m0 = rb * BM, n0 = cb * BN;
  const int G = K / 64;
  const int RB = Mpad / BM;

  const uint8_t* x_run = x_t + (int64_t)rb * G * X_GROUP;
  const uint8_t* w_run = w_t + (int64_t)cb * G * W_GROUP;

  // Copies of stage (groups g0 .. g0+ng-1, ng <= GPS) into buffer b.  Piece p
  // of a stage: p < ng*X_KB in the X run, then the W run; small copy s:
  // (group s / per, kind s % per) with per = QC (+ SC).
  auto dma = [&](int g0, int ng, int b) {
    const int xp = ng * X_KB;
    const int np = ng * (X_GROUP + W_GROUP) / 1024;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int p = wave * CPW + c;                         // wave-uniform
      if (p < np) {
        const uint8_t* src = p < xp ? x_run + (int64_t)g0 * X_GROUP + p * 1024
                                    : w_run + (int64_t)g0 * W_GROUP + (p - xp) * 1024;
        uint8_t* dst = p < xp ? &sX[b][p * 1024] : &sW[b][(p - xp) * 1024];
        __builtin_amdgcn_global_load_lds(src + lane * 16, dst, 16, 0, 0);
      }
    }
    constexpr int PER = QC + (YINT ? 0 : SC);
#pragma unroll
    for (int c = 0; c < SPW; ++c) {
      const int sidx = wave * SPW + c;                      // wave-uniform
      if (sidx < ng * PER) {
        const int gi = sidx / PER, kind = sidx % PER;
        const int g = g0 + gi;
        if (kind < QC) {
          const uint8_t* src = reinterpret_cast<const uint8_t*>(q_t) +
                               ((int64_t)g * RB + rb) * Q_GROUP + kind * 256 + lane * 4;
          __builtin_amdgcn_global_load_lds(src, reinterpret_cast<uint8_t*>(&sQ[b][gi * 3 * BM]) + kind * 256, 4, 0, 0);
        } else {
          const int col = min(n0 + (kind - QC) * 128 + 2 * lane, N - 2);
          const uint8_t* src = reinterpret_cast<const uint8_t*>(scale) + ((int64_t)g * N + col) * 2;
          __builtin_amdgcn_global_load_lds(src, reinterpret_cast<uint8_t*>(&sS[b][gi * BN]) + (kind - QC) * 256, 4, 0, 0);
        }
      }
    }
  };

  float yacc[XT][WT][16];
#pragma unroll
  for (int a = 0; a < XT; ++a)
#pragma unroll
    for (int c = 0; c < WT; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) yacc[a][c][i] = 0.0f;

  // Steps 9-11 for group g (index gi in its stage) from buffer b: the wave's
  // WT weight operands and XT x 3 level operands, then per output tile 3
  // MFMAs and the combine (4 VALU per output: three for the levels with the
  // row's weights, one for the column's scale and the running sum).
  auto compute = [&](int b, int gi, int g) {
    const uint8_t* sx = &sX[b][gi * X_GROUP];
    const uint8_t* sw = &sW[b][gi * W_GROUP];
    v8i_ wop[WT];
#pragma unroll
    for (int c = 0; c < WT; ++c) wop[c] = operand6(sw + (wn * WT + c) * TILE, lane);
    v8i_ xop[XT][3];
#pragma unroll
    for (int a = 0; a < XT; ++a)
#pragma unroll
      for (int l = 0; l < 3; ++l) xop[a][l] = operand6(sx + (l * RT + wm * XT + a) * TILE, lane);
    float q[XT][3];
    if constexpr (!YINT) {
#pragma unroll
      for (int a = 0; a < XT; ++a)
#pragma unroll
        for (int l = 0; l < 3; ++l) q[a][l] = sQ[b][gi * 3 * BM + l * BM + (wm * XT + a) * 32 + (lane & 31)];
    }
#pragma unroll
    for (int c = 0; c < WT; ++c) {
      uint2 sr[4];                                          // 16 scales: 4 runs of 4 columns
      if constexpr (!YINT) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sr[r] = *reinterpret_cast<const uint2*>(&sS[b][gi * BN + wn * WN + c * 32 + 8 * r + 4 * (lane >> 5)]);
      }
      // The MFMAs of AB row tiles first, then their combines: with AB = XT
      // (one column tile per wave) the second row tile's MFMAs run while the
      // first tile's results are combined; with two column tiles per wave the
      // registers allow one row tile at a time.
      constexpr int AB = WT == 1 ? XT : 1;
#pragma unroll
      for (int a0 = 0; a0 < XT; a0 += AB) {
      v16f_ d[XT][3];
#pragma unroll
      for (int a = a0; a < a0 + AB; ++a) {
#pragma unroll
        for (int l = 0; l < 3; ++l)
          d[a][l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wop[c], xop[a][l], v16f_{}, 2, 2, 0, kScaleW, 0, kScaleX);
        // An (empty) use of the operands together with the results: the
        // operands are live after the MFMAs, so no result is given registers
        // of its own A or B operand (the 16 result registers of this form are
        // written over several passes).
        // (VGPR constraints exist on the device pass only; on the host pass a
        // dependent operand would make the kernel template fail to instantiate.)
#if defined(__HIP_DEVICE_COMPILE__)
        asm volatile("" ::"v"(wop[c]), "v"(xop[a][0]), "v"(xop[a][1]), "v"(xop[a][2]), "v"(d[a][0]),
                     "v"(d[a][1]), "v"(d[a][2]));
#endif
      }
#pragma unroll
      for (int a = a0; a < a0 + AB; ++a) {
        if constexpr (YINT) {
          const int m = m0 + (wm * XT + a) * 32 + (lane & 31);
          const int64_t gi_out = g - g_begin;
          if (m < M) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int n = n0 + wn * WN + c * 32 + 8 * (i / 4) + 4 * (lane >> 5) + (i % 4);
              if (n < N) {
#pragma unroll
                for (int l = 0; l < 3; ++l)
                  y_int[((gi_out * 3 + l) * M + m) * (int64_t)N + n] = (int32_t)d[a][l][i];
              }
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t sw2 = (i % 4) < 2 ? sr[i / 4].x : sr[i / 4].y;
            const float sc = half_bits_to_float((i % 2) ? (sw2 >> 16) : (sw2 & 0xffffu));
            float tt = d[a][0][i] * q[a][0];
            tt = __builtin_fmaf(d[a][1][i], q[a][1], tt);
            tt = __builtin_fmaf(d[a][2][i], q[a][2], tt);
            yacc[a][c][i] = __builtin_fmaf(tt, sc, yacc[a][c][i]);
          }
        }
      }
      }
    }
  };

  // stages of GPS groups over [g_begin, g_end), double-buffered
  const int ngroups = g_end - g_begin;
  const int nstages = (ngroups + GPS - 1) / GPS;
  dma(g_begin, min(GPS, ngroups), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int s = 0; s < nstages; ++s) {
    const int b = s & 1;
    const int g0 = g_begin + s * GPS;
    const int ng = min(GPS, g_end - g0);
    if (s + 1 < nstages) dma(g0 + GPS, min(GPS, g_end - g0 - GPS), b ^ 1);
#pragma unroll
    for (int gi = 0; gi < GPS; ++gi)
      if (gi < ng) compute(b, gi, g0 + gi);                 // constant LDS offsets per gi
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if constexpr (!YINT) {
#pragma unroll
    for (int a = 0; a < XT; ++a) {
      const int m = m0 + (wm * XT + a) * 32 + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int c = 0; c < WT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + wn * WN + c * 32 + 8 * r + 4 * (lane >> 5);   // 4 consecutive columns
          if (n >= N) continue;
          const uint32_t lo = (uint32_t)float_to_half_bits(yacc[a][c][4 * r]) |
                              ((uint32_t)float_to_half_bits(yacc[a][c][4 * r + 1]) << 16);
          const uint32_t hi = (uint32_t)float_to_half_bits(yacc[a][c][4 * r + 2]) |
                              ((uint32_t)float_to_half_bits(yacc[a][c][4 * r + 3]) << 16);
          *reinterpret_cast<uint2*>(y + (int64_t)m * N + n) = make_uint2(lo, hi);
        }
    }
  }
}

// ---------------------------------------------------------------- GEMM, weights converted in the kernel
// With one or two row blocks (M <= 256) every weight is used by one or two
// workgroups, so converting the whole weight matrix into operand tiles ahead
// of the GEMM (read K*N/2, write 3*K*N/4 bytes, read again) costs more than
// the GEMM's own use of it.  This variant reads the tiled int4 weights itself
// and converts them to e2m3 operands one stage ahead of their use:
//   iteration s:  waves 0-7 convert the int4 block of stage s+1 (loaded into
//                 their registers during iteration s-1; wave w: column tile
//                 w % 4, group w / 4 of the stage) into the e2m3 buffer of the
//                 other parity; copies (global_load_lds) of stage s+1's x
//                 operands, level weights and scales; waves 0-7 load their
//                 part of the int4 block of stage s+2; all 16 waves compute
//                 stage s; one barrier.
// Two converter waves per SIMD, each converting one group: with one per SIMD
// converting both groups, the other three waited for that wave's extra VALU
// work at the barrier (outlier_m128 step 113.5-114.5 -> 111.9-112.4 us,
// medians of replays, four rounds alternating on one box).
// The int4 loads are the last memory operations of an iteration and stay in
// flight across its barrier (the wait before it leaves them outstanding).
// Buffers: x operands, level weights, scales and e2m3 weights double, 103 KB
// of LDS.  Workgroup tile 128 rows x 128 columns, 16 waves of one 32x32 tile
// each.
namespace p64w {
constexpr int BN = 128;
constexpr int CT = BN / 32;                 // column tiles of 32: 4
constexpr int WF_GROUP = CT * p64::TILE;    // e2m3 weight operands of a group: 6 KB
constexpr int X_STAGE = 2 * p64::X_GROUP;   // 36 KB
constexpr int XPW = 3;                      // 1 KB x pieces per wave (48 >= 36)
}  // namespace p64w

template <bool YINT>
__global__ __launch_bounds__(1024, 1) void msd_gemm64w_kernel(
    const uint8_t* __restrict__ x_t, const float* __restrict__ q_t,
    const uint8_t* __restrict__ wt, const uint16_t* __restrict__ scale, int M, int Mpad, int K,
    int N, int g_begin, int g_end, int mblocks, int nblocks, uint16_t* __restrict__ y,
    int32_t* __restrict__ y_int) {
  using namespace p64;
  using namespace p64w;
  static_assert(16 * XPW * 1024 >= X_STAGE, "x pieces");

  // One variable per buffer, named at compile time in every access (the
  // stage loop is unrolled by two), so that the compiler sees the reads of
  // one parity apart from the copies in flight into the other.
  __shared__ __attribute__((aligned(16))) uint8_t sX0[X_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sX1[X_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sWf0[2 * WF_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sWf1[2 * WF_GROUP];
  __shared__ __attribute__((aligned(16))) float sQ0[2 * 3 * BM];
  __shared__ __attribute__((aligned(16))) float sQ1[2 * 3 * BM];
  __shared__ __attribute__((aligned(16))) uint16_t sS0[2 * BN];
  __shared__ __attribute__((aligned(16))) uint16_t sS1[2 * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CT;                    // row tile of 32
  const int wn = wave % CT;                    // column tile of 32
  const bool converter = wave < 2 * CT;        // wave-uniform
  const int cst = wave / CT;                   // a converter wave's group of the stage

  // tile order: as the other GEMMs (contiguous ranges per XCD, bands of BAND
  // row blocks, column-major within a band); speed only
  const int total = mblocks * nblocks;
  int t = blockIdx.x;
  if (total % NXCD == 0) t = (blockIdx.x % NXCD) * (total / NXCD) + blockIdx.x / NXCD;
  const int band_tiles = BAND * nblocks;
  const int band = t / band_tiles;
  const int in_band = t % band_tiles;
  const int band_rows = min(BAND, mblocks - band * BAND);
  const int rb = band * BAND + in_band % band_rows;
  const int cb = in_band / band_rows;
  const int m0 = rb * BM, n0 = cb * BN;
  const int G = K / 64;
  const int RB = Mpad / BM;
  const int KB = (K + kTileRows - 1) / kTileRows;

  // stage s: 128-row block kb0 + s, groups 2(kb0 + s) and 2(kb0 + s) + 1
  const int kb0 = g_begin / 2;
  const int nst = (g_end + 1) / 2 - kb0;
  const uint8_t* x_run = x_t + (int64_t)rb * G * X_GROUP;
  const uint32_t s_off = 2u * (uint32_t)min(n0 + 2 * lane, N - 2);   // this lane's scale pair

  // Converter wave c, lane l: column 32(c % 4) + l%32 of the block, k-half
  // l/32 of group c / 4 of the stage; its int4 tile (16 columns; tiles past N
  // read a valid tile, their outputs are not stored) and the chunk lanes of
  // k-quarters 2(l/32) and 2(l/32)+1, whose 16 bytes hold the lane's 32 k of
  // both groups (dwords 2c', 2c'+1 of each: group c' = c / 4).
  const int wcol = wn * 32 + (lane & 31);
  const int wtile = min(cb * (BN / kTileCols) + wcol / kTileCols, N / kTileCols - 1);
  const uint8_t* w_lane = wt + (int64_t)wtile * KB * 1024 + ((wcol % kTileCols) + 32 * (lane >> 5)) * 16;

  // x operands, level weights and scales of the existing groups of stage s
  auto dma_x = [&](int s, uint8_t* sx, float* sq, uint16_t* ss) {
    const int g0 = 2 * (kb0 + s);
    const int ng = min(2, G - g0);
#pragma unroll
    for (int c = 0; c < XPW; ++c) {
      const int p = wave * XPW + c;                         // wave-uniform
      if (p < ng * (X_GROUP / 1024))
        __builtin_amdgcn_global_load_lds(x_run + (int64_t)g0 * X_GROUP + p * 1024 + lane * 16,
                                         sx + p * 1024, 16, 0, 0);
    }
    constexpr int PER = Q_GROUP / 256 + 1;                  // 6 level-weight copies + 1 scale copy
    if (wave < 2 * PER) {
      const int gi = wave / PER, kind = wave % PER;
      const int g = g0 + gi;
      if (gi < ng) {
        if (kind < PER - 1) {
          const uint8_t* src = reinterpret_cast<const uint8_t*>(q_t) + ((int64_t)g * RB + rb) * Q_GROUP + kind * 256;
          __builtin_amdgcn_global_load_lds(src + lane * 4, reinterpret_cast<uint8_t*>(sq + gi * 3 * BM) + kind * 256, 4, 0, 0);
        } else if (!YINT) {
          const uint8_t* row = reinterpret_cast<const uint8_t*>(scale) + (int64_t)g * N * 2;
          __builtin_amdgcn_global_load_lds(row + s_off, reinterpret_cast<uint8_t*>(ss + gi * BN), 4, 0, 0);
        }
      }
    }
  };
  // the converter wave's half of its int4 chunk lanes of stage s: dwords
  // 2cst, 2cst+1 of each
  auto load_w = [&](int s, uint2 (&wr)[2]) {
    const uint8_t* p = w_lane + (int64_t)(kb0 + s) * 1024 + 8 * cst;
    wr[0] = *reinterpret_cast<const uint2*>(p);
    wr[1] = *reinterpret_cast<const uint2*>(p + 256);
  };
  // those dwords -> the e2m3 operand lane of group cst of the stage
  auto convert = [&](const uint2 (&wr)[2], uint8_t* swf) {
    const uint32_t dw[4] = {wr[0].x, wr[0].y, wr[1].x, wr[1].y};
    store6(swf + cst * WF_GROUP + wn * TILE, lane, weight_operand6(dw));
  };

  float yacc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) yacc[i] = 0.0f;

  // Steps 9-11 for group g (index gi in its stage).  The levels are
  // multiplied and combined one after another, so that at most two 16-value
  // MFMA results are live (registers: four waves per SIMD).
  auto compute = [&](const uint8_t* sx, const uint8_t* swf, const float* sq, const uint16_t* ss, int gi,
                     int g) {
    const v8i_ wop = operand6(swf + gi * WF_GROUP + wn * TILE, lane);
    auto level = [&](int l) {
      const v8i_ xop = operand6(sx + gi * X_GROUP + (l * RT + wm) * TILE, lane);
      const v16f_ d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop, xop, v16f_{}, 2, 2, 0, kScaleW, 0,
                                                                       kScaleX);
      // operands kept live past the MFMA (its result is not given their
      // registers); their six defined dwords only, so that the undefined
      // upper two (which may share registers with the int4 loads in flight)
      // do not make the compiler wait for those loads
#if defined(__HIP_DEVICE_COMPILE__)
      asm volatile("" ::"v"(__builtin_shufflevector(wop, wop, 0, 1, 2, 3, 4, 5)),
                   "v"(__builtin_shufflevector(xop, xop, 0, 1, 2, 3, 4, 5)), "v"(d));
#endif
      return d;
    };
    if constexpr (YINT) {
      const int m = m0 + wm * 32 + (lane & 31);
      const int64_t gi_out = g - g_begin;
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        const v16f_ d = level(l);
        if (m < M) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int n = n0 + wn * 32 + 8 * (i / 4) + 4 * (lane >> 5) + (i % 4);
            if (n < N) y_int[((gi_out * 3 + l) * M + m) * (int64_t)N + n] = (int32_t)d[i];
          }
        }
      }
    } else {
      const int r0 = gi * 3 * BM + wm * 32 + (lane & 31);
      const float q0 = sq[r0], q1 = sq[r0 + BM], q2 = sq[r0 + 2 * BM];
      uint2 sr[4];                                          // 16 scales: 4 runs of 4 columns
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sr[r] = *reinterpret_cast<const uint2*>(ss + gi * BN + wn * 32 + 8 * r + 4 * (lane >> 5));
      const v16f_ d0 = level(0);
      const v16f_ d1 = level(1);
      float tt[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tt[i] = __builtin_fmaf(d1[i], q1, d0[i] * q0);
      const v16f_ d2 = level(2);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t sw2 = (i % 4) < 2 ? sr[i / 4].x : sr[i / 4].y;
        const float sc = half_bits_to_float((i % 2) ? (sw2 >> 16) : (sw2 & 0xffffu));
        yacc[i] = __builtin_fmaf(__builtin_fmaf(d2[i], q2, tt[i]), sc, yacc[i]);
      }
    }
  };

  // Iteration s from the buffers of parity B = s % 2 (see the top of this
  // kernel).  The barrier is issued without a fence (a workgroup fence would
  // wait for the int4 loads in flight); the compiler-level memory barriers
  // keep every LDS access on its side, and the explicit wait drains the LDS
  // operations and every copy except, in the converter waves, the two int4
  // loads issued last.
  uint2 wr[2];
  auto iteration = [&](auto P, int s) {
    constexpr int B = decltype(P)::value;
    uint8_t* sx = B ? sX1 : sX0;
    uint8_t* sxn = B ? sX0 : sX1;
    uint8_t* swf = B ? sWf1 : sWf0;
    uint8_t* swfn = B ? sWf0 : sWf1;
    float* sq = B ? sQ1 : sQ0;
    float* sqn = B ? sQ0 : sQ1;
    uint16_t* ss = B ? sS1 : sS0;
    uint16_t* ssn = B ? sS0 : sS1;
    if (converter && s + 1 < nst) convert(wr, swfn);
    if (s + 1 < nst) dma_x(s + 1, sxn, sqn, ssn);
    const bool w_ahead = converter && s + 2 < nst;          // wave-uniform
    if (w_ahead) load_w(s + 2, wr);
    const int g0 = 2 * (kb0 + s);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = g0 + gi;
      if (g >= g_begin && g < g_end) compute(sx, swf, sq, ss, gi, g);   // wave-uniform
    }
    // s_waitcnt immediates: vmcnt (bits 3:0) 2 or 0, expcnt (6:4) 7 = no
    // wait, lgkmcnt (11:8) 0
    if (w_ahead)
      __builtin_amdgcn_s_waitcnt(0x0072);
    else
      __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  dma_x(0, sX0, sQ0, sS0);
  if (converter) {
    load_w(0, wr);
    convert(wr, sWf0);
    if (nst > 1) load_w(1, wr);
  }
  __syncthreads();
  for (int s = 0; s < nst; s += 2) {
    iteration(std::integral_constant<int, 0>{}, s);
    if (s + 1 < nst) iteration(std::integral_constant<int, 1>{}, s + 1);
  }

  if constexpr (!YINT) {
    // y through LDS (free after the last barrier: no copy, load or
    // conversion is in flight): the workgroup's 128 x 128 tile as fp16 rows
    // of stride YS bytes, then whole 16-byte runs of 8 consecutive columns
    // (two per thread) instead of one 8-byte store per lane and 4 columns
    constexpr int YS = 272;
    static_assert(BM * YS <= X_STAGE && BN * 2 <= YS - 16, "staging fits an x buffer");
    uint8_t* st = sX0;
    const int row = wm * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = wn * 32 + 8 * r + 4 * (lane >> 5);   // 4 consecutive columns
      const uint32_t lo = (uint32_t)float_to_half_bits(yacc[4 * r]) |
                          ((uint32_t)float_to_half_bits(yacc[4 * r + 1]) << 16);
      const uint32_t hi = (uint32_t)float_to_half_bits(yacc[4 * r + 2]) |
                          ((uint32_t)float_to_half_bits(yacc[4 * r + 3]) << 16);
      *reinterpret_cast<uint2*>(st + row * YS + col * 2) = make_uint2(lo, hi);
    }
    __syncthreads();
    constexpr int RUNS = BN / 8;                        // 16-byte runs per row
#pragma unroll
    for (int j = 0; j < BM * RUNS / 1024; ++j) {
      const int run = j * 1024 + tid;
      const int rr = run / RUNS, cc = (run % RUNS) * 8;
      const int m = m0 + rr, n = n0 + cc;
      const v4i v = *reinterpret_cast<const v4i*>(st + rr * YS + cc * 2);
      if (m < M && n < N) *reinterpret_cast<v4i*>(y + (int64_t)m * N + n) = v;
    }
  }
}

// ---------------------------------------------------------------- launchers

// Up to two row blocks: weights converted in the GEMM (128-column blocks);
// more: converted once by the preparation kernel, column blocks of 256 or 128.
// The GEMM holds one workgroup per CU and a 128 x 256 tile takes about 15/8
// of a 128 x 128 one (213 against 114 us per tile at K = 8192, measured), so
// 256-column blocks when their rounds of 256 workgroups cost less by that
// count.
PrefillLayout prefill64_layout(int64_t M, int64_t K, int64_t N) {
  PrefillLayout L;
  L.mpad = (M + p64::BM - 1) / p64::BM * p64::BM;
  const int64_t mb = L.mpad / p64::BM;
  L.w_in_gemm = mb <= 2;
  const int64_t t256 = mb * ((N + 255) / 256), t128 = mb * ((N + 127) / 128);
  L.bn = (!L.w_in_gemm && ((t256 + 255) / 256) * 15 < ((t128 + 255) / 256) * 8) ? 256 : 128;
  L.npad = (N + L.bn - 1) / L.bn * L.bn;
  const int64_t G = K / 64;
  L.a_bytes = (size_t)(3 * (L.mpad / 32) * G) * p64::TILE;
  L.q_bytes = (size_t)(G * (L.mpad / p64::BM)) * p64::Q_GROUP;
  L.b_bytes = L.w_in_gemm ? 0 : (size_t)((L.npad / 32) * G) * p64::TILE;
  return L;
}

hipError_t launch_prefill64_prep(const void* x, const void* w, int64_t M, int64_t K, int64_t N,
                                 const PrefillLayout& L, uint8_t* x_t, float* q_t, uint8_t* w_t,
                                 hipStream_t stream) {
  const int64_t G = K / 64;
  const int64_t xwaves = (L.mpad / 32) * G;
  // one wave per (column tile, 128-row block), unless the GEMM converts them
  const int64_t wwaves = L.w_in_gemm ? 0 : (L.npad / 32) * tiled_kblocks(K);
  const unsigned blocks = (unsigned)((xwaves + wwaves + 3) / 4);
  hipLaunchKernelGGL(msd_prep64_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(w), (int)M,
                     (int)L.mpad, (int)K, (int)N, (int)L.npad, xwaves, x_t, q_t, w_t, (int)L.bn);
  return hipGetLastError();
}

hipError_t launch_prefill64_gemm(const uint8_t* x_t, const float* q_t, const uint8_t* w_t,
                                 const void* w_tiled, const void* scale, int64_t M, int64_t K, int64_t N,
                                 const PrefillLayout& L, int64_t g_begin, int64_t g_end, void* y,
                                 int32_t* y_int, hipStream_t stream) {
  if (L.bn != 128 && L.bn != 256) return hipErrorInvalidValue;
  const int mblocks = (int)(L.mpad / p64::BM);
  const int nblocks = (int)(L.npad / L.bn);
  const dim3 grid((unsigned)(mblocks * nblocks));
  const uint16_t* sp = static_cast<const uint16_t*>(scale);
  uint16_t* yp = static_cast<uint16_t*>(y);
  const int m = (int)M, mp = (int)L.mpad, k = (int)K, n = (int)N, gb = (int)g_begin, ge = (int)g_end;
  if (L.w_in_gemm) {
    if (L.bn != p64w::BN) return hipErrorInvalidValue;
    const uint8_t* wp = static_cast<const uint8_t*>(w_tiled);
    if (y_int)
      hipLaunchKernelGGL(msd_gemm64w_kernel<true>, grid, dim3(1024), 0, stream, x_t, q_t, wp, sp, m,
                         mp, k, n, gb, ge, mblocks, nblocks, yp, y_int);
    else
      hipLaunchKernelGGL(msd_gemm64w_kernel<false>, grid, dim3(1024), 0, stream, x_t, q_t, wp, sp, m,
                         mp, k, n, gb, ge, mblocks, nblocks, yp, y_int);
    return hipGetLastError();
  }
  // stages: 2 groups at BN = 256 (2 x 64 KB of LDS), 3 at BN = 128 (2 x 77 KB);
  // at BN = 128 a wave holds one 32x32 output tile, 16 waves per workgroup
  // (four per SIMD hide the MFMA and copy latencies of the short groups)
#define WQBMM_G64_LAUNCH(BN_, GPS_, WM_, Y_)                                                     \
  hipLaunchKernelGGL((msd_gemm64_kernel<BN_, GPS_, WM_, Y_>), grid, dim3(64 * 4 * (WM_)), 0,     \
                     stream, x_t, q_t, w_t, sp, m, mp, k, n, gb, ge, mblocks, nblocks, yp, y_int)
  if (y_int) {
    if (L.bn == 256) WQBMM_G64_LAUNCH(256, 2, 2, true); else WQBMM_G64_LAUNCH(128, 3, 4, true);
  } else {
    if (L.bn == 256) WQBMM_G64_LAUNCH(256, 2, 2, false); else WQBMM_G64_LAUNCH(128, 3, 4, false);
  }
#undef WQBMM_G64_LAUNCH
  return hipGetLastError();
}

}  // namespace wqbmm
