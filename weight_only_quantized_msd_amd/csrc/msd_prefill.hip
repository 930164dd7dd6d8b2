// msd_prefill.hip -- the MSD path for large M: an operand-preparation kernel
// and an MFMA GEMM with a fused per-group epilogue.
//
// WQBMM-Exp page (the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4
// PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145):
//   §4.1 steps 1-8   per (row, group) A_max and the three levels A1..A3
//   §4.1 step 9      Y_int = [Y1; Y2; Y3] = A_int . Weight_group, in integers
//                    (the M axis effectively tripled, cf. §8.1 singleCoreM = 3*M)
//   §4.1 step 10     Y_group = [(Y1/7.49 + Y2/(7.49*14.98) + Y3/(7.49*14.98^2)) * A_max] * scale_group
//   §4.1 step 11     Y^i = Y_group + Y^(i-1), over groups in order
//   §6.1             UnfoldA (pre-process), matmul, MergeY (post-process)
//   §6.2             PRELOAD_MSD: the next round's data movement overlaps the
//                    current round's matmul and merge
//
// The integer contraction runs on the MFMA in its FP6 form
// (v_mfma_scale_f32_16x16x128_f8f6f4 with both operands e2m3).  e2m3 (sign,
// 2 exponent bits with bias 1, 3 mantissa bits) holds every integer in
// [-7, 7] and every multiple of 1/2 in [-4, 3.5] exactly.  The levels (all in
// [-7, 7]) are stored as they are; a weight w in [-8, 7] is stored as w/2 and
// the B operand's E8M0 block scale 2^1 restores it.  Every product is exact,
// and a group's sum (|Y_l| <= 7*8*GS = 7168) is exact in the fp32
// accumulator, so the MFMA returns the integer Y_l exactly (the Y_int export
// converts it to int32).  Six bits per value is 3/4 of the bytes of fp8 (LDS
// and HBM traffic), and the FP6 form issues in about half the cycles of FP8
// or int8 at the same K.  Results in fp32 also spare the epilogue the
// int->float conversions an int8 contraction would need.
//
// Operand tiles (written by msd_prep_kernel, read by the GEMM):
//   An MFMA operand covers 16 rows (A) or 16 columns (B) x 128 k.  Lane l
//   holds row/column l%16 and 32 values in six dwords, packed by
//   v_cvt_scalef32_2xpk16_fp6_f32 from two 16-value vectors u, v (the packed
//   slots alternate u[j], v[j]); with kq = l/16 and group-relative k,
//       u[j] = value at k = 16*kq + j,   v[j] = value at k = 64 + 16*kq + j,
//   which are the two 64-row steps of tiled-weight chunk lane l, so a chunk
//   converts in place.  For GS = 64 only u is real and v is zero.  A and B
//   are packed by the same instruction from the same k assignment, so the
//   MFMA pairs equal k (whatever its own slot order).  Tiles are stored in
//   pairs (tile 2j, 2j+1; 3072 bytes): [lane][dwords 0-3 of tile 2j] (1 KB),
//   [lane][dwords 0-3 of tile 2j+1] (1 KB), [lane][dwords 4-5 of tile 2j]
//   (512 bytes), [lane][dwords 4-5 of tile 2j+1] (512 bytes).  A lane's two
//   operands are then one ds_read_b128 and one ds_read_b64 each, read into
//   registers that already form the six-dword operand (a 16-byte read of the
//   two tiles' dwords 4-5 together, which moves more bytes per cycle, needs
//   two register moves per operand pair to split it).  The pairs are the two
//   row tiles of a level that one GEMM wave holds, and two adjacent column
//   tiles.
//   A_t: [row block of 128][group][level][row tile 0..7][tile]
//   B_t: [block of 256 columns][group][column tile 0..15][tile]: a group's
//        B operands of a 256-column GEMM block are one run of 24 KB, those of
//        a 128-column block one half of it.  B_t depends on the weights
//        alone, so it is either written by the preparation kernel on each
//        call or converted once and kept (the weights' operand form); its
//        columns are padded to a multiple of 256 either way.
//   Q_t: [group][row block][128 rows] fp32: A_max * w_1 (w_1 = 1/7.49), the
//        row's step-10 weight of level 1, formed once per (row, group); the
//        GEMM weighs levels 2 and 3 by the constant ratio k = 1/14.98
//   Rows beyond M and columns beyond N hold zeros (written by the prep
//   kernel), so the operands of one group of a workgroup tile are two
//   contiguous runs: 36 KB of A and BN/16 * 1.5 KB of B.
//
// GEMM tiling: workgroup tile BM = 128 rows x BN = 256 (or 128) columns, 8
// waves as 4 (along M) x 2 (along N), wave tile 32 rows x BN/2 columns =
// 2 x NT MFMA tiles of 16x16, times 3 levels.  A wave holds its 2 x 3 level
// operands and the rows' weights for the group and walks its column tiles,
// reading the next column tile's B operand while the current one is used:
// per output tile 3 MFMAs, with the fp32 combine of the previous output tile
// interleaved (4 VALU per output and group: Y1 + k*(Y2 + k*Y3) with k =
// 1/14.98 in two, the row's A_max*w_1 in one, the scale and the running sum
// in one).  The operand reads from LDS are the
// GEMM's largest cost after the MFMA and the combine (FP6 MFMA and VALU
// issue overlap only partly on a SIMD, the less the more often the waves are
// realigned by a barrier): a wave reads 6 A + NT B tiles per group, the
// fewest for 16 x 16 output tiles per wave (64 x 64 waves read 12 + 4).
// Per group a workgroup reads 36 KB + BN/16 * 1.5 KB of operands; LDS holds
// one group's operands, weights and scales, double-buffered: the next group
// is copied global -> LDS directly (global_load_lds, no staging registers;
// each wave copies an equal share of 1 KB pieces, and the weights and
// scales in 4-byte lanes) while the current group is computed, one barrier
// per group.  The MFMA results stay in VGPRs.
// Tile order: workgroups are dealt to the 8 XCDs round-robin; the linear
// id is remapped so that each XCD gets a contiguous range of tiles, taken in
// bands of 4 row blocks (column-major within a band), so that the tiles an
// XCD runs together share 4 A runs and few B runs in its L2.  The mapping
// affects speed only.
#include <algorithm>

#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {
namespace pf {
constexpr int BM = 128;
constexpr int WAVES_M = 4;     // waves along M
constexpr int WAVES_N = 2;     // waves along N
constexpr int WAVES = WAVES_M * WAVES_N;
constexpr int THREADS = 64 * WAVES;
constexpr int WM = BM / WAVES_M;   // 32 rows per wave
constexpr int MT = WM / 16;    // 2 row tiles per wave
constexpr int RT = BM / 16;    // 8 row tiles per block
constexpr int TILE = 1536;     // bytes of one operand tile (16 x 128 k, e2m3)
constexpr int TILE_LO = 1024;  // its [lane][dwords 0-3] part
constexpr int TILE_HI = 512;   // its [lane][dwords 4-5] part
constexpr int A_GROUP = 3 * RT * TILE;   // one group of a row block: 36 KB
constexpr int Q_GROUP = BM * 4;          // level-1 weights of a row block: 512 bytes
constexpr int NXCD = 8;
constexpr int BAND = 4;        // row blocks per band of the tile order
}  // namespace pf

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Step-10 level weights for exact integer Y_l (no unpack scaling here): w_1
// per row (times A_max), and the ratio of consecutive level weights.
constexpr float kE1 = (float)(1.0 / (double)kF1);
constexpr float kK = (float)(1.0 / (double)kF2);   // 1/14.98: w_2/w_1 and w_3/w_2

// E8M0 block scales of the MFMA: 2^0 for A (levels as they are), 2^1 for B
// (weights stored halved).
constexpr int kScaleA = 127;
constexpr int kScaleB = 128;

// Signed bit field of v as a float.  The builtin's result type is unsigned, so
// it is reinterpreted as int32 before the conversion (v_cvt_f32_i32).
__device__ __forceinline__ float sfield(int32_t v, int off, int width) {
  return (float)(int32_t)__builtin_amdgcn_sbfe(v, off, width);
}

// 32 exactly representable values -> six dwords of e2m3 (value / div).
// The instruction writes its six result dwords while it still reads its two
// 16-dword sources, so the result must not overlap them: the compiler's
// builtin can be given a destination inside a source (which corrupts the
// packed values), so it is emitted here with an early-clobber destination.
__device__ __forceinline__ v6i pack_e2m3(const v16f& u, const v16f& v, float div) {
  v6i r;
  asm volatile("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(u), "v"(v), "v"(div));
  return r;
}

// ---------------------------------------------------------------- prep kernel
// Waves [0, xwaves): one (TPW 16-row tiles, group) each, steps 1-8 for its
// TPW x 16 x GS elements, one row tile after the other.  Lane l takes row
// l/4 and, with kq = l%4, the elements of operand lane 16*kq + row (u: k =
// 16*kq + j, v: k = 64 + 16*kq + j), so a group's maximum is a 4-lane
// reduction; the rows' level-1 weights A_max * w_1 go to Q_t.  Per row tile
// and level a wave stores dwords 0-3 (16 bytes per lane) and dwords 4-5 (8
// bytes per lane) into their parts of the tile pair.  A wave issues the loads
// of all its TPW row tiles before it decomposes the first.  (The launcher
// takes one row tile per wave up to 16 row blocks and a pair beyond; TPW = 4
// is built as well.)
// Waves [xwaves, xwaves + wwaves): one (pair of column tiles, pair of
// 128-row blocks) each: four 16-byte tiled-weight chunks per lane (column
// tiles up to the 256-padded width; those beyond N become zeros), all loaded
// before any is converted in place into operand lane l of its column tile,
// and each block's tile pair stored whole.  wwaves is 0 when the GEMM reads
// the weights' operand form; the one-time conversion into that form runs
// the weight waves alone (xwaves 0, x unused).
template <int GS, int TPW>
__global__ __launch_bounds__(256) void msd_prep_kernel(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ wt, int M,
                                                       int Mpad, int K, int N,
                                                       int64_t xwaves, int64_t wwaves,
                                                       uint8_t* __restrict__ a_t,
                                                       float* __restrict__ q_t,
                                                       uint8_t* __restrict__ b_t) {
  static_assert(GS == 128, "the group-128 path (group size 64 has a kernel of its own)");
  static_assert(TPW == 1 || TPW == 2 || TPW == 4, "one row tile, a pair or two pairs per wave");
  using namespace pf;
  const int G = K / GS;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid < xwaves) {
    const int tt = (int)(wid / G), g = (int)(wid % G);
    const int r = lane >> 2, kq = lane & 3;
    const int t0 = TPW * tt;                                // the wave's first row tile
    const int rb = t0 / RT;                                 // (its TPW tiles lie in one row block)
    // every tile's loads first (TPW x 64 bytes per lane in flight), then the
    // tiles one after the other
    uint4 xa[TPW][4];
    bool real[TPW];
#pragma unroll
    for (int pp = 0; pp < TPW; ++pp) {
      const int m = (t0 + pp) * 16 + r;
      real[pp] = m < M;                                     // padding rows decompose zeros
      const uint16_t* src = x + (real[pp] ? (int64_t)m * K + (int64_t)g * GS + 16 * kq : 0);
#pragma unroll
      for (int c = 0; c < 4; ++c)   // c = 0, 1: u (k = 16kq + 8c ..); c = 2, 3: v (k = 64 + 16kq + 8(c-2) ..)
        xa[pp][c] = *reinterpret_cast<const uint4*>(src + (c < 2 ? 8 * c : 64 + 8 * (c - 2)));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pp = 0; pp < TPW; ++pp) {
      const int p = (t0 + pp) & 1;                         // position within the pair
      const int rt0 = ((t0 + pp) & ~1) % RT;               // the pair's first row tile
      const int m = (t0 + pp) * 16 + r;
      uint4 xv[4];
      uint32_t mb = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        xv[c] = real[pp] ? xa[pp][c] : make_uint4(0u, 0u, 0u, 0u);
        mb = max(mb, chunk_max_bits(xv[c]));
      }
      // steps 1-8 (msd_device.hpp): the group is the 4 lanes of this row
      float amax, rcp;
      msd_group_scale(group_max_bits<4>(mb), amax, rcp);
      v16f lv[3][2];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t vw[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = 8 * c + j;
          float u[3], rl[3];
          msd_levels(j & 1 ? vw[j >> 1] >> 16 : vw[j >> 1] & 0xffffu, amax, rcp, u, rl);
#pragma unroll
          for (int l = 0; l < 3; ++l) lv[l][e / 16][e % 16] = rl[l];
        }
      }
      // this row tile's dwords 0-3 and 4-5 in their parts of the pair
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        uint8_t* pair = a_t + ((((int64_t)rb * G + g) * 3 + l) * RT + rt0) * TILE;
        const v6i pk = pack_e2m3(lv[l][0], lv[l][1], 1.0f);
        const int slot = 16 * kq + r;
        *reinterpret_cast<v4i*>(pair + p * TILE_LO + slot * 16) = v4i{pk[0], pk[1], pk[2], pk[3]};
        *reinterpret_cast<v2i*>(pair + 2 * TILE_LO + p * TILE_HI + slot * 8) = v2i{pk[4], pk[5]};
      }
      if (kq == 0)                                   // the row's level-1 weight
        q_t[((int64_t)g * (Mpad / BM) + rb) * BM + (m % BM)] = amax * kE1;
    }
    return;
  }
  // tiled weights: a wave converts the chunks of two adjacent column tiles
  // for two consecutive 128-row blocks (chunk t = (nt * KB + kb) * 64 + lane),
  // all four loads issued first, and stores each block's tile pair whole
  const int KB = (K + kTileRows - 1) / kTileRows;
  const int KBP = (KB + 1) / 2;
  const int64_t u = wid - xwaves;
  if (u >= wwaves) return;     // wwaves: (column tile pairs up to the 256-padded width) x KBP
  const int ctp = (int)(u / KBP), kbp = (int)(u % KBP);
  const int NTR = N / kTileCols;                     // real column tiles
  uint4 v[2][2];                                      // [block of the pair][column tile of the pair]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int nt = 2 * ctp + h, kb = 2 * kbp + i;
      const bool ok = nt < NTR && kb < KB;
      v[i][h] = *reinterpret_cast<const uint4*>(wt + (ok ? ((int64_t)nt * KB + kb) * 64 + lane : 0) * 16);
    }
  __builtin_amdgcn_sched_barrier(0);                 // every load ahead of the first conversion
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kb = 2 * kbp + i;
    if (kb >= KB) break;                              // wave-uniform
    v6i pk[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool real = 2 * ctp + h < NTR;            // columns beyond N become zeros
      const int32_t dw[4] = {real ? (int32_t)v[i][h].x : 0, real ? (int32_t)v[i][h].y : 0,
                             real ? (int32_t)v[i][h].z : 0, real ? (int32_t)v[i][h].w : 0};
      // step s (dwords 2s, 2s+1), element i = 8d + j: dword 2s + d, low nibble of
      // byte j for j < 4, high nibble of byte j - 4 otherwise
      v16f w[2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = e % 8;
          w[st][e] = sfield(dw[2 * st + e / 8], j < 4 ? 8 * j : 8 * (j - 4) + 4, 4);
        }
      pk[h] = pack_e2m3(w[0], w[1], 2.0f);
    }
    uint8_t* pair = b_t + (((int64_t)(ctp / 8) * KB + kb) * 8 + ctp % 8) * (2 * TILE);
    *reinterpret_cast<v4i*>(pair + lane * 16) = v4i{pk[0][0], pk[0][1], pk[0][2], pk[0][3]};
    *reinterpret_cast<v4i*>(pair + TILE_LO + lane * 16) = v4i{pk[1][0], pk[1][1], pk[1][2], pk[1][3]};
    *reinterpret_cast<v2i*>(pair + 2 * TILE_LO + lane * 8) = v2i{pk[0][4], pk[0][5]};
    *reinterpret_cast<v2i*>(pair + 2 * TILE_LO + TILE_HI + lane * 8) = v2i{pk[1][4], pk[1][5]};
  }
}

// ---------------------------------------------------------------- GEMM kernel
// The two operands (six dwords each) of lane `lane` from an LDS tile pair
// (address of its first tile), as the MFMA's eight-dword arguments (the last
// two are unused by the FP6 form): per operand one ds_read_b128 and one
// ds_read_b64.
// The 8-byte reads are volatile: the compiler would otherwise merge two of
// them (of this pair or of two pairs) into one read of four registers and
// then move two of those into place.
__device__ __forceinline__ void lds_operand_pair(const uint8_t* pair, int lane, v8i& op0, v8i& op1) {
  const v4i lo0 = *reinterpret_cast<const v4i*>(pair + lane * 16);
  const v4i lo1 = *reinterpret_cast<const v4i*>(pair + pf::TILE_LO + lane * 16);
  typedef const volatile __attribute__((address_space(3))) v2i lds_v2i;
  typedef const __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* lp = (lds_u8*)pair;
  const v2i hi0 = *(lds_v2i*)(lp + 2 * pf::TILE_LO + lane * 8);
  const v2i hi1 = *(lds_v2i*)(lp + 2 * pf::TILE_LO + pf::TILE_HI + lane * 8);
  op0 = v8i{lo0[0], lo0[1], lo0[2], lo0[3], hi0[0], hi0[1], 0, 0};
  op1 = v8i{lo1[0], lo1[1], lo1[2], lo1[3], hi1[0], hi1[1], 0, 0};
}

template <int GS, int BN, bool YINT>
__global__ __launch_bounds__(pf::THREADS, 1) void msd_gemm_kernel(
    const uint8_t* __restrict__ a_t, const float* __restrict__ q_t,
    const uint8_t* __restrict__ b_t, const uint16_t* __restrict__ scale, int M, int Mpad, int K,
    int N, int g_begin, int g_end, int mblocks, int nblocks, int splits, int gps,
    uint16_t* __restrict__ y, int32_t* __restrict__ y_int, float* __restrict__ part) {
  using namespace pf;
  constexpr int CT = BN / 16;                          // column tiles per block
  constexpr int NT = CT / WAVES_N;                     // column tiles per wave: 8, 4 or 2
  constexpr int WN = NT * 16;                          // columns per wave
  constexpr int B_GROUP = CT * TILE;                   // one group of a column block
  constexpr int A_KB = A_GROUP / 1024;                 // 36 pieces of 1 KB
  constexpr int PIECES = A_KB + B_GROUP / 1024;        // 60, 48 or 42
  constexpr int CPW = (PIECES + WAVES - 1) / WAVES;    // pieces per wave: 8 or 6
  constexpr int QW = Q_GROUP / 256;                    // 256-byte copies of the level-1 weights: 2
  constexpr int SW = (BN * 2 + 255) / 256;             // 256-byte copies of the scales: 2 or 1
  constexpr int SN = SW * 128;                         // scales copied per group (>= BN)
  static_assert(QW + SW <= WAVES, "one small copy per wave");
  static_assert(B_GROUP % 1024 == 0, "whole pieces");

  // Named buffers (not one array indexed by the group) so that the copies
  // into one and the reads of another are visibly disjoint.  128-column
  // blocks have three (149 KB of LDS: the copies run two groups ahead),
  // 256- and 64-column blocks two (a third would not fit at 256).
  constexpr int NBUF = BN == 128 ? 3 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t sA0[A_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[A_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sA2[NBUF == 3 ? A_GROUP : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[B_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[B_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sB2[NBUF == 3 ? B_GROUP : 16];
  __shared__ __attribute__((aligned(16))) float sQ0[BM];
  __shared__ __attribute__((aligned(16))) float sQ1[BM];
  __shared__ __attribute__((aligned(16))) float sQ2[NBUF == 3 ? BM : 4];
  __shared__ __attribute__((aligned(16))) uint16_t sS0[SN];
  __shared__ __attribute__((aligned(16))) uint16_t sS1[SN];
  __shared__ __attribute__((aligned(16))) uint16_t sS2[NBUF == 3 ? SN : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;   // rows WM*wm of the tile
  const int wn = wave % WAVES_N;   // columns WN*wn of the tile

  // Tile order: XCD x (= id % 8) runs the contiguous range of tiles
  // [x * total/8, (x+1) * total/8); tiles are numbered in bands of BAND row
  // blocks, column-major within a band.
  const int tiles = mblocks * nblocks;
  const int total = tiles * splits;
  int t = blockIdx.x;
  if (total % NXCD == 0) t = (blockIdx.x % NXCD) * (total / NXCD) + blockIdx.x / NXCD;
  // K-split (few tiles): split sp takes groups [g_lo, g_hi) of the range and,
  // unless Y_int is exported, leaves an fp32 partial sum for the reduction
  const int sp = t / tiles;
  t %= tiles;
  const int g_lo = g_begin + sp * gps;
  const int g_hi = min(g_end, g_lo + gps);
  const int band_tiles = BAND * nblocks;
  const int band = t / band_tiles;
  const int in_band = t % band_tiles;
  const int band_rows = min(BAND, mblocks - band * BAND);
  const int rb = band * BAND + in_band % band_rows;
  const int cb = in_band / band_rows;
  const int m0 = rb * BM;
  const int n0 = cb * BN;
  const int G = K / GS;
  const int RB = Mpad / BM;

  // Group g_'s operands -> LDS by DMA (global_load_lds, 16 bytes per lane:
  // lane i's bytes land at the destination + 16*i, so a 1 KB piece keeps its
  // layout).  Pieces [0, 36) are the block's A run, the rest its B run.  The
  // level-1 weights (fp32) and the scales (fp16 pairs) go 4 bytes per lane, one
  // 256-byte copy per wave.  (The 4-byte copies take byte pointers: typed
  // float pointers made the compiler crash in its SGPR-copy pass.)
  const uint8_t* a_run = a_t + (int64_t)rb * G * A_GROUP;
  // the block's B run of group 0 (groups 24 KB apart: 16 column tiles)
  constexpr int B_STRIDE = 16 * TILE;
  const uint8_t* b_run = b_t + (int64_t)(cb * BN / 256) * G * B_STRIDE + (cb * BN % 256) / 16 * TILE;
  const int sc_col = min(n0 + 2 * (wave - QW) * 64 + 2 * lane, N - 2);
  auto dma = [&](int g_, uint8_t* sa, uint8_t* sb, float* sq, uint16_t* ss) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int p = wave * CPW + c;                   // wave-uniform
      if (p < PIECES) {
        const uint8_t* src = p < A_KB ? a_run + (int64_t)g_ * A_GROUP + p * 1024
                                      : b_run + (int64_t)g_ * B_STRIDE + (p - A_KB) * 1024;
        uint8_t* dst = p < A_KB ? sa + p * 1024 : sb + (p - A_KB) * 1024;
        __builtin_amdgcn_global_load_lds(src + lane * 16, dst, 16, 0, 0);
      }
    }
    if (wave < QW) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(q_t) +
                           ((int64_t)g_ * RB + rb) * Q_GROUP + wave * 256 + lane * 4;
      __builtin_amdgcn_global_load_lds(src, reinterpret_cast<uint8_t*>(sq) + wave * 256, 4, 0, 0);
    } else if (wave < QW + SW && !YINT) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(scale) + ((int64_t)g_ * N + sc_col) * 2;
      __builtin_amdgcn_global_load_lds(src, reinterpret_cast<uint8_t*>(ss) + (wave - QW) * 256, 4, 0, 0);
    }
  };

  float yacc[MT][NT][4];
#pragma unroll
  for (int r = 0; r < MT; ++r)
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) yacc[r][c][i] = 0.0f;

  // Steps 10-11 for output tile (row tile PR, column tile PC) from its three
  // level results; or the Y_int export.  The level sums are folded as
  // Y1 + k*(Y2 + k*Y3) with k = 1/14.98 (= w_2/w_1 = w_3/w_2), then multiplied
  // by the row's A_max*w_1 and the column's scale and added to the running
  // sum: 4 VALU per output and group, with one level weight per row held.
  auto epilogue = [&](int pr, int pc, const v4f (&a3)[3], const v4f& q1, const uint32_t (&sraw)[NT], int g_) {
    if constexpr (YINT) {
      const int64_t gi = g_ - g_begin;
      const int n = n0 + wn * WN + pc * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * WM + pr * 16 + (lane >> 4) * 4 + i;
        if (m < M && n < N) {
#pragma unroll
          for (int l = 0; l < 3; ++l)
            y_int[((gi * 3 + l) * M + m) * (int64_t)N + n] = (int32_t)a3[l][i];
        }
      }
    } else {
      const float sc = half_bits_to_float(sraw[pc]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float tt = __builtin_fmaf(a3[2][i], kK, a3[1][i]);
        tt = __builtin_fmaf(tt, kK, a3[0][i]);
        tt = tt * q1[i];
        yacc[pr][pc][i] = __builtin_fmaf(tt, sc, yacc[pr][pc][i]);
      }
    }
  };

  // Steps 9-11 for one group from one buffer.  The wave reads its first pair
  // of B operands and its 2 x 3 level operands (one pair per level), then
  // walks its column tiles with the next pair of B operands read ahead (two
  // pairs of B registers in turn): per output tile 3 MFMAs, then the combine
  // of the output tile D before it (so the combine never waits for the MFMAs
  // it follows).  A register that a load overwrites was last read by MFMAs
  // issued before that load.  (Issuing one MFMA, then a few VALU, in turn,
  // through scheduling-group barriers, was slower: 80 -> 84-90 us at
  // prefill_m2048, the combines then waiting on MFMA results.)
  static_assert(MT == 2 && NT % 2 == 0, "operand tiles are read in pairs");
  auto compute = [&](const uint8_t* sa, const uint8_t* sb, const float* sq, const uint16_t* ss, int g_) {
    v8i bf[2][2];
    lds_operand_pair(sb + (wn * NT) * TILE, lane, bf[0][0], bf[0][1]);
    v8i af[MT][3];
#pragma unroll
    for (int l = 0; l < 3; ++l) lds_operand_pair(sa + (l * RT + wm * MT) * TILE, lane, af[0][l], af[1][l]);
    uint32_t sraw[NT];
    v4f q[MT];                   // the row tiles' level-1 weights A_max * w_1
    if constexpr (!YINT) {
#pragma unroll
      for (int c = 0; c < NT; ++c) sraw[c] = ss[wn * WN + c * 16 + (lane & 15)];
#pragma unroll
      for (int r = 0; r < MT; ++r)
        q[r] = *reinterpret_cast<const v4f*>(sq + (wm * MT + r) * 16 + 4 * (lane >> 4));
    }
    // output tiles between an MFMA and its combine: two at 256-column blocks
    // (the combine then reads results six MFMAs old; prefill_m2048 step
    // 79.7-80.9 -> 78.2-78.4 us on one box), one otherwise (mixed at 128)
    constexpr int D = BN == 256 ? 2 : 1;
    v4f acc[D + 1][3];           // MFMA results of the current and the D previous output tiles
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int cp = c / 2;
      if (c % 2 == 0 && cp + 1 < NT / 2)
        lds_operand_pair(sb + (wn * NT + c + 2) * TILE, lane, bf[(cp + 1) & 1][0], bf[(cp + 1) & 1][1]);
#pragma unroll
      for (int r = 0; r < MT; ++r) {
        const int j = c * MT + r, cur = j % (D + 1);
#pragma unroll
        for (int l = 0; l < 3; ++l)
          acc[cur][l] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[r][l], bf[cp & 1][c & 1], v4f{0.f, 0.f, 0.f, 0.f}, 2, 2, 0, kScaleA, 0, kScaleB);
        if (j >= D) {
          const int pj = j - D, pc = pj / MT, pr = pj % MT;
          epilogue(pr, pc, acc[pj % (D + 1)], q[pr], sraw, g_);
        }
      }
    }
#pragma unroll
    for (int pj = MT * NT - D; pj < MT * NT; ++pj)
      epilogue(pj % MT, pj / MT, acc[pj % (D + 1)], q[pj % MT], sraw, g_);
  };

  if constexpr (NBUF == 2) {
    // Buffer 0 holds the even-indexed groups of the range, buffer 1 the odd
    // ones.  While a group is computed from one buffer, the next group is
    // copied into the other; each wave waits for its own copies, and the
    // barrier then publishes all of them and frees the buffer just read.
    // At 64-column blocks a scheduling barrier keeps the wait after the whole
    // group's compute: the compiler otherwise hoists it above the last third
    // of the group's MFMAs (they touch no memory), and the wave waits on its
    // copies early (M = 96 and 128 at K = N = 4096: GEMM 17.6 -> 16.6 and
    // 18.5 -> 17.6 us).  At 256-column blocks the hoisted form is faster
    // (prefill_m2048 GEMM 73.2 against 73.4 us, M = 1536 67.6 against 68.9):
    // there the MFMAs left after the barrier overlap the next group's
    // operand reads.
    dma(g_lo, sA0, sB0, sQ0, sS0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int g = g_lo; g < g_hi; g += 2) {
      if (g + 1 < g_hi) dma(g + 1, sA1, sB1, sQ1, sS1);
      compute(sA0, sB0, sQ0, sS0, g);
      if constexpr (BN == 64) __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (g + 1 >= g_hi) break;
      if (g + 2 < g_hi) dma(g + 2, sA0, sB0, sQ0, sS0);
      compute(sA1, sB1, sQ1, sS1, g + 1);
      if constexpr (BN == 64) __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    // Group i of the range in buffer i % 3.  The step that computes group g
    // first issues the copies of group g+2 (into the buffer group g-1 used,
    // which every wave finished reading before the last barrier), then waits
    // for its own copies of group g+1 only: a wave issues CPW pieces plus, in
    // waves 0..QW+SW-1 (QW with Y_int), one small copy per group, and vector
    // memory operations complete in order, so vmcnt(that count) leaves
    // exactly group g+2's copies in flight.  The barrier is issued without a
    // fence (a workgroup fence would wait for those copies too); the
    // compiler-level memory barriers keep every LDS access on its side.
    static_assert(PIECES == CPW * WAVES, "every wave issues CPW pieces");
    const int ahead = CPW + (wave < QW + (YINT ? 0 : SW) ? 1 : 0);   // wave-uniform
    auto end_step = [&](bool copies_ahead) {
      // s_waitcnt immediates: vmcnt (bits 3:0) 7, 6 or 0, expcnt (6:4) 7 =
      // no wait, lgkmcnt (11:8) 0
      static_assert(CPW + 1 <= 15, "vmcnt immediate");
      if (copies_ahead) {
        if (ahead == CPW + 1) __builtin_amdgcn_s_waitcnt(0x0070 | (CPW + 1));
        else __builtin_amdgcn_s_waitcnt(0x0070 | CPW);
      } else {
        __builtin_amdgcn_s_waitcnt(0x0070);
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    dma(g_lo, sA0, sB0, sQ0, sS0);
    asm volatile("" ::: "memory");
    if (g_lo + 1 < g_hi) dma(g_lo + 1, sA1, sB1, sQ1, sS1);
    end_step(g_lo + 1 < g_hi);
    for (int g = g_lo; g < g_hi; g += 3) {
      if (g + 2 < g_hi) dma(g + 2, sA2, sB2, sQ2, sS2);
      compute(sA0, sB0, sQ0, sS0, g);
      end_step(g + 2 < g_hi);
      if (g + 1 >= g_hi) break;
      if (g + 3 < g_hi) dma(g + 3, sA0, sB0, sQ0, sS0);
      compute(sA1, sB1, sQ1, sS1, g + 1);
      end_step(g + 3 < g_hi);
      if (g + 2 >= g_hi) break;
      if (g + 4 < g_hi) dma(g + 4, sA1, sB1, sQ1, sS1);
      compute(sA2, sB2, sQ2, sS2, g + 2);
      end_step(g + 4 < g_hi);
    }
  }

  if constexpr (!YINT) {
    // y (or a split's fp32 partial sum) through LDS (the operand buffers are
    // free: every wave passed the barrier after its last group and no copy
    // is in flight): each wave writes its 32 x WN tile in rows of stride YS
    // bytes (68 dwords: the four row groups of an MFMA result land on
    // distinct banks), then stores whole 16-byte runs of consecutive
    // columns instead of one 2- or 4-byte store per output.
    constexpr int YS = 272;
    static_assert(4 * WM * YS <= A_GROUP && WN * 2 <= YS - 16, "staging fits the A buffers");
    uint8_t* st = (wave < 4 ? sA0 : sA1) + (wave % 4) * (WM * YS);
    if (splits > 1) {
      if constexpr (BN <= 128) {                         // a split GEMM has 128- or 64-column blocks
        static_assert(WN * 4 <= YS - 16, "fp32 rows fit the stride");
#pragma unroll
        for (int r = 0; r < MT; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = r * 16 + (lane >> 4) * 4 + i;
#pragma unroll
            for (int c = 0; c < NT; ++c)
              *reinterpret_cast<float*>(st + row * YS + (c * 16 + (lane & 15)) * 4) = yacc[r][c][i];
          }
        __syncthreads();
        constexpr int RUNS = WN / 4;                     // 16-byte runs of 4 floats per row
#pragma unroll
        for (int j = 0; j < WM * RUNS / 64; ++j) {
          const int run = j * 64 + lane;
          const int row = run / RUNS, col = (run % RUNS) * 4;
          const int m = m0 + wm * WM + row, n = n0 + wn * WN + col;
          const v4i v = *reinterpret_cast<const v4i*>(st + row * YS + col * 4);
          if (m < M && n < N) *reinterpret_cast<v4i*>(part + ((int64_t)sp * M + m) * N + n) = v;
        }
      }
      return;
    }
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r * 16 + (lane >> 4) * 4 + i;
#pragma unroll
        for (int c = 0; c < NT; ++c)
          *reinterpret_cast<uint16_t*>(st + row * YS + (c * 16 + (lane & 15)) * 2) =
              float_to_half_bits(yacc[r][c][i]);
      }
    __syncthreads();
    constexpr int RUNS = WN / 8;                         // 16-byte runs per row
#pragma unroll
    for (int j = 0; j < WM * RUNS / 64; ++j) {
      const int run = j * 64 + lane;
      const int row = run / RUNS, col = (run % RUNS) * 8;
      const int m = m0 + wm * WM + row, n = n0 + wn * WN + col;
      const v4i v = *reinterpret_cast<const v4i*>(st + row * YS + col * 2);
      if (m < M && n < N) *reinterpret_cast<v4i*>(y + (int64_t)m * N + n) = v;
    }
  }
}

// ------------------------------------------------------- split-K reduction
// y[m][n] = fp16_rne(sum over splits s = 0, 1, .. of part[s][m][n]), the
// splits added in ascending order (each split holds its groups' sum, groups
// ascending), so the result is the same on every run.  Four consecutive
// outputs per thread (N % 4 == 0).
__global__ __launch_bounds__(256) void msd_splitk_reduce_kernel(const float* __restrict__ part,
                                                                int splits, int64_t MN,
                                                                uint16_t* __restrict__ y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int s = 1; s < splits; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(part + (int64_t)s * MN + i);
    acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
  }
  const uint32_t lo = (uint32_t)float_to_half_bits(acc.x) | ((uint32_t)float_to_half_bits(acc.y) << 16);
  const uint32_t hi = (uint32_t)float_to_half_bits(acc.z) | ((uint32_t)float_to_half_bits(acc.w) << 16);
  *reinterpret_cast<uint2*>(y + i) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------- launchers

// K-split of the GEMM when its tiles alone would leave CUs idle: enough
// splits to bring the workgroups to about one per CU (the GEMM holds one
// workgroup per CU), each split at least two groups long.  The splits' fp32
// partial sums [splits][M][N] follow the operand tiles in the workspace.
void set_splits(PrefillLayout& L, int64_t tiles, int64_t G, int64_t M, int64_t N) {
  int64_t s = tiles >= 256 ? 1 : 256 / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, G / 2));
  const int64_t gps = (G + s - 1) / s;
  L.splits = (G + gps - 1) / gps;
  L.part_bytes = L.splits > 1 ? (size_t)L.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// Column blocks of 256, 128 or 64.  The GEMM holds one workgroup per CU, so its
// time is about (rounds of 256 workgroups) x (one workgroup's time), and a
// 128 x 256 tile takes about 7/4 of a 128 x 128 one (72 against 41 us per
// tile at K = 4096, measured).  256-column blocks when their rounds cost less
// (M = 1280 or 1536 at N = 4096: one round of 256-column tiles against two of
// 128-column ones); with fewer than 256 tiles of 128 columns, 128 and a K-split.
PrefillLayout prefill_layout(int gs, int64_t M, int64_t K, int64_t N) {
  if (gs == 64) return prefill64_layout(M, K, N);
  PrefillLayout L;
  L.mpad = (M + pf::BM - 1) / pf::BM * pf::BM;
  const int64_t mb = L.mpad / pf::BM;
  const int64_t t256 = mb * ((N + 255) / 256), t128 = mb * ((N + 127) / 128);
  L.bn = (t128 >= 256 && ((t256 + 255) / 256) * 7 < ((t128 + 255) / 256) * 4) ? 256 : 128;
  // At most 32 tiles of 128 columns (eight or more K-splits at K = 4096):
  // 64-column blocks halve the splits for the same workgroups, and with them
  // the fp32 partial sums (M = 128, K = N = 4096: 24.4 -> 22.4 us; with 64 or
  // more tiles of 128 they were slower: M = 256, 29.2 against 28.5 us).
  if (t128 <= 32) L.bn = 64;
  L.npad = (N + L.bn - 1) / L.bn * L.bn;
  const int64_t G = K / gs;
  L.a_bytes = (size_t)(3 * (L.mpad / 16) * G) * pf::TILE;
  L.q_bytes = (size_t)(G * (L.mpad / pf::BM)) * pf::Q_GROUP;
  L.b_bytes = (size_t)(operand_weight_npad(N) / 16 * G) * pf::TILE;   // 256-column blocks
  L.w_in_gemm = false;
  set_splits(L, (L.mpad / pf::BM) * (L.npad / L.bn), G, M, N);
  return L;
}

hipError_t launch_prefill_prep(const void* x, const void* w, int gs, int64_t M, int64_t K,
                               int64_t N, const PrefillLayout& L, uint8_t* a_t, float* q_t,
                               uint8_t* b_t, bool weights, hipStream_t stream) {
  if (gs == 64) return launch_prefill64_prep(x, w, M, K, N, L, a_t, q_t, b_t, stream);
  // up to 16 row blocks: one row tile per x wave (twice the waves, each half
  // as long); beyond, a tile pair per wave (measured: one tile per wave is
  // faster up to M = 2048, 9.3 -> 8.9 us there, slower at 4096)
  const int tpw = L.mpad <= 16 * pf::BM ? 1 : 2;
  const int64_t xwaves = (L.mpad / (16 * tpw)) * (K / gs);          // (row tile(s), group) tasks
  const int64_t npw = operand_weight_npad(N);                      // B_t's 256-column blocks
  const int64_t wwaves =                                            // (column tile pair, block pair)
      weights ? (npw / 32) * ((tiled_kblocks(K) + 1) / 2) : 0;
  const unsigned blocks = (unsigned)((xwaves + wwaves + 3) / 4);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const int m = (int)M, mp = (int)L.mpad, k = (int)K, n = (int)N;
  if (tpw == 1)
    hipLaunchKernelGGL((msd_prep_kernel<128, 1>), dim3(blocks), dim3(256), 0, stream, xp, wp, m, mp,
                       k, n, xwaves, wwaves, a_t, q_t, b_t);
  else if (tpw == 2)
    hipLaunchKernelGGL((msd_prep_kernel<128, 2>), dim3(blocks), dim3(256), 0, stream, xp, wp, m, mp,
                       k, n, xwaves, wwaves, a_t, q_t, b_t);
  else
    hipLaunchKernelGGL((msd_prep_kernel<128, 4>), dim3(blocks), dim3(256), 0, stream, xp, wp, m, mp,
                       k, n, xwaves, wwaves, a_t, q_t, b_t);
  return hipGetLastError();
}

size_t operand_weight_bytes(int64_t K, int64_t N) {
  return (size_t)(operand_weight_npad(N) / 16) * (size_t)tiled_kblocks(K) * pf::TILE;
}

// The weights' part of the preparation kernel alone.
hipError_t launch_operand_weights(const void* w_tiled, int64_t K, int64_t N, uint8_t* w_op,
                                  hipStream_t stream) {
  const int64_t npad = operand_weight_npad(N);
  const int64_t wwaves = (npad / 32) * ((tiled_kblocks(K) + 1) / 2);
  const unsigned blocks = (unsigned)((wwaves + 3) / 4);
  hipLaunchKernelGGL((msd_prep_kernel<128, 2>), dim3(blocks), dim3(256), 0, stream, nullptr,
                     static_cast<const uint8_t*>(w_tiled), 0, 0, (int)K, (int)N,
                     (int64_t)0, wwaves, nullptr, nullptr, w_op);
  return hipGetLastError();
}

hipError_t launch_prefill_gemm(const uint8_t* a_t, const float* q_t, const uint8_t* b_t,
                               const void* w_tiled, const void* scale, int gs, int64_t M, int64_t K, int64_t N,
                               const PrefillLayout& L, int64_t g_begin, int64_t g_end, void* y,
                               int32_t* y_int, float* part, hipStream_t stream) {
  if (gs == 64)
    return launch_prefill64_gemm(a_t, q_t, b_t, w_tiled, scale, M, K, N, L, g_begin, g_end, y, y_int,
                                 stream);
  if (L.bn != 64 && L.bn != 128 && L.bn != 256) return hipErrorInvalidValue;
  const int mblocks = (int)(L.mpad / pf::BM);
  const int nblocks = (int)(L.npad / L.bn);
  // the layout's split count over this group range (a Y_int export needs no
  // partial sums: each split stores its own groups)
  const int64_t range = g_end - g_begin;
  int64_t splits = std::min<int64_t>(L.splits, range);
  const int64_t gps = (range + splits - 1) / splits;
  splits = (range + gps - 1) / gps;
  // (a split GEMM stages its fp32 partial sums for 128- and 64-column blocks;
  // the layout splits only below 256 tiles, where the blocks are that wide)
  if (splits > 1 && !y_int && (!part || splits > L.splits || L.bn > 128)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(mblocks * nblocks * splits));
  const uint16_t* sp = static_cast<const uint16_t*>(scale);
  uint16_t* yp = static_cast<uint16_t*>(y);
  const int m = (int)M, mp = (int)L.mpad, k = (int)K, n = (int)N, gb = (int)g_begin, ge = (int)g_end;
  const int S = (int)splits, GPS = (int)gps;
#define WQBMM_GEMM_LAUNCH(GS_, BN_, Y_)                                                          \
  hipLaunchKernelGGL((msd_gemm_kernel<GS_, BN_, Y_>), grid, dim3(pf::THREADS), 0, stream, a_t,  \
                     q_t, b_t, sp, m, mp, k, n, gb, ge, mblocks, nblocks, S, GPS, yp, y_int, part)
#define WQBMM_GEMM_BN(GS_, Y_)                                                                   \
  do {                                                                                           \
    if (L.bn == 256) WQBMM_GEMM_LAUNCH(GS_, 256, Y_);                                           \
    else if (L.bn == 128) WQBMM_GEMM_LAUNCH(GS_, 128, Y_);                                      \
    else WQBMM_GEMM_LAUNCH(GS_, 64, Y_);                                                        \
  } while (0)
  if (y_int) WQBMM_GEMM_BN(128, true); else WQBMM_GEMM_BN(128, false);
#undef WQBMM_GEMM_BN
#undef WQBMM_GEMM_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || y_int || S == 1) return e;
  const int64_t MN = M * N;
  hipLaunchKernelGGL(msd_splitk_reduce_kernel, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, stream,
                     part, S, MN, yp);
  return hipGetLastError();
}

}  // namespace wqbmm
