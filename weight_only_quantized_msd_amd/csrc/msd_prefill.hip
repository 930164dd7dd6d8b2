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
//   MFMA pairs equal k (whatever its own slot order).  A tile is stored as
//   [lane][dwords 0-3] (1 KB) then [lane][dwords 4-5] (512 bytes), 1536
//   bytes, read by one conflict-free ds_read_b128 and one ds_read_b64.
//   A_t: [row block of 128][group][level][row tile 0..7][tile]
//   B_t: [column block of 128][group][column tile 0..7][tile]
//   Rows beyond M and columns beyond N hold zeros (written by the prep
//   kernel), so the operands of one group of a workgroup tile are two
//   contiguous runs: 36 KB of A and 12 KB of B.
//   A_max_t: [group][row]  fp32, rows padded to 128.
//
// GEMM tiling: workgroup tile BM=128 rows x BN=128 columns, 8 waves as 4
// (along M) x 2 (along N), wave tile 32 rows x 64 columns = 2x4 MFMA tiles of
// 16x16, times 3 levels: each wave reuses its three A operands across its 4
// column tiles, which keeps the LDS reads per MFMA low (the A operand is
// three times the bytes of an ordinary GEMM's).  LDS holds one group's A
// (3 x 8 tiles) and B (8 tiles), double-buffered; the next group is copied
// global -> LDS directly (global_load_lds, 16 bytes per lane, no staging
// registers; each wave copies an equal share of the chunks, the last wave
// also the group's A_max and scale slices) while the current group is
// computed, one barrier per group.  Within a group a wave walks its 8 output
// tiles: a tile's 3 MFMAs are issued, then the fp32 combine of the previous
// tile, so the combine never waits for the MFMA it follows.  The combine
// (4 VALU per output per group) does not run concurrently with MFMA on the
// same SIMD -- it is issued between MFMAs -- so it adds to the MFMA time;
// two waves per SIMD hide part of it.  The MFMA results stay in VGPRs.
// Tile order: the linear workgroup id is remapped so that each XCD
// (workgroups are dealt to the 8 XCDs round-robin) gets a contiguous range of
// row-major tiles, keeping the A rows its tiles share in that XCD's L2.  The
// mapping affects speed only.
#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {
namespace pf {
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int WAVES_N = 2;     // waves along N
constexpr int WAVES_M = 4;     // waves along M
constexpr int WAVES = WAVES_M * WAVES_N;
constexpr int THREADS = 64 * WAVES;
constexpr int WM = BM / WAVES_M;   // 32 rows per wave
constexpr int WN = BN / WAVES_N;   // 64 columns per wave
constexpr int MT = WM / 16;    // 2 row tiles per wave
constexpr int NT = WN / 16;    // 4 column tiles per wave
constexpr int RT = BM / 16;    // 8 row tiles per block
constexpr int CT = BN / 16;    // 8 column tiles per block
constexpr int TILE = 1536;     // bytes of one operand tile (16 x 128 k, e2m3)
constexpr int TILE_LO = 1024;  // its [lane][dwords 0-3] part
constexpr int A_GROUP = 3 * RT * TILE;   // one group of a row block: 36 KB
constexpr int B_GROUP = CT * TILE;       // one group of a column block: 12 KB
constexpr int NXCD = 8;
}  // namespace pf

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Step-10 level weights for exact integer Y_l (no unpack scaling here).
constexpr float kE1 = (float)(1.0 / (double)kF1);
constexpr float kE2 = (float)(1.0 / (double)(kF1 * kF2));
constexpr float kE3 = (float)(1.0 / (double)(kF1 * kF2 * kF2));

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
__device__ __forceinline__ v6i pack_e2m3(const v16f& u, const v16f& v, float div) {
  return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(u, v, div);
}

// One packed operand lane -> its tile slot: dwords 0-3 at 16*slot, dwords 4-5
// at 1024 + 8*slot.
__device__ __forceinline__ void store_operand(uint8_t* tile, int slot, const v6i& p) {
  *reinterpret_cast<v4i*>(tile + slot * 16) = v4i{p[0], p[1], p[2], p[3]};
  *reinterpret_cast<v2i*>(tile + pf::TILE_LO + slot * 8) = v2i{p[4], p[5]};
}

// ---------------------------------------------------------------- prep kernel
// Waves [0, xwaves): one (16-row tile, group) each, steps 1-8 for its 16 x GS
// elements.  Lane l takes row l/4 and, with kq = l%4, the elements of operand
// lane 16*kq + row (u: k = 16*kq + j, v: k = 64 + 16*kq + j), so a group's
// maximum is a 4-lane reduction and the wave's stores fill one whole tile per
// level.
// Waves [xwaves, ...): one 16-byte tiled-weight chunk per thread (column
// tiles up to the padded width; those beyond N become zeros), converted in
// place into operand lane l of its column tile.
template <int GS>
__global__ __launch_bounds__(256) void msd_prep_kernel(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ wt, int M,
                                                       int Mpad, int K, int N, int Npad,
                                                       int64_t xwaves, uint8_t* __restrict__ a_t,
                                                       float* __restrict__ amax_t,
                                                       uint8_t* __restrict__ b_t) {
  using namespace pf;
  constexpr int EPL = GS / 4;                        // real elements per lane: 32 or 16
  const int G = K / GS;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid < xwaves) {
    const int mt = (int)(wid / G), g = (int)(wid % G);
    const int r = lane >> 2, kq = lane & 3;
    const int m = mt * 16 + r;
    const bool real = m < M;                         // padding rows decompose zeros
    const uint16_t* src = x + (real ? (int64_t)m * K + (int64_t)g * GS + 16 * kq : 0);
    float a[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // c = 0, 1: u (k = 16kq + 8c ..); c = 2, 3: v (k = 64 + 16kq + 8(c-2) ..)
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (c < 2 || GS == 128) v = *reinterpret_cast<const uint4*>(src + (c < 2 ? 8 * c : 64 + 8 * (c - 2)));
      const uint32_t vw[4] = {real ? v.x : 0u, real ? v.y : 0u, real ? v.z : 0u, real ? v.w : 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[8 * c + 2 * i] = half_bits_to_float(vw[i] & 0xffffu);
        a[8 * c + 2 * i + 1] = half_bits_to_float(vw[i] >> 16);
      }
    }
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(a[e]));
    const float amax = group_max<4>(mx);
    v16f lv[3][2];
#pragma unroll
    for (int l = 0; l < 3; ++l)
#pragma unroll
      for (int e = 0; e < 16; ++e) lv[l][0][e] = lv[l][1][e] = 0.0f;
    if (amax > 0.0f) {
      const float rcp = msd_recip(amax);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if (GS == 64 && e >= 16) break;              // v is zero for GS = 64
        float r1, r2, r3;
        msd_expand_f(a[e], amax, rcp, r1, r2, r3);
        lv[0][e / 16][e % 16] = r1;
        lv[1][e / 16][e % 16] = r2;
        lv[2][e / 16][e % 16] = r3;
      }
    }
    const int rb = mt / RT, rt = mt % RT;
#pragma unroll
    for (int l = 0; l < 3; ++l) {
      uint8_t* tile = a_t + ((((int64_t)rb * G + g) * 3 + l) * RT + rt) * TILE;
      store_operand(tile, 16 * kq + r, pack_e2m3(lv[l][0], lv[l][1], 1.0f));
    }
    if (kq == 0) amax_t[(int64_t)g * Mpad + m] = amax;
    return;
  }
  // tiled weights: chunk t = (nt * KB + kb) * 64 + lane
  const int KB = (K + kTileRows - 1) / kTileRows;
  const int64_t t = (wid - xwaves) * 64 + lane;
  if (t >= (int64_t)(Npad / kTileCols) * KB * 64) return;
  const int kb = (int)((t >> 6) % KB);
  const int nt = (int)((t >> 6) / KB);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (nt < N / kTileCols) v = *reinterpret_cast<const uint4*>(wt + t * 16);
  const int32_t dw[4] = {(int32_t)v.x, (int32_t)v.y, (int32_t)v.z, (int32_t)v.w};
  // step s (dwords 2s, 2s+1), element i = 8d + j: dword 2s + d, low nibble of
  // byte j for j < 4, high nibble of byte j - 4 otherwise
  v16f w[2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = i % 8;
      w[st][i] = sfield(dw[2 * st + i / 8], j < 4 ? 8 * j : 8 * (j - 4) + 4, 4);
    }
  const int cb = nt / CT, ct = nt % CT;
  if constexpr (GS == 128) {
    uint8_t* tile = b_t + (((int64_t)cb * G + kb) * CT + ct) * TILE;
    store_operand(tile, lane, pack_e2m3(w[0], w[1], 2.0f));
  } else {
    v16f zero;
#pragma unroll
    for (int i = 0; i < 16; ++i) zero[i] = 0.0f;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int g = 2 * kb + st;
      if (g >= G) break;                              // padding rows of the last block
      uint8_t* tile = b_t + (((int64_t)cb * G + g) * CT + ct) * TILE;
      store_operand(tile, lane, pack_e2m3(w[st], zero, 2.0f));
    }
  }
}

// ---------------------------------------------------------------- GEMM kernel
template <int GS, bool YINT>
__global__ __launch_bounds__(pf::THREADS, 1) void msd_gemm_kernel(
    const uint8_t* __restrict__ a_t, const float* __restrict__ amax_t,
    const uint8_t* __restrict__ b_t, const uint16_t* __restrict__ scale, int M, int Mpad, int K,
    int N, int g_begin, int g_end, int mblocks, int nblocks, uint16_t* __restrict__ y,
    int32_t* __restrict__ y_int) {
  using namespace pf;
  constexpr int A_KB = A_GROUP / 1024;                 // 1 KB copies per group: 36
  constexpr int B_KB = B_GROUP / 1024;                 // 12
  constexpr int CPW = (A_KB + B_KB) / WAVES;           // copies per wave: 6
  static_assert((A_KB + B_KB) % WAVES == 0 && A_KB % CPW == 0, "copy split");

  // Two named buffers (not one array indexed by the parity of the group) so
  // that the copies into one and the reads of the other are visibly disjoint.
  __shared__ __attribute__((aligned(16))) uint8_t sA0[A_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[A_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[B_GROUP];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[B_GROUP];
  __shared__ __attribute__((aligned(16))) float sAm0[BM];
  __shared__ __attribute__((aligned(16))) float sAm1[BM];
  __shared__ __attribute__((aligned(16))) uint16_t sSc0[BN];
  __shared__ __attribute__((aligned(16))) uint16_t sSc1[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;   // rows WM*wm of the tile
  const int wn = wave % WAVES_N;   // columns WN*wn of the tile

  const int total = mblocks * nblocks;
  int t = blockIdx.x;
  if (total % NXCD == 0) t = (blockIdx.x % NXCD) * (total / NXCD) + blockIdx.x / NXCD;
  const int rb = t / nblocks, cb = t % nblocks;
  const int m0 = rb * BM;
  const int n0 = cb * BN;
  const int G = K / GS;

  // This wave's share of a group's copies: waves [0, A_KB/CPW) copy 1 KB
  // pieces of the block's A run, the others pieces of its B run.
  const bool a_wave = wave * CPW < A_KB;
  const int piece = a_wave ? wave * CPW : wave * CPW - A_KB;
  const uint8_t* dma_src = (a_wave ? a_t + (int64_t)rb * G * A_GROUP : b_t + (int64_t)cb * G * B_GROUP) +
                           piece * 1024 + lane * 16;
  const int64_t dma_stride = a_wave ? A_GROUP : B_GROUP;
  const int am_row0 = m0 + lane, am_row1 = m0 + 64 + lane;   // < Mpad (a multiple of BM)
  const int sc_col = min(n0 + 2 * lane, N - 2);

  // Group g_'s operands -> LDS, by DMA (global_load_lds, 16 bytes per lane:
  // lane i's bytes land at the destination + 16*i, so a 1 KB piece keeps its
  // layout).  A_max (fp32) and the scales (fp16 pairs) go 4 bytes per lane.
  // (The 4-byte copies take byte pointers: typed float pointers made the
  // compiler crash in its SGPR-copy pass.)
#define WQBMM_DMA(g_, SA_, SB_, SAM_, SSC_)                                                        \
  do {                                                                                             \
    const uint8_t* src_ = dma_src + (int64_t)(g_) * dma_stride;                                    \
    uint8_t* dst_ = (a_wave ? (SA_) : (SB_)) + piece * 1024;                                       \
    _Pragma("unroll") for (int c = 0; c < CPW; ++c)                                                \
      __builtin_amdgcn_global_load_lds(src_ + c * 1024, dst_ + c * 1024, 16, 0, 0);                \
    if (wave == WAVES - 1) {                                                                       \
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(amax_t) + ((int64_t)(g_) * Mpad + am_row0) * 4, reinterpret_cast<uint8_t*>(SAM_), 4, 0, 0);  \
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(amax_t) + ((int64_t)(g_) * Mpad + am_row1) * 4, reinterpret_cast<uint8_t*>(SAM_) + 256, 4, 0, 0); \
      if constexpr (!YINT)                                                                         \
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(scale) + ((int64_t)(g_) * N + sc_col) * 2, reinterpret_cast<uint8_t*>(SSC_), 4, 0, 0);     \
    }                                                                                              \
  } while (0)

  // One operand (six dwords) of lane `lane` from an LDS tile, as the MFMA's
  // eight-dword argument (the last two are unused by the FP6 form).
#define WQBMM_OPERAND(TILE_PTR_)                                                                   \
  __builtin_shufflevector(*reinterpret_cast<const v4i*>((TILE_PTR_) + lane * 16),                  \
                          __builtin_shufflevector(*reinterpret_cast<const v2i*>((TILE_PTR_) + TILE_LO + lane * 8), \
                                                  v2i{0, 0}, 0, 1, -1, -1),                         \
                          0, 1, 2, 3, 4, 5, -1, -1)

  // Steps 10-11 for one 16x16 output tile (row tile PM_, column tile PN_)
  // from its three level accumulators ACC_; or the Y_int export.
#define WQBMM_PF_EPILOGUE(PM_, PN_, ACC_, G_)                                                      \
  do {                                                                                             \
    if constexpr (YINT) {                                                                          \
      const int64_t gi = (G_) - g_begin;                                                           \
      const int n = n0 + wn * WN + (PN_) * 16 + (lane & 15);                                       \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                              \
        const int m = m0 + wm * WM + (PM_) * 16 + (lane >> 4) * 4 + i;                             \
        if (m < M && n < N) {                                                                      \
          _Pragma("unroll") for (int l = 0; l < 3; ++l)                                            \
              y_int[((gi * 3 + l) * M + m) * (int64_t)N + n] = (int32_t)(ACC_)[l][i];              \
        }                                                                                          \
      }                                                                                            \
    } else {                                                                                       \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                              \
        float tt = (ACC_)[0][i] * q[PM_][i][0];                                                    \
        tt = __builtin_fmaf((ACC_)[1][i], q[PM_][i][1], tt);                                       \
        tt = __builtin_fmaf((ACC_)[2][i], q[PM_][i][2], tt);                                       \
        yacc[PM_][PN_][i] = __builtin_fmaf(tt, sc[PN_], yacc[PM_][PN_][i]);                        \
      }                                                                                            \
    }                                                                                              \
  } while (0)

  // One group from one buffer: the wave's 2 x 3 A operands stay in registers;
  // per column tile, its B operand and 2 x 3 MFMAs, the combine of each
  // output tile interleaved with the next tile's MFMAs.
#define WQBMM_COMPUTE(SA_, SB_, SAM_, SSC_, G_)                                                    \
  do {                                                                                             \
    float q[MT][4][3], sc[NT];                                                                     \
    if constexpr (!YINT) {                                                                         \
      _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                                            \
          sc[nt] = half_bits_to_float((SSC_)[wn * WN + nt * 16 + (lane & 15)]);                    \
      _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                                          \
        const float4 a4 = *reinterpret_cast<const float4*>(&(SAM_)[wm * WM + mt * 16 + (lane >> 4) * 4]); \
        const float am[4] = {a4.x, a4.y, a4.z, a4.w};                                              \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                            \
          q[mt][i][0] = am[i] * kE1;                                                               \
          q[mt][i][1] = am[i] * kE2;                                                               \
          q[mt][i][2] = am[i] * kE3;                                                               \
        }                                                                                          \
      }                                                                                            \
    }                                                                                              \
    v8i af[MT][3];                                                                                 \
    _Pragma("unroll") for (int mt = 0; mt < MT; ++mt)                                              \
      _Pragma("unroll") for (int l = 0; l < 3; ++l)                                                \
        af[mt][l] = WQBMM_OPERAND((SA_) + (l * RT + wm * MT + mt) * TILE);                         \
    v4f acc[2][3];                                                                                 \
    _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) {                                            \
      const v8i bf = WQBMM_OPERAND((SB_) + (wn * NT + nt) * TILE);                                 \
      _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                                          \
        const int j = nt * MT + mt, cur = j & 1;                                                   \
        _Pragma("unroll") for (int l = 0; l < 3; ++l)                                              \
            acc[cur][l] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                        \
                af[mt][l], bf, v4f{0.f, 0.f, 0.f, 0.f}, 2, 2, 0, kScaleA, 0, kScaleB);             \
        if (j > 0) {                                                                               \
          const int pm = (j - 1) % MT, pn = (j - 1) / MT;                                          \
          WQBMM_PF_EPILOGUE(pm, pn, acc[cur ^ 1], G_);                                             \
        }                                                                                          \
      }                                                                                            \
    }                                                                                              \
    {                                                                                              \
      constexpr int jl = MT * NT - 1;                                                              \
      WQBMM_PF_EPILOGUE(jl % MT, jl / MT, acc[jl & 1], G_);                                        \
    }                                                                                              \
  } while (0)

  float yacc[MT][NT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) yacc[mt][nt][i] = 0.0f;

  // Buffer 0 holds the even-indexed groups of the range, buffer 1 the odd
  // ones.  While a group is computed from one buffer, the next group is
  // copied into the other; each wave waits for its own copies, and the
  // barrier then publishes all of them and frees the buffer just read.
  WQBMM_DMA(g_begin, sA0, sB0, sAm0, sSc0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int g = g_begin; g < g_end; g += 2) {
    if (g + 1 < g_end) WQBMM_DMA(g + 1, sA1, sB1, sAm1, sSc1);
    WQBMM_COMPUTE(sA0, sB0, sAm0, sSc0, g);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (g + 1 >= g_end) break;
    if (g + 2 < g_end) WQBMM_DMA(g + 2, sA0, sB0, sAm0, sSc0);
    WQBMM_COMPUTE(sA1, sB1, sAm1, sSc1, g + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
#undef WQBMM_COMPUTE
#undef WQBMM_PF_EPILOGUE
#undef WQBMM_OPERAND
#undef WQBMM_DMA

  if constexpr (!YINT) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * WM + mt * 16 + (lane >> 4) * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = n0 + wn * WN + nt * 16 + (lane & 15);
          if (n < N) y[(int64_t)m * N + n] = float_to_half_bits(yacc[mt][nt][i]);
        }
      }
  }
}

// ---------------------------------------------------------------- launchers

PrefillLayout prefill_layout(int gs, int64_t M, int64_t K, int64_t N) {
  PrefillLayout L;
  L.mpad = (M + pf::BM - 1) / pf::BM * pf::BM;
  L.npad = (N + pf::BN - 1) / pf::BN * pf::BN;
  const int64_t G = K / gs;
  L.a_bytes = (size_t)(3 * (L.mpad / 16) * G) * pf::TILE;
  L.amax_bytes = (size_t)(G * L.mpad) * sizeof(float);
  L.b_bytes = (size_t)((L.npad / 16) * G) * pf::TILE;
  return L;
}

hipError_t launch_prefill_prep(const void* x, const void* w, int gs, int64_t M, int64_t K,
                               int64_t N, const PrefillLayout& L, uint8_t* a_t, float* amax_t,
                               uint8_t* b_t, hipStream_t stream) {
  const int64_t xwaves = (L.mpad / 16) * (K / gs);                // (row tile, group) tasks
  const int64_t wwaves = (L.npad / kTileCols) * tiled_kblocks(K);  // 64 weight chunks each
  const unsigned blocks = (unsigned)((xwaves + wwaves + 3) / 4);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const int m = (int)M, mp = (int)L.mpad, k = (int)K, n = (int)N, np = (int)L.npad;
  if (gs == 64)
    hipLaunchKernelGGL(msd_prep_kernel<64>, dim3(blocks), dim3(256), 0, stream, xp, wp, m, mp, k, n,
                       np, xwaves, a_t, amax_t, b_t);
  else
    hipLaunchKernelGGL(msd_prep_kernel<128>, dim3(blocks), dim3(256), 0, stream, xp, wp, m, mp, k,
                       n, np, xwaves, a_t, amax_t, b_t);
  return hipGetLastError();
}

hipError_t launch_prefill_gemm(const uint8_t* a_t, const float* amax_t, const uint8_t* b_t,
                               const void* scale, int gs, int64_t M, int64_t K, int64_t N,
                               const PrefillLayout& L, int64_t g_begin, int64_t g_end, void* y,
                               int32_t* y_int, hipStream_t stream) {
  const int mblocks = (int)(L.mpad / pf::BM);
  const int nblocks = (int)(L.npad / pf::BN);
  const dim3 grid((unsigned)(mblocks * nblocks));
  const uint16_t* sp = static_cast<const uint16_t*>(scale);
  uint16_t* yp = static_cast<uint16_t*>(y);
  const int m = (int)M, mp = (int)L.mpad, k = (int)K, n = (int)N, gb = (int)g_begin, ge = (int)g_end;
#define WQBMM_GEMM_LAUNCH(GS_, Y_)                                                                 \
  hipLaunchKernelGGL((msd_gemm_kernel<GS_, Y_>), grid, dim3(pf::THREADS), 0, stream, a_t, amax_t, \
                     b_t, sp, m, mp, k, n, gb, ge, mblocks, nblocks, yp, y_int)
  if (y_int) {
    if (gs == 64) WQBMM_GEMM_LAUNCH(64, true); else WQBMM_GEMM_LAUNCH(128, true);
  } else {
    if (gs == 64) WQBMM_GEMM_LAUNCH(64, false); else WQBMM_GEMM_LAUNCH(128, false);
  }
#undef WQBMM_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace wqbmm
