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
// The integer contraction runs on the fp8 MFMA (v_mfma_scale_f32_16x16x128_
// f8f6f4, unit scales).  Every level value lies in [-7, 7] and every weight in
// [-8, 7]; both are exact in fp8 e4m3, their products are exact, and a
// group's sum (|Y_l| <= 7*8*GS = 7168) is exact in the fp32 accumulator, so
// the MFMA returns the integer Y_l exactly (the Y_int export converts it to
// int32).  At the same dense rate as int8 this spares the epilogue three
// int->float conversions per output per group, which otherwise made the
// fp32 combine (VALU) slower than the contraction (MFMA).
//
// Operand tiles (written by msd_prep_kernel, read by the GEMM):
//   An MFMA operand covers 16 rows (A) or 16 columns (B) x 128 k, 32 bytes per
//   lane.  Lane l holds row/column l%16 and, in byte j of its half h (h = 0, 1),
//   k = 64*h + 16*(l/16) + j of the group: the half is a 64-row step of the
//   tiled weight format, so a tiled-weight chunk converts into one lane's two
//   halves in place.  For GS = 64 only half 0 is stored and half 1 is zero.
//   The contraction is the same for any byte -> k assignment that A and B
//   share.  A tile (per 16 rows or columns and group) is stored as
//   [half][lane][16 bytes], GS*16 bytes, so each half is one conflict-free
//   1 KB ds_read_b128 per wave.
//   A_t: [level][row tile][group][tile]   (rows padded to 16 with zeros)
//   B_t: [column tile][group][tile]
//   A_max_t: [group][row]  fp32
//
// GEMM tiling: workgroup tile BM=128 rows x BN=128 columns, 4 waves, wave
// tile 32 rows x 128 columns = 2x8 MFMA tiles of 16x16, times 3 levels: each
// wave reuses its three A operands across all 8 column tiles, which keeps
// the LDS reads per MFMA low (the A operand is three times the bytes of an
// ordinary GEMM's).  LDS holds one group's A (3 x 8 tiles) and B (8 tiles),
// double-buffered; the next group is copied global -> LDS directly
// (global_load_lds, 16 bytes per lane, no staging registers) while the
// current group is computed, one barrier per group.  Within a group a wave
// walks its 16 output tiles: the tile's 3 MFMAs are issued, then the fp32
// combine of the previous tile, so MFMA and VALU overlap in the wave.
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
constexpr int NXCD = 8;
}  // namespace pf

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Step-10 level weights for exact integer Y_l (no unpack scaling here).
constexpr float kE1 = (float)(1.0 / (double)kF1);
constexpr float kE2 = (float)(1.0 / (double)(kF1 * kF2));
constexpr float kE3 = (float)(1.0 / (double)(kF1 * kF2 * kF2));

// Signed bit field of v as a float.  The builtin's result type is unsigned, so
// it is reinterpreted as int32 before the conversion (v_cvt_f32_i32).
__device__ __forceinline__ float sfield(int32_t v, int off, int width) {
  return (float)(int32_t)__builtin_amdgcn_sbfe(v, off, width);
}

// Four integer-valued floats -> four e4m3 bytes (exact), byte i from f_i.
__device__ __forceinline__ uint32_t pack4_fp8(float f0, float f1, float f2, float f3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, lo, true);
}

// ---------------------------------------------------------------- prep kernel
// Waves [0, xwaves): one (16-row tile, group) each, steps 1-8 for its 16 x GS
// elements.  Lane l takes row l/4 and the GS/4 consecutive elements at
// (l%4)*GS/4 of the group, so a group's maximum is a 4-lane reduction and
// every 16-byte chunk it writes is one operand slot (slot 16*kb + row of half
// h, for k = 64h + 16kb + j): each store of a wave fills whole 256-byte runs.
// Waves [xwaves, ...): one 16-byte tiled-weight chunk per thread, whose two
// 64-row steps become the lane's two 16-byte fp8 operand halves.
template <int GS>
__global__ __launch_bounds__(256) void msd_prep_kernel(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ wt, int M,
                                                       int Mpad, int K, int N, int64_t xwaves,
                                                       uint8_t* __restrict__ a_t,
                                                       float* __restrict__ amax_t,
                                                       uint8_t* __restrict__ b_t) {
  constexpr int TILE = GS * 16;
  constexpr int EPL = GS / 4;                        // elements per lane: 32 or 16
  const int G = K / GS;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid < xwaves) {
    const int mt = (int)(wid / G), g = (int)(wid % G);
    const int r = lane >> 2, q = lane & 3;
    const int m = mt * 16 + r;
    const bool real = m < M;                         // padding rows decompose zeros
    const uint16_t* src = x + (real ? (int64_t)m * K + (int64_t)g * GS + q * EPL : 0);
    float a[EPL];
    float mx = 0.0f;
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * c);
      const uint32_t vw[4] = {real ? v.x : 0u, real ? v.y : 0u, real ? v.z : 0u, real ? v.w : 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[8 * c + 2 * i] = half_bits_to_float(vw[i] & 0xffffu);
        a[8 * c + 2 * i + 1] = half_bits_to_float(vw[i] >> 16);
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) mx = fmaxf(mx, fabsf(a[e]));
    const float amax = group_max<4>(mx);
    uint32_t out[3][EPL / 4];
#pragma unroll
    for (int l = 0; l < 3; ++l)
#pragma unroll
      for (int d = 0; d < EPL / 4; ++d) out[l][d] = 0u;
    if (amax > 0.0f) {
      const float rcp = msd_recip(amax);
#pragma unroll
      for (int d = 0; d < EPL / 4; ++d) {
        float r3[3][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) msd_expand_f(a[4 * d + i], amax, rcp, r3[0][i], r3[1][i], r3[2][i]);
#pragma unroll
        for (int l = 0; l < 3; ++l) out[l][d] = pack4_fp8(r3[l][0], r3[l][1], r3[l][2], r3[l][3]);
      }
    }
    const int64_t MTILES = Mpad / 16;
#pragma unroll
    for (int c = 0; c < EPL / 16; ++c) {
      const int kk = q * EPL + 16 * c;               // group-relative k of this chunk
      const int slot = (kk >> 6) * 64 + 16 * ((kk >> 4) & 3) + r;
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        uint8_t* dst = a_t + ((l * MTILES + mt) * G + g) * (int64_t)TILE + slot * 16;
        *reinterpret_cast<uint4*>(dst) =
            make_uint4(out[l][4 * c], out[l][4 * c + 1], out[l][4 * c + 2], out[l][4 * c + 3]);
      }
    }
    if (q == 0) amax_t[(int64_t)g * Mpad + m] = amax;
    return;
  }
  // tiled weights: chunk t = (nt * KB + kb) * 64 + lane
  const int KB = (K + kTileRows - 1) / kTileRows;
  const int64_t t = (wid - xwaves) * 64 + lane;
  if (t >= (int64_t)(N / kTileCols) * KB * 64) return;
  const int kb = (int)((t >> 6) % KB);
  const int64_t nt = (t >> 6) / KB;
  const uint4 v = *reinterpret_cast<const uint4*>(wt + t * 16);
  const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    // step st: dwords 2st, 2st+1; rows j in the low nibbles, j+4 in the high
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int32_t e = (int32_t)dw[2 * st + d];
      o[2 * d] = pack4_fp8(sfield(e, 0, 4), sfield(e, 8, 4), sfield(e, 16, 4), sfield(e, 24, 4));
      o[2 * d + 1] = pack4_fp8(sfield(e, 4, 4), sfield(e, 12, 4), sfield(e, 20, 4), sfield(e, 28, 4));
    }
    uint8_t* dst;
    if constexpr (GS == 128) {
      dst = b_t + ((nt * G + kb) * 2 + st) * 1024 + lane * 16;
    } else {
      const int g = 2 * kb + st;
      if (g >= G) continue;                           // padding rows of the last block
      dst = b_t + (nt * G + g) * 1024 + lane * 16;
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
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
  constexpr int TILE = GS * 16;                        // bytes per operand tile and group
  constexpr int HALVES = GS / 64;                      // 1 KB chunks per tile
  constexpr int A_CHUNKS = 3 * (BM / 16) * HALVES;     // per group: 48 or 24
  constexpr int B_CHUNKS = (BN / 16) * HALVES;         // per group: 16 or 8
  constexpr int CPW = (A_CHUNKS + B_CHUNKS) / WAVES;   // chunks copied per wave
  static_assert((A_CHUNKS + B_CHUNKS) % WAVES == 0 && A_CHUNKS % CPW == 0, "chunk split");

  // Two named buffers (not one array indexed by the parity of the group) so
  // that the copies into one and the reads of the other are visibly disjoint.
  __shared__ __attribute__((aligned(16))) uint8_t sA0[A_CHUNKS * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[A_CHUNKS * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[B_CHUNKS * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[B_CHUNKS * 1024];
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
  const int m0 = (t / nblocks) * BM;
  const int n0 = (t % nblocks) * BN;
  const int G = K / GS;
  const int64_t MTILES = Mpad / 16;

  // This wave's share of a group's operand chunks: chunk q = tile * HALVES +
  // half, A tiles (level, row tile) first, then B tiles; a wave's chunks are
  // all A or all B.  csrc[c] is the chunk's byte offset at group 0 (uniform).
  // Tiles of rows beyond the padded row count, and of columns beyond N, are
  // read from a clamped valid tile: they only feed outputs never stored.
  const bool a_wave = wave * CPW < A_CHUNKS;
  int64_t csrc[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int q = wave * CPW + c;
    if (q < A_CHUNKS) {
      const int tile = q / HALVES, h = q % HALVES;
      const int l = tile / (BM / 16), mt = min(m0 / 16 + tile % (BM / 16), (int)MTILES - 1);
      csrc[c] = (l * MTILES + mt) * G * (int64_t)TILE + h * 1024;
    } else {
      const int tile = (q - A_CHUNKS) / HALVES, h = (q - A_CHUNKS) % HALVES;
      const int nt = min(n0 / 16 + tile, N / 16 - 1);
      csrc[c] = (int64_t)nt * G * TILE + h * 1024;
    }
  }
  const int am_row0 = min(m0 + lane, Mpad - 1), am_row1 = min(m0 + 64 + lane, Mpad - 1);
  const int sc_col = min(n0 + 2 * lane, N - 2);

  // Group g_'s operands -> LDS, by DMA (global_load_lds, 16 bytes per lane:
  // lane i's bytes land at the destination + 16*i, i.e. a [lane][16] chunk).
  // A_max (fp32) and the scales (fp16 pairs) go 4 bytes per lane.  (The
  // 4-byte copies take byte pointers: typed float pointers made the
  // compiler crash in its SGPR-copy pass.)
#define WQBMM_DMA(g_, SA_, SB_, SAM_, SSC_)                                                        \
  do {                                                                                             \
    const int64_t goff_ = (int64_t)(g_) * TILE;                                                    \
    _Pragma("unroll") for (int c = 0; c < CPW; ++c) {                                              \
      const int q = wave * CPW + c;                                                                \
      const uint8_t* src_ = (a_wave ? a_t : b_t) + (csrc[c] + goff_) + lane * 16;                  \
      uint8_t* dst_ = a_wave ? (SA_) + q * 1024 : (SB_) + (q - A_CHUNKS) * 1024;                   \
      __builtin_amdgcn_global_load_lds(src_, dst_, 16, 0, 0);                                      \
    }                                                                                              \
    if (wave == WAVES - 1) {                                                                       \
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(amax_t) + ((int64_t)(g_) * Mpad + am_row0) * 4, reinterpret_cast<uint8_t*>(SAM_), 4, 0, 0);  \
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(amax_t) + ((int64_t)(g_) * Mpad + am_row1) * 4, reinterpret_cast<uint8_t*>(SAM_) + 256, 4, 0, 0); \
      if constexpr (!YINT)                                                                         \
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(scale) + ((int64_t)(g_) * N + sc_col) * 2, reinterpret_cast<uint8_t*>(SSC_), 4, 0, 0);     \
    }                                                                                              \
  } while (0)

  // Steps 10-11 for one 16x16 output tile (row tile PM_, column tile PN_)
  // from its three level accumulators ACC_; or the Y_int export.
#define WQBMM_PF_EPILOGUE(PM_, PN_, ACC_, G_)                                                      \
  do {                                                                                             \
    if constexpr (YINT) {                                                                          \
      const int64_t gi = (G_) - g_begin;                                                           \
      const int n = n0 + wn * WN + (PN_) * 16 + (lane & 15);                                                 \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                              \
        const int m = m0 + wm * WM + (PM_) * 16 + (lane >> 4) * 4 + i;                           \
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
          sc[nt] = half_bits_to_float((SSC_)[wn * WN + nt * 16 + (lane & 15)]);                              \
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
      _Pragma("unroll") for (int l = 0; l < 3; ++l) {                                              \
        const uint8_t* base = (SA_) + (l * (BM / 16) + wm * MT + mt) * TILE;                     \
        const v4i lo = *reinterpret_cast<const v4i*>(base + lane * 16);                            \
        const v4i hi = HALVES == 2 ? *reinterpret_cast<const v4i*>(base + 1024 + lane * 16) : v4i{0, 0, 0, 0}; \
        af[mt][l] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};                   \
      }                                                                                            \
    v4f acc[2][3];                                                                                 \
    _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) {                                            \
      const uint8_t* bb = (SB_) + (wn * NT + nt) * TILE;                                                       \
      const v4i blo = *reinterpret_cast<const v4i*>(bb + lane * 16);                               \
      const v4i bhi = HALVES == 2 ? *reinterpret_cast<const v4i*>(bb + 1024 + lane * 16) : v4i{0, 0, 0, 0}; \
      const v8i bf = v8i{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};          \
      _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                                          \
        const int j = nt * MT + mt, cur = j & 1;                                                   \
        _Pragma("unroll") for (int l = 0; l < 3; ++l)                                              \
            acc[cur][l] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                        \
                af[mt][l], bf, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);                     \
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
  L.mpad = (M + 15) / 16 * 16;
  const int64_t G = K / gs;
  L.a_bytes = (size_t)(3 * L.mpad * K);
  L.amax_bytes = (size_t)(G * L.mpad) * sizeof(float);
  L.b_bytes = (size_t)(K * N);
  return L;
}

hipError_t launch_prefill_prep(const void* x, const void* w, int gs, int64_t M, int64_t K,
                               int64_t N, const PrefillLayout& L, uint8_t* a_t, float* amax_t,
                               uint8_t* b_t, hipStream_t stream) {
  const int64_t xwaves = (L.mpad / 16) * (K / gs);             // (row tile, group) tasks
  const int64_t wwaves = (N / kTileCols) * tiled_kblocks(K);   // 64 weight chunks each
  const unsigned blocks = (unsigned)((xwaves + wwaves + 3) / 4);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const int m = (int)M, mp = (int)L.mpad, k = (int)K, n = (int)N;
  if (gs == 64)
    hipLaunchKernelGGL(msd_prep_kernel<64>, dim3(blocks), dim3(256), 0, stream, xp, wp, m, mp, k, n,
                       xwaves, a_t, amax_t, b_t);
  else
    hipLaunchKernelGGL(msd_prep_kernel<128>, dim3(blocks), dim3(256), 0, stream, xp, wp, m, mp, k, n,
                       xwaves, a_t, amax_t, b_t);
  return hipGetLastError();
}

hipError_t launch_prefill_gemm(const uint8_t* a_t, const float* amax_t, const uint8_t* b_t,
                               const void* scale, int gs, int64_t M, int64_t K, int64_t N,
                               const PrefillLayout& L, int64_t g_begin, int64_t g_end, void* y,
                               int32_t* y_int, hipStream_t stream) {
  const int mblocks = (int)((M + pf::BM - 1) / pf::BM);
  const int nblocks = (int)((N + pf::BN - 1) / pf::BN);
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
