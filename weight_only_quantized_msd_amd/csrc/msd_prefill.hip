// msd_prefill.hip -- int8 MFMA GEMM of the MSD method for large M.
//
// WQBMM-Exp page (the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4
// PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145):
//   §4.1 step 9   Y_int = [Y1; Y2; Y3] = A_int . Weight_group  (integer GEMM,
//                 the M axis effectively tripled, cf. §8.1 singleCoreM = 3*M)
//   §4.1 step 10  Y_group = [(Y1/7.49 + Y2/(7.49*14.98) + Y3/(7.49*14.98^2)) * A_max] * scale_group
//   §4.1 step 11  Y^i = Y_group + Y^(i-1), over groups in order
//   §6.1          MergeY reads Y_int, A_max and antiquant_scale and writes y
//
// The page runs these as separate Cube (matmul) and Vector (merge) stages
// that exchange Y_int through global memory.  Here one workgroup keeps the
// three int32 accumulators of a group in registers, so the combine and the
// fp32 accumulation over groups are fused after each group's MFMAs and only
// the fp16 result is stored.
//
// Tiling: workgroup tile BM=128 rows x BN=128 columns, 4 waves in a 2x2 grid,
// wave tile 64x64 = 4x4 MFMA tiles of 16x16, times 3 levels: one W fragment
// feeds the 12 MFMAs of its column (4 row tiles x 3 levels).  Per group the
// workgroup stages in LDS: the 3 x 128 x GS bytes of A_int, and the
// GS x 64 bytes of int4 W unpacked and transposed to [column][k] int8 so each
// MFMA operand is one 16-byte LDS read.
#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {
namespace pf {
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int THREADS = 256;
constexpr int WM = 64;
constexpr int WN = 64;
constexpr int MT = WM / 16;
constexpr int NT = WN / 16;
constexpr int PAD = 16;
}  // namespace pf

template <int GS, bool YINT>
__global__ __launch_bounds__(256, 1) void msd_prefill_kernel(
    const int8_t* __restrict__ a_int, const float* __restrict__ a_max,
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ scale, int M, int K, int N,
    int g_begin, int g_end, uint16_t* __restrict__ y, int32_t* __restrict__ y_int) {
  using namespace pf;
  constexpr int ROW = GS + PAD;  // LDS bytes per staged row (A: per m, B: per column)
  __shared__ __attribute__((aligned(16))) int8_t sA[3 * BM * ROW];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * ROW];
  __shared__ float sAmax[BM];
  __shared__ float sScale[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int64_t MK = (int64_t)M * K;
  const int G = K / GS;
  const int NB2 = N / 2;  // bytes per W row

  float yacc[MT][NT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) yacc[mt][nt][i] = 0.0f;

  for (int g = g_begin; g < g_end; ++g) {
    const int k0 = g * GS;
    __syncthreads();  // the previous group's LDS reads are complete

    // ---- stage A_int: 3 levels x BM rows x GS bytes, 16-byte chunks
    constexpr int CPR = GS / 16;
    constexpr int A_CHUNKS = 3 * BM * CPR;
    for (int c = tid; c < A_CHUNKS; c += THREADS) {
      const int row = c / CPR, ch = c % CPR;
      const int lvl = row / BM, r = row % BM, m = m0 + r;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < M) v = *reinterpret_cast<const uint4*>(a_int + lvl * MK + (int64_t)m * K + k0 + ch * 16);
      *reinterpret_cast<uint4*>(sA + row * ROW + ch * 16) = v;
    }
    if (tid < BM) {
      const int m = m0 + tid;
      sAmax[tid] = (m < M) ? a_max[(int64_t)m * G + g] : 0.0f;
    } else if constexpr (!YINT) {
      const int c = tid - BM, n = n0 + c;
      sScale[c] = (n < N) ? half_bits_to_float(scale[(int64_t)g * N + n]) : 0.0f;
    }

    // ---- stage W: units of 8 rows x 8 columns (one dword per row)
    constexpr int UNITS = (GS / 8) * (BN / 8);
    for (int u = tid; u < UNITS; u += THREADS) {
      const int cc = u % (BN / 8), rb = u / (BN / 8);
      const int ncol = n0 + cc * 8;
      uint32_t d[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        d[r] = (ncol < N) ? *reinterpret_cast<const uint32_t*>(
                                w + (int64_t)(k0 + rb * 8 + r) * NB2 + ncol / 2)
                          : 0u;
      uint32_t e0[4], e1[4];
      transpose4x4(d[0], d[1], d[2], d[3], e0[0], e0[1], e0[2], e0[3]);
      transpose4x4(d[4], d[5], d[6], d[7], e1[0], e1[1], e1[2], e1[3]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int col = cc * 8 + 2 * b;
        *reinterpret_cast<uint2*>(sB + col * ROW + rb * 8) = make_uint2(lo16(e0[b]), lo16(e1[b]));
        *reinterpret_cast<uint2*>(sB + (col + 1) * ROW + rb * 8) = make_uint2(hi16(e0[b]), hi16(e1[b]));
      }
    }
    __syncthreads();

    // ---- step 9: three integer GEMMs sharing each W fragment
    v4i acc[3][MT][NT];
#pragma unroll
    for (int l = 0; l < 3; ++l)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[l][mt][nt] = v4i{0, 0, 0, 0};

    const int kofs = (lane >> 4) * 16;
#pragma unroll
    for (int ks = 0; ks < GS / 64; ++ks) {
      v4i bf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bf[nt] = *reinterpret_cast<const v4i*>(sB + (wn * WN + nt * 16 + (lane & 15)) * ROW + ks * 64 + kofs);
#pragma unroll
      for (int l = 0; l < 3; ++l)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const v4i af = *reinterpret_cast<const v4i*>(
              sA + (l * BM + wm * WM + mt * 16 + (lane & 15)) * ROW + ks * 64 + kofs);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[l][mt][nt] = mfma_i8(af, bf[nt], acc[l][mt][nt]);
        }
    }

    if constexpr (YINT) {
      // Y_int export: undo the 16*w scaling exactly (arithmetic shift)
      const int64_t gi = g - g_begin;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wm * WM + mt * 16 + (lane >> 4) * 4 + i;
          if (m >= M) continue;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int n = n0 + wn * WN + nt * 16 + (lane & 15);
            if (n >= N) continue;
#pragma unroll
            for (int l = 0; l < 3; ++l)
              y_int[((gi * 3 + l) * M + m) * (int64_t)N + n] = acc[l][mt][nt][i] >> 4;
          }
        }
    } else {
      // ---- steps 10-11: combine the levels, scale, accumulate in fp32
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float am = sAmax[wm * WM + mt * 16 + (lane >> 4) * 4 + i];
          const float q1 = am * kC1, q2 = am * kC2, q3 = am * kC3;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float sc = sScale[wn * WN + nt * 16 + (lane & 15)];
            float t = (float)acc[0][mt][nt][i] * q1;
            t = __builtin_fmaf((float)acc[1][mt][nt][i], q2, t);
            t = __builtin_fmaf((float)acc[2][mt][nt][i], q3, t);
            yacc[mt][nt][i] = __builtin_fmaf(t, sc, yacc[mt][nt][i]);
          }
        }
    }
  }

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
  (void)G;
}

hipError_t launch_prefill_gemm(const int8_t* a_int, const float* a_max, const void* w,
                               const void* scale, int gs, int64_t M, int64_t K, int64_t N,
                               int64_t g_begin, int64_t g_end, void* y, int32_t* y_int,
                               hipStream_t stream) {
  const dim3 grid((unsigned)((N + pf::BN - 1) / pf::BN), (unsigned)((M + pf::BM - 1) / pf::BM));
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint16_t* sp = static_cast<const uint16_t*>(scale);
  uint16_t* yp = static_cast<uint16_t*>(y);
  const int m = (int)M, k = (int)K, n = (int)N, gb = (int)g_begin, ge = (int)g_end;
  if (y_int) {
    if (gs == 64)
      hipLaunchKernelGGL((msd_prefill_kernel<64, true>), grid, dim3(pf::THREADS), 0, stream, a_int, a_max, wp, sp, m, k, n, gb, ge, yp, y_int);
    else
      hipLaunchKernelGGL((msd_prefill_kernel<128, true>), grid, dim3(pf::THREADS), 0, stream, a_int, a_max, wp, sp, m, k, n, gb, ge, yp, y_int);
  } else {
    if (gs == 64)
      hipLaunchKernelGGL((msd_prefill_kernel<64, false>), grid, dim3(pf::THREADS), 0, stream, a_int, a_max, wp, sp, m, k, n, gb, ge, yp, y_int);
    else
      hipLaunchKernelGGL((msd_prefill_kernel<128, false>), grid, dim3(pf::THREADS), 0, stream, a_int, a_max, wp, sp, m, k, n, gb, ge, yp, y_int);
  }
  return hipGetLastError();
}

}  // namespace wqbmm
