// msd_prepass.hip -- the MSD pre-pass: WQBMM-Exp page (the page
// "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4 PerGroup 伪量化 MatMul 的
// MSD 算法与双模板流水设计", lpnh.cn/news/2294145) §4.1 steps 1-8, and §6.1's
// pre-processing stage (UnfoldA: A_max and the unfolded A).
//
// HBM-bound elementwise work: each thread reads one 16-byte chunk of x
// (8 fp16), the GS/8 lanes of a group reduce |x| to A_max with cross-lane
// shuffles, and each thread writes 8 bytes per level.  Per element: 2 bytes
// read, 3 bytes written (+4 bytes of A_max per group).
#include "msd_device.hpp"
#include "msd_launch.hpp"

namespace wqbmm {

template <int GS>
__global__ __launch_bounds__(256) void msd_prepass_kernel(const uint16_t* __restrict__ x,
                                                          int64_t MK, int8_t* __restrict__ a_int,
                                                          float* __restrict__ a_max) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t e0 = t * 8;
  const bool live = e0 < MK;  // MK is a multiple of GS: a group is all-live or all-dead
  uint4 xv = make_uint4(0u, 0u, 0u, 0u);
  if (live) xv = *reinterpret_cast<const uint4*>(x + e0);
  uint32_t lv[3][2];
  float amax;
  msd_decompose8<GS>(xv, lv, amax);
  if (live) {
#pragma unroll
    for (int l = 0; l < 3; ++l)
      *reinterpret_cast<uint2*>(a_int + (int64_t)l * MK + e0) = make_uint2(lv[l][0], lv[l][1]);
    if ((threadIdx.x & (GS / 8 - 1)) == 0) a_max[e0 / GS] = amax;
  }
}

hipError_t launch_prepass(const void* x, int gs, int64_t M, int64_t K, int8_t* a_int,
                          float* a_max, hipStream_t stream) {
  const int64_t MK = M * K;
  const int64_t threads = MK / 8;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (blocks == 0) return hipSuccess;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (gs == 64)
    hipLaunchKernelGGL(msd_prepass_kernel<64>, dim3(blocks), dim3(256), 0, stream, xp, MK, a_int, a_max);
  else
    hipLaunchKernelGGL(msd_prepass_kernel<128>, dim3(blocks), dim3(256), 0, stream, xp, MK, a_int, a_max);
  return hipGetLastError();
}

}  // namespace wqbmm
