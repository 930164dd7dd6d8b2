// msd_prepack.hip -- one-time re-layout of the int4 weights into the tiled
// format every MSD kernel reads.
//
// The WQBMM-Exp page (the page "WeightQuantBatchMatmulExperiment 算子深度解析：
// A16W4 PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145)
// takes the weight as a K x N int4 ND matrix, two values per byte (§4.2,
// §4.3).  Weights are static across calls, so, like the weight re-layout in the
// call example (section 调用示例) of the page "CANN ops-math：
// aclnnCalculateMatmulWeightSizeV2 接口详解" (zskr.cn/news/2299903) -- query the
// re-laid-out size, allocate, convert the ND weight once, then hand the
// converted weight to the quantized matmul -- the library converts them once
// into a layout shaped after its MFMA operands:
//   * a 16-column x 128-row tile is 1 KB, one 16-byte chunk per lane of a
//     wave, so any workgroup's share of W is read as whole 1 KB runs however
//     few columns it covers;
//   * the chunk of lane l holds column l%16 and rows 16*(l/16) .. +15 of each
//     64-row step, i.e. exactly the lane's B operand of v_mfma_i32_16x16x64_i8;
//   * within a dword, byte j pairs row j (low nibble) with row j+4 (high
//     nibble), so masking the high nibbles (and shifting the low ones up)
//     yields four int8 values 16*w in ascending row order.
// The exact bit layout is stated with the launcher interface.
#include "msd_launch.hpp"

namespace wqbmm {

// One thread per 16-byte chunk.  Reads the 32 nibbles of its column from 32
// rows of the ND matrix (a one-time conversion; the reads are gathers).
__global__ __launch_bounds__(256) void msd_prepack_kernel(const uint8_t* __restrict__ w_nd, int K,
                                                          int N, int KB, int64_t chunks,
                                                          uint8_t* __restrict__ w_tiled) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= chunks) return;
  const int l = (int)(t & 63);
  const int64_t tk = t >> 6;                 // nt * KB + kb
  const int kb = (int)(tk % KB);
  const int nt = (int)(tk / KB);
  const int n = nt * kTileCols + (l & 15);
  const int shift = 4 * (n & 1);
  const uint8_t* col = w_nd + n / 2;
  auto nib = [&](int k) -> uint32_t {
    return k < K ? (uint32_t)(col[(int64_t)k * (N / 2)] >> shift) & 0xFu : 0u;
  };
  uint32_t out[4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int k0 = kb * kTileRows + 64 * s + 16 * (l >> 4) + 8 * d;
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) v |= (nib(k0 + j) | (nib(k0 + 4 + j) << 4)) << (8 * j);
      out[2 * s + d] = v;
    }
  *reinterpret_cast<uint4*>(w_tiled + t * 16) = make_uint4(out[0], out[1], out[2], out[3]);
}

hipError_t launch_prepack(const void* w_nd, int64_t K, int64_t N, void* w_tiled, hipStream_t stream) {
  const int64_t KB = tiled_kblocks(K);
  const int64_t chunks = (N / kTileCols) * KB * 64;
  hipLaunchKernelGGL(msd_prepack_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(w_nd), (int)K, (int)N, (int)KB, chunks,
                     static_cast<uint8_t*>(w_tiled));
  return hipGetLastError();
}

}  // namespace wqbmm
