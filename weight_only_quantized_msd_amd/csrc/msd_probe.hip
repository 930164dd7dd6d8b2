// msd_probe.hip -- measurement helpers, not part of the operator.
//
// (1) A plain streaming read of a byte range, the achievable-bandwidth
// reference that the weight-streaming (decode) kernels are compared with.  It reads every byte
// once with 16-byte nontemporal loads (the loads the decode kernels use for
// their weights): a wave's load covers 1 KB, four loads in flight per lane.
// Each lane folds what it read into one word and stores it only if it equals
// a value the caller's data never produces, so the loads cannot be dropped
// and the kernel writes nothing in practice.
//
// (2) An MFMA / VALU co-issue probe: whether the FP6 MFMAs and the fp32
// FMAs of the prefill GEMMs' combine overlap on a SIMD.  256 workgroups of 8
// waves (two per SIMD, as in the group-128 GEMM), each round a block of 12
// independent v_mfma_scale_f32_16x16x128_f8f6f4 (eight accumulators) and/or
// a block of 64 fp32 FMAs in 16 independent chains, no memory traffic inside
// the loop; the results are summed into one float per thread at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wqbmm_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void msd_probe_read_kernel(const u32x4* __restrict__ src,
                                                                  int64_t chunks,
                                                                  uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t h = 0;
  for (; i + (kUnroll - 1) * stride < chunks; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) h ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < chunks; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    h ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (h == 0x9E3779B9u) sink[0] = h;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kOvlThreads = 512;
constexpr int kOvlBlocks = 256;
constexpr int kOvlMfma = 12;    // MFMAs per round
constexpr int kOvlFma = 64;     // fp32 FMAs per round

// mode 0: MFMA blocks only; 1: FMA blocks only; 2: every wave an MFMA block
// then an FMA block per round; 3: waves 0-3 MFMA blocks only, waves 4-7 FMA
// blocks only (one of each kind per SIMD); 4: as 2 with a workgroup barrier
// after every round (the waves of a SIMD kept in the same phase, as a GEMM's
// group barrier keeps them); 5, 6, 7: as 2, 0, 1 with waves 4-7 idle (one
// wave per SIMD); 8, 9, 10: as 2, 0, 1 with twice the workgroups (two per
// CU: four waves per SIMD).
__global__ __launch_bounds__(kOvlThreads) void msd_probe_mfma_valu_kernel(int mode, int iters,
                                                                         float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // e2m3 codes of small values in every byte (any bit pattern is a valid
  // operand; these keep the sums finite)
  const int pat = 0x08080808 | (lane & 3);
  const i32x8 a = {pat, pat, pat, pat, pat, pat, 0, 0};
  const i32x8 b = {pat ^ 1, pat, pat ^ 2, pat, pat, pat ^ 3, 0, 0};
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = (float)(lane + i) * 0.001f;
  const float m = 0.999f, c = 0.001f;
  const bool one_per_simd = mode >= 5 && mode <= 7;
  const bool do_mfma = mode == 0 || mode == 2 || mode == 4 || mode == 5 || mode == 6 ||
                       mode == 8 || mode == 9 || (mode == 3 && wave < 4);   // wave-uniform
  const bool do_fma = mode == 1 || mode == 2 || mode == 4 || mode == 5 || mode == 7 ||
                      mode == 8 || mode == 10 || (mode == 3 && wave >= 4);
  if (one_per_simd && wave >= 4) {   // idle waves write their slot and leave
    out[(int64_t)blockIdx.x * kOvlThreads + threadIdx.x] = 0.f;
    return;
  }
  for (int it = 0; it < iters; ++it) {
    if (do_mfma) {
#pragma unroll
      for (int j = 0; j < kOvlMfma; ++j)
        acc[j & 7] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j & 7], 2, 2, 0, 127, 0, 127);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_fma) {
#pragma unroll
      for (int j = 0; j < kOvlFma; ++j) x[j & 15] = __builtin_fmaf(x[j & 15], m, c);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (mode == 4) __builtin_amdgcn_s_barrier();   // every wave of the workgroup takes it
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += x[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[(int64_t)blockIdx.x * kOvlThreads + threadIdx.x] = sum;
}

}  // namespace

extern "C" int wqbmm_probe_mfma_valu(int mode, int iters, void* out, void* stream) {
  if (!out) return 1;
  if (mode < 0 || mode > 10 || iters < 1 || iters > (1 << 20)) return 2;
  const unsigned blocks = mode >= 8 ? 2 * kOvlBlocks : kOvlBlocks;
  hipLaunchKernelGGL(msd_probe_mfma_valu_kernel, dim3(blocks), dim3(kOvlThreads), 0,
                     static_cast<hipStream_t>(stream), mode, iters, static_cast<float*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int wqbmm_probe_stream_read(const void* src, int64_t bytes, void* sink, void* stream) {
  if (!src || !sink) return 1;
  if (bytes <= 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0) return 2;
  const int64_t chunks = bytes / 16;
  int64_t grid = (chunks + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (grid > WQBMM_PROBE_MAX_GRID) grid = WQBMM_PROBE_MAX_GRID;
  hipLaunchKernelGGL(msd_probe_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), chunks,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
