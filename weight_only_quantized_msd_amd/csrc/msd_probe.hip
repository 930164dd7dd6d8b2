// msd_probe.hip -- measurement helper, not part of the operator: a plain
// streaming read of a byte range, the achievable-bandwidth reference that the
// weight-streaming (decode) kernels are compared with.  It reads every byte
// once with 16-byte nontemporal loads (the loads the decode kernels use for
// their weights): a wave's load covers 1 KB, four loads in flight per lane.
// Each lane folds what it read into one word and stores it only if it equals
// a value the caller's data never produces, so the loads cannot be dropped
// and the kernel writes nothing in practice.
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

}  // namespace

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
