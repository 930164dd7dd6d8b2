// msd_launch.hpp -- internal launcher interface between the host API
// (msd_api.cpp) and the kernel translation units.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wqbmm {

// Steps 1-8 (WQBMM-Exp page §4.1): x fp16 [M][K] -> a_int int8 [3][M][K],
// a_max fp32 [M][K/gs].
hipError_t launch_prepass(const void* x, int gs, int64_t M, int64_t K, int8_t* a_int,
                          float* a_max, hipStream_t stream);

// Steps 9-11 on a pre-computed A_int/A_max with the int8 MFMA GEMM.
// y_int == nullptr: groups [0, G) are combined into y (fp16 [M][N]).
// y_int != nullptr: groups [g_begin, g_end) are stored as int32 Y_int.
hipError_t launch_prefill_gemm(const int8_t* a_int, const float* a_max, const void* w,
                               const void* scale, int gs, int64_t M, int64_t K, int64_t N,
                               int64_t g_begin, int64_t g_end, void* y, int32_t* y_int,
                               hipStream_t stream);

// The fused decode kernel (M <= 16): steps 1-11 in one launch, with a
// deterministic split-K reduction through `partials` and one self-re-arming
// counter per column block (`counters` must be zero before the first launch).
struct DecodePlan {
  int64_t col_blocks;   // blocks of columns per launch
  int64_t splits;       // K-slices per column block
  int64_t cols;         // columns per block
  int wn, wk;           // waves per workgroup along N and along K
};
DecodePlan decode_plan(int gs, int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end);
size_t decode_partials_bytes(const DecodePlan& p, int64_t M, int64_t N);

hipError_t launch_decode(const void* x, const void* w, const void* scale, int gs, int64_t M,
                         int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                         int32_t* y_int, float* partials, uint32_t* counters,
                         const DecodePlan& plan, hipStream_t stream);

// Zero n counter words (a kernel, not a memset).
hipError_t launch_zero_counters(uint32_t* counters, int64_t n, hipStream_t stream);

}  // namespace wqbmm
