// msd_launch.hpp -- internal launcher interface between the host API
// (msd_api.cpp) and the kernel translation units.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wqbmm {

// ---- tiled int4 weights (the kernels' weight format) ------------------------
// Chunk (column tile nt of 16 columns, k-block kb of 128 rows, lane l) is 16
// bytes at ((nt * KB + kb) * 64 + l) * 16, KB = ceil(K / 128).  It holds column
// n = 16*nt + l%16 at k = 128*kb + 64*s + 16*(l/16) + i (i = 0..15) for the two
// 64-row steps s = 0, 1 (bytes 8s .. 8s+7).  In dword d (0, 1) of a step, byte
// j carries k-offset 8d + j in its low nibble and 8d + 4 + j in its high
// nibble (4-bit two's complement).  Rows k >= K hold 0.
constexpr int kTileCols = 16;
constexpr int kTileRows = 128;
inline int64_t tiled_kblocks(int64_t K) { return (K + kTileRows - 1) / kTileRows; }
inline size_t tiled_weight_bytes(int64_t K, int64_t N) {
  return (size_t)(N / kTileCols) * (size_t)tiled_kblocks(K) * 1024u;
}
// Row-major w [K][N/2] (column 2j in the low nibble of byte j) -> tiled.
hipError_t launch_prepack(const void* w_nd, int64_t K, int64_t N, void* w_tiled, hipStream_t stream);

// Steps 1-8 (WQBMM-Exp page §4.1): x fp16 [M][K] -> a_int int8 [3][M][K],
// a_max fp32 [M][K/gs].
hipError_t launch_prepass(const void* x, int gs, int64_t M, int64_t K, int8_t* a_int,
                          float* a_max, hipStream_t stream);

// Prefill path (any M): a preparation kernel writes the MFMA operand tiles
// (the three levels of x and the tiled weights, as FP6 e2m3) and the rows'
// step-10 level weights (A_max * w_l, fp32), then the GEMM contracts them and
// applies steps 10-11.
struct PrefillLayout {
  int64_t mpad;        // rows padded to a multiple of 128
  int64_t bn;          // columns per GEMM workgroup tile: 128 or 256
  int64_t npad;        // columns padded to a multiple of bn
  size_t a_bytes;      // level tiles of x: 3 * (mpad/16) * G tiles of 1536 bytes
  size_t q_bytes;      // level weights, [group][row block][level][128] fp32
  size_t b_bytes;      // weight tiles (0 if w_in_gemm); at group size 128 their columns are
                       // padded to a multiple of 256 whatever bn is
  bool w_in_gemm;      // the GEMM converts the tiled int4 weights itself (few row blocks)
  int64_t splits = 1;  // K-splits of the GEMM (few tiles); > 1: fp32 partial sums + a reduction
  size_t part_bytes = 0;   // splits * M * N fp32 partial sums (0 without a split)
};
PrefillLayout prefill_layout(int gs, int64_t M, int64_t K, int64_t N);

// weights == false (group size 128 only): the weight tiles b_t are the
// weights' operand form from launch_operand_weights and are not written.
hipError_t launch_prefill_prep(const void* x, const void* w, int gs, int64_t M, int64_t K,
                               int64_t N, const PrefillLayout& L, uint8_t* a_t, float* q_t,
                               uint8_t* b_t, bool weights, hipStream_t stream);

// The weights' operand form for the group-128 GEMM: the weight tiles the
// preparation kernel writes (FP6 e2m3, [256-column block][128-row block][16
// column tiles of 1536 bytes], columns padded to a multiple of 256 with
// zeros), converted once from the tiled weights.
inline int64_t operand_weight_npad(int64_t N) { return (N + 255) / 256 * 256; }
size_t operand_weight_bytes(int64_t K, int64_t N);
hipError_t launch_operand_weights(const void* w_tiled, int64_t K, int64_t N, uint8_t* w_op,
                                  hipStream_t stream);

// y_int == nullptr: groups [g_begin, g_end) are combined into y (fp16 [M][N]);
// otherwise they are stored as int32 Y_int.  With L.splits > 1 the GEMM
// splits the group range and writes fp32 partial sums to `part`
// (L.part_bytes), which a second kernel adds in split order into y.
hipError_t launch_prefill_gemm(const uint8_t* a_t, const float* q_t, const uint8_t* b_t,
                               const void* w_tiled,
                               const void* scale, int gs, int64_t M, int64_t K, int64_t N,
                               const PrefillLayout& L, int64_t g_begin, int64_t g_end, void* y,
                               int32_t* y_int, float* part, hipStream_t stream);

// Group size 64 (msd_prefill64.hip): the same roles on the 32x32x64 FP6 MFMA
// (one group per instruction); the launchers above dispatch to these.
PrefillLayout prefill64_layout(int64_t M, int64_t K, int64_t N);
hipError_t launch_prefill64_prep(const void* x, const void* w, int64_t M, int64_t K, int64_t N,
                                 const PrefillLayout& L, uint8_t* x_t, float* q_t, uint8_t* w_t,
                                 hipStream_t stream);
hipError_t launch_prefill64_gemm(const uint8_t* x_t, const float* q_t, const uint8_t* w_t,
                                 const void* w_tiled,
                                 const void* scale, int64_t M, int64_t K, int64_t N,
                                 const PrefillLayout& L, int64_t g_begin, int64_t g_end, void* y,
                                 int32_t* y_int, hipStream_t stream);

// The fused decode kernel (M <= 4): steps 1-11 in one launch.  A K-split
// (K > 4096) hands its partials off through `accum` (int64 per output; zero
// before the first launch, re-armed by the kernel).
struct DecodePlan {
  int shape;            // workgroup shape (one shape: 0)
  int64_t cols;         // columns per workgroup
  int64_t col_blocks;   // column blocks
  int64_t splits;       // K-slices per column block (<= 32)
  int64_t nch;          // row chunks per K-slice
  int64_t kb_begin;     // first 128-row block of the group range
};
DecodePlan decode_plan(int gs, int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end);
size_t decode_accum_bytes(const DecodePlan& p, int64_t M, int64_t N);

hipError_t launch_decode(const void* x, const void* w, const void* scale, int gs, int64_t M,
                         int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                         int32_t* y_int, uint64_t* accum, const DecodePlan& plan, hipStream_t stream);

// Decode for 4 < M <= 96 (msd_decode_gemv.hip): an operand kernel decomposes
// x once into int4-packed level operands (slices of 16 rows) and level
// weights in `ws` (decode_gemv_workspace_bytes), then a contraction kernel
// covers all of K per 16-column tile (no K-split hand-off).  stage 0: both
// kernels; 1: the operand kernel only; 2: the contraction only, on the
// operands in `ws`.
size_t decode_gemv_workspace_bytes(int gs, int64_t M, int64_t K);
hipError_t launch_decode_gemv(const void* x, const void* w, const void* scale, int gs, int64_t M,
                              int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                              int32_t* y_int, uint8_t* ws, int stage, hipStream_t stream);

// Zero n 32-bit words (a kernel, not a memset).
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream);

}  // namespace wqbmm
