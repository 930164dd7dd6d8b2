// msd_api.cpp -- host side of the C ABI declared in include/wqbmm.h:
// argument validation, kernel-path dispatch and the library-owned workspace.
//
// Operator: the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4 PerGroup
// 伪量化 MatMul 的 MSD 算法与双模板流水设计" (lpnh.cn/news/2294145), §4.1-§4.2.
// Its host tiling rejects anything but 2-D fp16 x / int4 weight / fp16 y
// (§4.2, last sentence); the dtypes here are fixed by the entry points and the
// shape rules are checked before any device call, in the order null pointer ->
// shape -> support, like the aclnn parameter checks (nullptr, then invalid
// shape, then unsupported product) described on the page "CANN
// ops-math：aclnnCalculateMatmulWeightSizeV2 接口详解" (zskr.cn/news/2299903),
// section 返回值说明.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/wqbmm.h"
#include "msd_launch.hpp"

namespace {

using wqbmm::DecodePlan;

constexpr int64_t kMaxM = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxN = int64_t(1) << 20;
constexpr int kDecodeMaxM = 16;

// NULL counts as aligned: it is only accepted where the array is empty (M == 0).
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

wqbmm_status check_shape(int64_t gs, int64_t M, int64_t K, int64_t N) {
  if (gs <= 0 || M < 0 || K <= 0 || N <= 0) return WQBMM_ERR_INVALID;
  if (M > kMaxM || K > kMaxK || N > kMaxN) return WQBMM_ERR_INVALID;
  if (K % gs != 0 || N % 32 != 0) return WQBMM_ERR_INVALID;
  return WQBMM_OK;
}

wqbmm_status check_support(int64_t gs) {
  return (gs == 64 || gs == 128) ? WQBMM_OK : WQBMM_ERR_UNSUPPORTED;
}

// ---- device check (gfx950 only), cached per device
std::mutex g_mu;
std::map<int, bool> g_arch_ok;

wqbmm_status check_device(int* dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return WQBMM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_arch_ok.find(dev);
  if (it == g_arch_ok.end()) {
    hipDeviceProp_t prop;
    bool ok = false;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
      ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    it = g_arch_ok.emplace(dev, ok).first;
  }
  *dev_out = dev;
  return it->second ? WQBMM_OK : WQBMM_ERR_UNSUPPORTED;
}

// ---- per-(device, stream) workspace, grown on demand
// Layout: [decode accumulators][scratch].  The decode accumulators must be
// zero before a decode launch; the kernel re-arms every element it uses, and
// no other kernel writes that region, so it is zeroed only when allocated.
// The scratch region holds the prefill operand tiles.
struct Workspace {
  void* base = nullptr;
  size_t acc_bytes = 0;
  size_t scratch_bytes = 0;
  // path and shape whose operands the scratch region currently holds
  // (prep_path 0: none, WQBMM_PATH_DECODE or WQBMM_PATH_PREFILL)
  int prep_path = 0;
  int64_t prep_gs = 0, prep_m = -1, prep_k = 0, prep_n = 0;
};
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Returns an accumulator region of at least `acc` bytes (zeroed) and a
// scratch region of at least `scratch` bytes for launches on `stream`.
// Growth synchronizes `stream` so that no launch still using the old buffer
// is pending before it is freed; a new buffer gets its accumulator region
// zeroed by a kernel enqueued on `stream`.
wqbmm_status get_workspace(int dev, hipStream_t stream, size_t acc, size_t scratch,
                           uint64_t** acc_out, uint8_t** scratch_out) {
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& ws = g_ws[std::make_pair(dev, stream)];
  acc = round_up(acc, 256);
  scratch = round_up(scratch, 256);
  if (ws.acc_bytes < acc || ws.scratch_bytes < scratch || !ws.base) {
    const size_t new_acc = std::max(ws.acc_bytes, acc + acc / 4);
    const size_t new_scratch = std::max(ws.scratch_bytes, scratch + scratch / 4);
    if (ws.base) {
      if (hipStreamSynchronize(stream) != hipSuccess) return WQBMM_ERR_LAUNCH;
      (void)hipFree(ws.base);
      ws.base = nullptr;
      ws.acc_bytes = ws.scratch_bytes = 0;
    }
    void* p = nullptr;
    const size_t total = round_up(new_acc, 256) + round_up(new_scratch, 256) + 256;
    if (hipMalloc(&p, total) != hipSuccess) return WQBMM_ERR_ALLOC;
    if (wqbmm::launch_zero_words(static_cast<uint32_t*>(p), (int64_t)(round_up(new_acc, 256) / 4),
                                 stream) != hipSuccess) {
      (void)hipFree(p);
      return WQBMM_ERR_LAUNCH;
    }
    ws.base = p;
    ws.acc_bytes = round_up(new_acc, 256);
    ws.scratch_bytes = round_up(new_scratch, 256);
    ws.prep_path = 0;
  }
  *acc_out = static_cast<uint64_t*>(ws.base);
  *scratch_out = static_cast<uint8_t*>(ws.base) + ws.acc_bytes;
  return WQBMM_OK;
}

int resolve_path(int path, int64_t M, int64_t K, int64_t N, int64_t gs) {
  if (path == WQBMM_PATH_AUTO) return wqbmm_select_path(M, K, N, gs);
  return path;
}

wqbmm_status launch_status(hipError_t e) { return e == hipSuccess ? WQBMM_OK : WQBMM_ERR_LAUNCH; }

// Records (stage 0 or 1) or checks (stage 2) which path and shape the
// operands in the scratch region of (dev, stream) belong to.
wqbmm_status track_operands(int dev, hipStream_t stream, int path, int stage, int64_t gs, int64_t M,
                            int64_t K, int64_t N) {
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& ws = g_ws[std::make_pair(dev, stream)];
  if (stage == 2)
    return (ws.prep_path == path && ws.prep_gs == gs && ws.prep_m == M && ws.prep_k == K && ws.prep_n == N)
               ? WQBMM_OK : WQBMM_ERR_INVALID;
  ws.prep_path = path;
  ws.prep_gs = gs; ws.prep_m = M; ws.prep_k = K; ws.prep_n = N;
  return WQBMM_OK;
}

wqbmm_status run_prefill(int dev, const void* x, const void* w, const void* scale, int64_t gs,
                         int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                         int32_t* y_int, int stage, hipStream_t stream);

// The decode path.  M <= 4: one fused kernel (stage 1 launches nothing);
// 4 < M <= 16: the operand kernel (stage 1) and the contraction (stage 2).
wqbmm_status run_decode(int dev, const void* x, const void* w, const void* scale, int64_t gs,
                        int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                        int32_t* y_int, int stage, hipStream_t stream) {
  uint64_t* accum = nullptr;
  uint8_t* scratch = nullptr;
  wqbmm_status st;
  if (M > 4) {
    st = get_workspace(dev, stream, 0, wqbmm::decode_gemv_workspace_bytes((int)gs, K), &accum, &scratch);
    if (st != WQBMM_OK) return st;
    st = track_operands(dev, stream, WQBMM_PATH_DECODE, stage, gs, M, K, N);
    if (st != WQBMM_OK) return st;
    return launch_status(wqbmm::launch_decode_gemv(x, w, scale, (int)gs, M, K, N, g_begin, g_end, y,
                                                   y_int, scratch, stage, stream));
  }
  if (stage == 1) return WQBMM_OK;
  const DecodePlan plan = wqbmm::decode_plan((int)gs, M, K, N, g_begin, g_end);
  const size_t abytes = y_int ? 0 : wqbmm::decode_accum_bytes(plan, M, N);
  if (abytes) {
    st = get_workspace(dev, stream, abytes, 0, &accum, &scratch);
    if (st != WQBMM_OK) return st;
  }
  return launch_status(wqbmm::launch_decode(x, w, scale, (int)gs, M, K, N, g_begin, g_end, y,
                                            y_int, accum, plan, stream));
}

// Steps 1-11 (or 1-9 with y_int) on one of the two kernel paths.
wqbmm_status run(const void* x, const void* w, const void* scale, int64_t gs, int64_t M,
                 int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y, int32_t* y_int,
                 int path, hipStream_t stream) {
  int dev = -1;
  wqbmm_status st = check_device(&dev);
  if (st != WQBMM_OK) return st;
  if (path == WQBMM_PATH_DECODE)
    return run_decode(dev, x, w, scale, gs, M, K, N, g_begin, g_end, y, y_int, 0, stream);
  // prefill: operand preparation into the workspace, then the MFMA GEMM
  return run_prefill(dev, x, w, scale, gs, M, K, N, g_begin, g_end, y, y_int, 0, stream);
}

// The prefill path.  stage 0: both kernels; 1: preparation only; 2: GEMM only,
// on the operands a previous stage 0/1 call left in this stream's workspace
// for the same shape (checked).
wqbmm_status run_prefill(int dev, const void* x, const void* w, const void* scale, int64_t gs,
                         int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                         int32_t* y_int, int stage, hipStream_t stream) {
  const wqbmm::PrefillLayout L = wqbmm::prefill_layout((int)gs, M, K, N);
  const size_t a_off = 0;
  const size_t q_off = round_up(L.a_bytes, 256);
  const size_t b_off = q_off + round_up(L.q_bytes, 256);
  const size_t total = b_off + round_up(L.b_bytes, 256);
  uint64_t* accum = nullptr;
  uint8_t* scratch = nullptr;
  wqbmm_status st = get_workspace(dev, stream, 0, total, &accum, &scratch);
  if (st != WQBMM_OK) return st;
  uint8_t* a_t = scratch + a_off;
  float* q_t = reinterpret_cast<float*>(scratch + q_off);
  uint8_t* b_t = scratch + b_off;
  st = track_operands(dev, stream, WQBMM_PATH_PREFILL, stage, gs, M, K, N);
  if (st != WQBMM_OK) return st;
  if (stage != 2) {
    st = launch_status(wqbmm::launch_prefill_prep(x, w, (int)gs, M, K, N, L, a_t, q_t, b_t, stream));
    if (st != WQBMM_OK || stage == 1) return st;
  }
  return launch_status(wqbmm::launch_prefill_gemm(a_t, q_t, b_t, w, scale, (int)gs, M, K, N, L,
                                                  g_begin, g_end, y, y_int, stream));
}

}  // namespace

extern "C" {

int wqbmm_select_path(int64_t M, int64_t K, int64_t N, int64_t group_size) {
  (void)K; (void)N; (void)group_size;
  return M <= kDecodeMaxM ? WQBMM_PATH_DECODE : WQBMM_PATH_PREFILL;
}

const char* wqbmm_status_string(int status) {
  switch (status) {
    case WQBMM_OK: return "WQBMM_OK";
    case WQBMM_ERR_NULLPTR: return "WQBMM_ERR_NULLPTR: a required pointer is NULL";
    case WQBMM_ERR_INVALID: return "WQBMM_ERR_INVALID: shape, range or alignment rule violated";
    case WQBMM_ERR_UNSUPPORTED: return "WQBMM_ERR_UNSUPPORTED: group_size not 64/128 or device not gfx950";
    case WQBMM_ERR_LAUNCH: return "WQBMM_ERR_LAUNCH: a HIP call or kernel launch failed";
    case WQBMM_ERR_ALLOC: return "WQBMM_ERR_ALLOC: workspace allocation failed";
    default: return "WQBMM_ERR_UNKNOWN: not a wqbmm_status value";
  }
}

int wqbmm_version(void) { return 1 * 10000 + 1 * 100 + 0; }

int64_t wqbmm_a16w4_tiled_weight_bytes(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0 || K > kMaxK || N > kMaxN || N % 32 != 0) return -1;
  return (int64_t)wqbmm::tiled_weight_bytes(K, N);
}

wqbmm_status wqbmm_a16w4_tile_weights(const void* w_nd, int64_t K, int64_t N, void* w_tiled,
                                      void* stream) {
  if (!w_nd || !w_tiled) return WQBMM_ERR_NULLPTR;
  if (K <= 0 || N <= 0 || K > kMaxK || N > kMaxN || N % 32 != 0) return WQBMM_ERR_INVALID;
  if (!aligned16(w_nd) || !aligned16(w_tiled)) return WQBMM_ERR_INVALID;
  int dev = -1;
  wqbmm_status st = check_device(&dev);
  if (st != WQBMM_OK) return st;
  return launch_status(wqbmm::launch_prepack(w_nd, K, N, w_tiled, static_cast<hipStream_t>(stream)));
}

wqbmm_status wqbmm_a16w4_msd_path(const void* x, const void* w_tiled,
                                  const void* antiquant_scale, int64_t group_size, int64_t M,
                                  int64_t K, int64_t N, void* y, int path, void* stream) {
  // x and y have no elements when M == 0 and may then be NULL
  if ((!x && M != 0) || !w_tiled || !antiquant_scale || (!y && M != 0))
    return WQBMM_ERR_NULLPTR;
  wqbmm_status st = check_shape(group_size, M, K, N);
  if (st != WQBMM_OK) return st;
  if (!aligned16(x) || !aligned16(w_tiled) || !aligned16(antiquant_scale) || !aligned16(y))
    return WQBMM_ERR_INVALID;
  if (path < WQBMM_PATH_AUTO || path > WQBMM_PATH_PREFILL) return WQBMM_ERR_INVALID;
  const int p = resolve_path(path, M, K, N, group_size);
  if (p == WQBMM_PATH_DECODE && M > kDecodeMaxM) return WQBMM_ERR_INVALID;
  st = check_support(group_size);
  if (st != WQBMM_OK) return st;
  if (M == 0) return WQBMM_OK;
  return run(x, w_tiled, antiquant_scale, group_size, M, K, N, 0, K / group_size, y,
             nullptr, p, static_cast<hipStream_t>(stream));
}

wqbmm_status wqbmm_a16w4_msd(const void* x, const void* w_tiled,
                             const void* antiquant_scale, int64_t group_size, int64_t M,
                             int64_t K, int64_t N, void* y, void* stream) {
  return wqbmm_a16w4_msd_path(x, w_tiled, antiquant_scale, group_size, M, K, N, y,
                              WQBMM_PATH_AUTO, stream);
}

wqbmm_status wqbmm_a16w4_msd_prepass(const void* x, int64_t group_size, int64_t M, int64_t K,
                                     int8_t* a_int, float* a_max, void* stream) {
  if (M != 0 && (!x || !a_int || !a_max)) return WQBMM_ERR_NULLPTR;
  wqbmm_status st = check_shape(group_size, M, K, 32);
  if (st != WQBMM_OK) return st;
  if (!aligned16(x) || !aligned16(a_int) || !aligned16(a_max)) return WQBMM_ERR_INVALID;
  st = check_support(group_size);
  if (st != WQBMM_OK) return st;
  if (M == 0) return WQBMM_OK;
  int dev = -1;
  st = check_device(&dev);
  if (st != WQBMM_OK) return st;
  return launch_status(wqbmm::launch_prepass(x, (int)group_size, M, K, a_int, a_max,
                                             static_cast<hipStream_t>(stream)));
}

wqbmm_status wqbmm_a16w4_msd_yint(const void* x, const void* w_tiled, int64_t group_size,
                                  int64_t M, int64_t K, int64_t N, int64_t g_begin,
                                  int64_t g_end, int32_t* y_int, int path, void* stream) {
  if ((!x && M != 0) || !w_tiled || (!y_int && M != 0)) return WQBMM_ERR_NULLPTR;
  wqbmm_status st = check_shape(group_size, M, K, N);
  if (st != WQBMM_OK) return st;
  if (!aligned16(x) || !aligned16(w_tiled) || !aligned16(y_int)) return WQBMM_ERR_INVALID;
  if (g_begin < 0 || g_end > K / group_size || g_begin >= g_end) return WQBMM_ERR_INVALID;
  if (path < WQBMM_PATH_AUTO || path > WQBMM_PATH_PREFILL) return WQBMM_ERR_INVALID;
  const int p = resolve_path(path, M, K, N, group_size);
  if (p == WQBMM_PATH_DECODE && M > kDecodeMaxM) return WQBMM_ERR_INVALID;
  st = check_support(group_size);
  if (st != WQBMM_OK) return st;
  if (M == 0) return WQBMM_OK;
  return run(x, w_tiled, nullptr, group_size, M, K, N, g_begin, g_end, nullptr, y_int, p,
             static_cast<hipStream_t>(stream));
}

wqbmm_status wqbmm_a16w4_msd_profile_stage(const void* x, const void* w_tiled,
                                           const void* antiquant_scale, int64_t group_size,
                                           int64_t M, int64_t K, int64_t N, void* y, int path,
                                           int stage, void* stream) {
  if ((!x && M != 0) || !w_tiled || !antiquant_scale || (!y && M != 0))
    return WQBMM_ERR_NULLPTR;
  wqbmm_status st = check_shape(group_size, M, K, N);
  if (st != WQBMM_OK) return st;
  if (!aligned16(x) || !aligned16(w_tiled) || !aligned16(antiquant_scale) || !aligned16(y))
    return WQBMM_ERR_INVALID;
  if (stage < 1 || stage > 2) return WQBMM_ERR_INVALID;
  if (path < WQBMM_PATH_AUTO || path > WQBMM_PATH_PREFILL) return WQBMM_ERR_INVALID;
  const int p = resolve_path(path, M, K, N, group_size);
  if (p == WQBMM_PATH_DECODE && M > kDecodeMaxM) return WQBMM_ERR_INVALID;
  st = check_support(group_size);
  if (st != WQBMM_OK) return st;
  if (M == 0) return WQBMM_OK;
  int dev = -1;
  st = check_device(&dev);
  if (st != WQBMM_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p == WQBMM_PATH_DECODE)
    return run_decode(dev, x, w_tiled, antiquant_scale, group_size, M, K, N, 0, K / group_size, y,
                      nullptr, stage, s);
  return run_prefill(dev, x, w_tiled, antiquant_scale, group_size, M, K, N, 0, K / group_size, y,
                     nullptr, stage, s);
}

}  // extern "C"
