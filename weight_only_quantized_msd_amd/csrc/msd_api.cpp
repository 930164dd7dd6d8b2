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
#include <vector>

#include "../../include/wqbmm.h"
#include "msd_launch.hpp"

namespace {

using wqbmm::DecodePlan;

constexpr int64_t kMaxM = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxN = int64_t(1) << 20;
constexpr int kDecodeMaxM = 96;

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

// ---- device check (gfx950 only), cached per device in a fixed table
constexpr int kMaxDevices = 64;
std::mutex g_mu;
int g_arch[kMaxDevices];   // 0: not checked yet, 1: gfx950, 2: another device

wqbmm_status check_device(int* dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WQBMM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_arch[dev] == 0) {
    hipDeviceProp_t prop;
    bool ok = false;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
      ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_arch[dev] = ok ? 1 : 2;
  }
  *dev_out = dev;
  return g_arch[dev] == 1 ? WQBMM_OK : WQBMM_ERR_UNSUPPORTED;
}

// ---- scratch memory of one call
// A call's kernels use up to two regions beside its inputs and outputs:
//   acc: the split-K accumulators of the fused decode kernel (M <= 4 with K
//        split over workgroups).  They must be zero before a launch; every
//        launch that completes leaves the elements it used at zero again, and
//        no other kernel writes this region, so it is zeroed once, when the
//        memory is first handed out;
//   ops: the operands that the two-kernel paths pass from their operand
//        kernel to their contraction kernel (decode at 4 < M <= 16, prefill).
struct Buffers {
  uint64_t* acc = nullptr;
  size_t acc_bytes = 0;
  uint8_t* ops = nullptr;
  size_t ops_bytes = 0;
};

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Bytes of each region a call needs.
struct Needs {
  size_t acc = 0;
  size_t ops = 0;
};

// The group-128 prefill path reads the weights' operand form instead of
// converting the tiled weights when the caller passes it.
bool uses_operand_weights(int path, int64_t gs, const void* w_op) {
  return w_op != nullptr && path == WQBMM_PATH_PREFILL && gs == 128;
}

size_t prefill_ops_bytes(const wqbmm::PrefillLayout& L, bool own_weight_tiles) {
  return round_up(L.a_bytes, 256) + round_up(L.q_bytes, 256) +
         (own_weight_tiles ? round_up(L.b_bytes, 256) : 0) + round_up(L.part_bytes, 256);
}

Needs needs_of(int path, int64_t gs, int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end,
               bool yint, bool operand_weights) {
  Needs n;
  if (path == WQBMM_PATH_DECODE) {
    if (M > 4) {
      n.ops = wqbmm::decode_gemv_workspace_bytes((int)gs, M, K);
    } else if (!yint) {
      n.acc = wqbmm::decode_accum_bytes(wqbmm::decode_plan((int)gs, M, K, N, g_begin, g_end), M, N);
    }
  } else {
    n.ops = prefill_ops_bytes(wqbmm::prefill_layout((int)gs, M, K, N), !operand_weights);
  }
  n.acc = round_up(n.acc, 256);
  n.ops = round_up(n.ops, 256);
  return n;
}

// Whether `stream` is being captured into a graph (an invalidated capture
// counts as one).  False with *err set if the query fails.
bool capturing(hipStream_t stream, wqbmm_status* err) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    *err = WQBMM_ERR_LAUNCH;
    return false;
  }
  *err = WQBMM_OK;
  return cs != hipStreamCaptureStatusNone;
}

// ---- per-(device, stream) workspace of wqbmm_a16w4_msd and friends
// Grown on demand, never while the stream is being captured (a captured graph
// would hold the growth's allocation and zeroing only inside the graph), and
// never freed: a buffer that a larger one replaces is retired but stays
// allocated until the process ends, because a graph captured earlier may
// still replay kernels that use it, and because freeing it would have to wait
// for the stream.  Sizes at least double on growth, so the retired buffers
// of a stream add up to less than its current one.  The accumulator region
// of a new buffer is zeroed by a kernel on the stream, ahead of the call's
// own kernels; nothing synchronizes the host.
struct Workspace {
  void* base = nullptr;
  size_t acc_bytes = 0;
  size_t ops_bytes = 0;
  // path and shape whose operands the ops region currently holds
  // (prep_path 0: none, WQBMM_PATH_DECODE or WQBMM_PATH_PREFILL)
  int prep_path = 0;
  int64_t prep_gs = 0, prep_m = -1, prep_k = 0, prep_n = 0;
  bool prep_opw = false;
};
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<void*> g_retired;

size_t grown(size_t have, size_t need) {
  if (need <= have) return have;
  return std::max(need + need / 4, 2 * have);
}

wqbmm_status get_workspace(int dev, hipStream_t stream, const Needs& need, Buffers* out) {
  if (need.acc == 0 && need.ops == 0) {   // e.g. the fused decode kernel without a K split
    *out = Buffers{};
    return WQBMM_OK;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& ws = g_ws[std::make_pair(dev, stream)];
  if (!ws.base || ws.acc_bytes < need.acc || ws.ops_bytes < need.ops) {
    wqbmm_status st;
    if (capturing(stream, &st)) return WQBMM_ERR_CAPTURE;
    if (st != WQBMM_OK) return st;
    const size_t acc = round_up(grown(ws.acc_bytes, need.acc), 256);
    const size_t ops = round_up(grown(ws.ops_bytes, need.ops), 256);
    void* p = nullptr;
    if (hipMalloc(&p, acc + ops + 256) != hipSuccess) return WQBMM_ERR_ALLOC;
    if (wqbmm::launch_zero_words(static_cast<uint32_t*>(p), (int64_t)(acc / 4), stream) != hipSuccess) {
      g_retired.push_back(p);
      return WQBMM_ERR_LAUNCH;
    }
    if (ws.base) g_retired.push_back(ws.base);
    ws.base = p;
    ws.acc_bytes = acc;
    ws.ops_bytes = ops;
    ws.prep_path = 0;
  }
  out->acc = static_cast<uint64_t*>(ws.base);
  out->acc_bytes = ws.acc_bytes;
  out->ops = static_cast<uint8_t*>(ws.base) + ws.acc_bytes;
  out->ops_bytes = ws.ops_bytes;
  return WQBMM_OK;
}

}  // namespace

// ---- scratch of the allocation-free entry point (wqbmm_a16w4_msd_noalloc)
// One fixed array per device, loaded with the library: the first 2 MiB hold
// the fused decode kernel's split-K accumulators (zeroed at set-up, left zero
// by every completed launch), the rest the two-kernel paths' operands.  In
// host code `scratch` only names the array's host-side stand-in; its device
// address on the current device comes from hipGetSymbolAddress, once per
// device, and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr size_t kScratchAccBytes = size_t(2) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

uint8_t* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (null: not set up)

// The scratch of device `dev`, set up on its first use: the symbol's device
// address, and a kernel on `stream` that zeroes the accumulator region.  The
// set-up is refused while `stream` is being captured (the zeroing would exist
// only inside the graph).  WQBMM_ERR_TOO_LARGE if the call needs more than
// the array holds.
wqbmm_status scratch_buffers(int dev, hipStream_t stream, const Needs& need, Buffers* out) {
  if (need.acc > kScratchAccBytes || need.ops > kScratchBytes - kScratchAccBytes)
    return WQBMM_ERR_TOO_LARGE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    wqbmm_status st;
    if (capturing(stream, &st)) return WQBMM_ERR_CAPTURE;
    if (st != WQBMM_OK) return st;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WQBMM_ERR_LAUNCH;
    if (wqbmm::launch_zero_words(static_cast<uint32_t*>(p), (int64_t)(kScratchAccBytes / 4), stream) !=
        hipSuccess)
      return WQBMM_ERR_LAUNCH;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  out->acc = reinterpret_cast<uint64_t*>(g_scratch_ptr[dev]);
  out->acc_bytes = kScratchAccBytes;
  out->ops = g_scratch_ptr[dev] + kScratchAccBytes;
  out->ops_bytes = kScratchBytes - kScratchAccBytes;
  return WQBMM_OK;
}

int resolve_path(int path, int64_t M, int64_t K, int64_t N, int64_t gs) {
  if (path == WQBMM_PATH_AUTO) return wqbmm_select_path(M, K, N, gs);
  return path;
}

wqbmm_status launch_status(hipError_t e) { return e == hipSuccess ? WQBMM_OK : WQBMM_ERR_LAUNCH; }

// Records (stage 0 or 1) or checks (stage 2) which path and shape the
// operands in the ops region of (dev, stream) belong to, and whether the
// weights' operand form stood in for the weight tiles.
wqbmm_status track_operands(int dev, hipStream_t stream, int path, int stage, int64_t gs, int64_t M,
                            int64_t K, int64_t N, bool opw) {
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& ws = g_ws[std::make_pair(dev, stream)];
  if (stage == 2)
    return (ws.prep_path == path && ws.prep_gs == gs && ws.prep_m == M && ws.prep_k == K &&
            ws.prep_n == N && ws.prep_opw == opw)
               ? WQBMM_OK : WQBMM_ERR_INVALID;
  ws.prep_path = path;
  ws.prep_gs = gs; ws.prep_m = M; ws.prep_k = K; ws.prep_n = N;
  ws.prep_opw = opw;
  return WQBMM_OK;
}

// The decode path.  M <= 4: one fused kernel (stage 1 launches nothing);
// 4 < M <= 16: the operand kernel (stage 1) and the contraction (stage 2).
// `b` holds at least needs_of(...) bytes in each region.
wqbmm_status run_decode(const Buffers& b, const void* x, const void* w, const void* scale, int64_t gs,
                        int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                        int32_t* y_int, int stage, hipStream_t stream) {
  if (M > 4)
    return launch_status(wqbmm::launch_decode_gemv(x, w, scale, (int)gs, M, K, N, g_begin, g_end, y,
                                                   y_int, b.ops, stage, stream));
  if (stage == 1) return WQBMM_OK;
  const DecodePlan plan = wqbmm::decode_plan((int)gs, M, K, N, g_begin, g_end);
  return launch_status(wqbmm::launch_decode(x, w, scale, (int)gs, M, K, N, g_begin, g_end, y,
                                            y_int, b.acc, plan, stream));
}

// The prefill path.  stage 0: both kernels; 1: preparation only; 2: GEMM only.
// With the weights' operand form (w_op, group size 128) the GEMM reads its
// weight tiles there and the preparation kernel converts only x.
wqbmm_status run_prefill(const Buffers& b, const void* x, const void* w, const void* w_op,
                         const void* scale, int64_t gs, int64_t M, int64_t K, int64_t N,
                         int64_t g_begin, int64_t g_end, void* y, int32_t* y_int, int stage,
                         hipStream_t stream) {
  const wqbmm::PrefillLayout L = wqbmm::prefill_layout((int)gs, M, K, N);
  const bool opw = uses_operand_weights(WQBMM_PATH_PREFILL, gs, w_op);
  uint8_t* a_t = b.ops;
  float* q_t = reinterpret_cast<float*>(b.ops + round_up(L.a_bytes, 256));
  uint8_t* own_b = b.ops + round_up(L.a_bytes, 256) + round_up(L.q_bytes, 256);
  float* part = reinterpret_cast<float*>(own_b + (opw ? 0 : round_up(L.b_bytes, 256)));
  uint8_t* b_t = opw ? static_cast<uint8_t*>(const_cast<void*>(w_op)) : own_b;
  if (stage != 2) {
    const wqbmm_status st = launch_status(
        wqbmm::launch_prefill_prep(x, w, (int)gs, M, K, N, L, a_t, q_t, b_t, !opw, stream));
    if (st != WQBMM_OK || stage == 1) return st;
  }
  return launch_status(wqbmm::launch_prefill_gemm(a_t, q_t, b_t, w, scale, (int)gs, M, K, N, L,
                                                  g_begin, g_end, y, y_int, part, stream));
}

wqbmm_status run_path(const Buffers& b, int path, const void* x, const void* w, const void* w_op,
                      const void* scale, int64_t gs, int64_t M, int64_t K, int64_t N,
                      int64_t g_begin, int64_t g_end, void* y, int32_t* y_int, int stage,
                      hipStream_t stream) {
  if (path == WQBMM_PATH_DECODE)
    return run_decode(b, x, w, scale, gs, M, K, N, g_begin, g_end, y, y_int, stage, stream);
  return run_prefill(b, x, w, w_op, scale, gs, M, K, N, g_begin, g_end, y, y_int, stage, stream);
}

// Steps 1-11 (or 1-9 with y_int) on one of the two kernel paths, with this
// stream's workspace.  Stages as in wqbmm_a16w4_msd_profile_stage (0: all).
wqbmm_status run(const void* x, const void* w, const void* w_op, const void* scale, int64_t gs,
                 int64_t M, int64_t K, int64_t N, int64_t g_begin, int64_t g_end, void* y,
                 int32_t* y_int, int path, int stage, hipStream_t stream) {
  int dev = -1;
  wqbmm_status st = check_device(&dev);
  if (st != WQBMM_OK) return st;
  const bool opw = uses_operand_weights(path, gs, w_op);
  Buffers b;
  st = get_workspace(dev, stream, needs_of(path, gs, M, K, N, g_begin, g_end, y_int != nullptr, opw), &b);
  if (st != WQBMM_OK) return st;
  const bool two_kernels = path == WQBMM_PATH_PREFILL || M > 4;
  if (two_kernels) {
    st = track_operands(dev, stream, path, stage, gs, M, K, N, opw);
    if (st != WQBMM_OK) return st;
  }
  return run_path(b, path, x, w, w_op, scale, gs, M, K, N, g_begin, g_end, y, y_int, stage, stream);
}

}  // namespace

extern "C" {

// The split between the two kernel paths, from sweeps of both paths over M
// (MALL-cold step time, one MI355X; the group-128 prefill path with the
// weights' operand form).  The decode contraction's cost grows with the row
// slices (every column tile reads every slice's level chunks) times the
// rounds of column tiles; the prefill path's stays about flat up to one
// 128-row block:
//   K = N = 4096, group size 128: decode 7.6 / 9.8 / 11.9 / 13.3 / 15.9 /
//     17.5 us at M = 16 / 32 / 48 / 64 / 80 / 96 against prefill 16-21 us;
//   K = 4096, N = 11008: decode 16.7 / 21.7 / 29.2 / 35.2 us at M = 32 / 48 /
//     64 / 80 against prefill 31-32 us;
//   K = 4096, N = 14336 and K = N = 8192: decode 26-27 us at M = 48, 35-37 us
//     at 64, against prefill 31-32 us;
//   K = 8192, N = 28672, group size 64: decode 41 / 63 / 85 / 128 us at M =
//     16 / 32 / 48 / 64 against prefill 110-111 us.
// Decode up to 48 rows everywhere; at group size 128 up to 96 rows for at
// most 2^24 weights and up to 64 for at most 3 * 2^24.
int wqbmm_select_path(int64_t M, int64_t K, int64_t N, int64_t group_size) {
  if (M <= 48) return WQBMM_PATH_DECODE;
  if (group_size == 128) {
    const int64_t weights = K * N;
    if (M <= 96 && weights <= (int64_t(1) << 24)) return WQBMM_PATH_DECODE;
    if (M <= 64 && weights <= 3 * (int64_t(1) << 24)) return WQBMM_PATH_DECODE;
  }
  return WQBMM_PATH_PREFILL;
}

const char* wqbmm_status_string(int status) {
  switch (status) {
    case WQBMM_OK: return "WQBMM_OK";
    case WQBMM_ERR_NULLPTR: return "WQBMM_ERR_NULLPTR: a required pointer is NULL";
    case WQBMM_ERR_INVALID: return "WQBMM_ERR_INVALID: shape, range or alignment rule violated";
    case WQBMM_ERR_UNSUPPORTED: return "WQBMM_ERR_UNSUPPORTED: group_size not 64/128 or device not gfx950";
    case WQBMM_ERR_LAUNCH: return "WQBMM_ERR_LAUNCH: a HIP call or kernel launch failed";
    case WQBMM_ERR_ALLOC: return "WQBMM_ERR_ALLOC: workspace allocation failed";
    case WQBMM_ERR_TOO_LARGE:
      return "WQBMM_ERR_TOO_LARGE: the shape needs more than the allocation-free entry point's "
             "fixed scratch (2 MiB of accumulators, 62 MiB of operands)";
    case WQBMM_ERR_CAPTURE:
      return "WQBMM_ERR_CAPTURE: the stream's workspace would have to grow while the stream is "
             "captured into a graph (make one eager call of the largest shape on it first)";
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

}  // extern "C"

namespace {

// Host validation shared by the operator entry points, in the order null
// pointer -> shape -> support.  `scale`/`y` are checked only when the entry
// point takes them (y_int stands in for y where Y_int is exported).  On
// success *p_out is the resolved kernel path.
wqbmm_status validate_call(const void* x, const void* w_tiled, const void* scale, bool takes_scale,
                           const void* y, int64_t gs, int64_t M, int64_t K, int64_t N, int path,
                           int* p_out) {
  // x and y have no elements when M == 0 and may then be NULL
  if ((!x && M != 0) || !w_tiled || (takes_scale && !scale) || (!y && M != 0))
    return WQBMM_ERR_NULLPTR;
  wqbmm_status st = check_shape(gs, M, K, N);
  if (st != WQBMM_OK) return st;
  if (!aligned16(x) || !aligned16(w_tiled) || (takes_scale && !aligned16(scale)) || !aligned16(y))
    return WQBMM_ERR_INVALID;
  if (path < WQBMM_PATH_AUTO || path > WQBMM_PATH_PREFILL) return WQBMM_ERR_INVALID;
  const int p = resolve_path(path, M, K, N, gs);
  if (p == WQBMM_PATH_DECODE && M > kDecodeMaxM) return WQBMM_ERR_INVALID;
  st = check_support(gs);
  if (st != WQBMM_OK) return st;
  *p_out = p;
  return WQBMM_OK;
}

}  // namespace

extern "C" {

wqbmm_status wqbmm_a16w4_msd_ex(const void* x, const void* w_tiled, const void* w_operand,
                                const void* antiquant_scale, int64_t group_size, int64_t M,
                                int64_t K, int64_t N, void* y, int path, void* stream) {
  int p = 0;
  const wqbmm_status st = validate_call(x, w_tiled, antiquant_scale, true, y, group_size, M, K, N, path, &p);
  if (st != WQBMM_OK) return st;
  if (!aligned16(w_operand)) return WQBMM_ERR_INVALID;
  if (M == 0) return WQBMM_OK;
  return run(x, w_tiled, w_operand, antiquant_scale, group_size, M, K, N, 0, K / group_size, y,
             nullptr, p, 0, static_cast<hipStream_t>(stream));
}

wqbmm_status wqbmm_a16w4_msd_path(const void* x, const void* w_tiled,
                                  const void* antiquant_scale, int64_t group_size, int64_t M,
                                  int64_t K, int64_t N, void* y, int path, void* stream) {
  return wqbmm_a16w4_msd_ex(x, w_tiled, nullptr, antiquant_scale, group_size, M, K, N, y, path,
                            stream);
}

int64_t wqbmm_a16w4_operand_weight_bytes(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0 || K > kMaxK || N > kMaxN || N % 32 != 0) return -1;
  return (int64_t)wqbmm::operand_weight_bytes(K, N);
}

wqbmm_status wqbmm_a16w4_operand_weights(const void* w_tiled, int64_t K, int64_t N, void* w_operand,
                                         void* stream) {
  if (!w_tiled || !w_operand) return WQBMM_ERR_NULLPTR;
  if (K <= 0 || N <= 0 || K > kMaxK || N > kMaxN || N % 32 != 0) return WQBMM_ERR_INVALID;
  if (!aligned16(w_tiled) || !aligned16(w_operand)) return WQBMM_ERR_INVALID;
  int dev = -1;
  wqbmm_status st = check_device(&dev);
  if (st != WQBMM_OK) return st;
  return launch_status(wqbmm::launch_operand_weights(w_tiled, K, N, static_cast<uint8_t*>(w_operand),
                                                     static_cast<hipStream_t>(stream)));
}

wqbmm_status wqbmm_a16w4_msd(const void* x, const void* w_tiled,
                             const void* antiquant_scale, int64_t group_size, int64_t M,
                             int64_t K, int64_t N, void* y, void* stream) {
  return wqbmm_a16w4_msd_path(x, w_tiled, antiquant_scale, group_size, M, K, N, y,
                              WQBMM_PATH_AUTO, stream);
}

wqbmm_status wqbmm_a16w4_msd_noalloc(const void* x, const void* w_tiled,
                                     const void* antiquant_scale, int64_t group_size, int64_t M,
                                     int64_t K, int64_t N, void* y, void* stream) {
  int p = 0;
  wqbmm_status st = validate_call(x, w_tiled, antiquant_scale, true, y, group_size, M, K, N,
                                  WQBMM_PATH_AUTO, &p);
  if (st != WQBMM_OK || M == 0) return st;
  int dev = -1;
  st = check_device(&dev);
  if (st != WQBMM_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Buffers b;
  st = scratch_buffers(dev, s, needs_of(p, group_size, M, K, N, 0, K / group_size, false, false), &b);
  if (st != WQBMM_OK) return st;
  return run_path(b, p, x, w_tiled, nullptr, antiquant_scale, group_size, M, K, N, 0, K / group_size,
                  y, nullptr, 0, s);
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
  int p = 0;
  wqbmm_status st = validate_call(x, w_tiled, nullptr, false, y_int, group_size, M, K, N, path, &p);
  if (st != WQBMM_OK) return st;
  if (g_begin < 0 || g_end > K / group_size || g_begin >= g_end) return WQBMM_ERR_INVALID;
  if (M == 0) return WQBMM_OK;
  return run(x, w_tiled, nullptr, nullptr, group_size, M, K, N, g_begin, g_end, nullptr, y_int, p, 0,
             static_cast<hipStream_t>(stream));
}

wqbmm_status wqbmm_a16w4_msd_profile_stage(const void* x, const void* w_tiled,
                                           const void* w_operand, const void* antiquant_scale,
                                           int64_t group_size, int64_t M, int64_t K, int64_t N,
                                           void* y, int path, int stage, void* stream) {
  int p = 0;
  const wqbmm_status st = validate_call(x, w_tiled, antiquant_scale, true, y, group_size, M, K, N, path, &p);
  if (st != WQBMM_OK) return st;
  if (!aligned16(w_operand) || stage < 1 || stage > 2) return WQBMM_ERR_INVALID;
  if (M == 0) return WQBMM_OK;
  return run(x, w_tiled, w_operand, antiquant_scale, group_size, M, K, N, 0, K / group_size, y,
             nullptr, p, stage, static_cast<hipStream_t>(stream));
}

}  // extern "C"
