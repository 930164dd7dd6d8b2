"""A16W4 per-group MSD weight-quantized matmul for AMD MI355X (gfx950).

    w_tiled = wqbmm_a16w4_tile_weights(w_nd)          # once per weight
    y = wqbmm_a16w4_msd(x, w_tiled, antiquant_scale, group_size)

    w_op = wqbmm_a16w4_operand_weights(w_tiled, K)    # optional, once per weight
    y = wqbmm_a16w4_msd(x, w_tiled, antiquant_scale, group_size, w_operand=w_op)

x: fp16 [M][K]; w_nd: uint8 [K][N/2] (two int4 per byte, column 2j in the low
nibble), converted once on the device into the library's tiled layout
(uint8 [N/16][ceil(K/128)*1024]); antiquant_scale: fp16 [K/group_size][N];
y: fp16 [M][N].  The optional operand form of the weights (FP6 MFMA operand
tiles, 0.75 byte per weight) spares the group-size-128 prefill path its
per-call weight conversion; results are bit-identical with or without it.

The method is the multi-step decomposition (MSD) of the page
"WeightQuantBatchMatmulExperiment 算子深度解析：A16W4 PerGroup 伪量化 MatMul 的
MSD 算法与双模板流水设计" (lpnh.cn/news/2294145), §4.1.  Everything runs in
the HIP kernels of libwqbmm.so behind the C ABI of include/wqbmm.h; these
wrappers only check tensor metadata and pass device pointers and the
current HIP stream.  PyTorch supplies device memory and streams.
"""
from __future__ import annotations

from ._lib import (WQBMM_ERR_ALLOC, WQBMM_ERR_CAPTURE, WQBMM_ERR_INVALID,  # noqa: F401
                   WQBMM_ERR_LAUNCH, WQBMM_ERR_NULLPTR, WQBMM_ERR_TOO_LARGE,
                   WQBMM_ERR_UNSUPPORTED, WQBMM_OK, WQBMM_PATH_AUTO,
                   WQBMM_PATH_DECODE, WQBMM_PATH_PREFILL, WqbmmError, check, lib,
                   status_string, wqbmm_select_path, wqbmm_version)

__all__ = [
    "wqbmm_a16w4_tile_weights", "wqbmm_a16w4_operand_weights", "wqbmm_a16w4_msd",
    "wqbmm_a16w4_msd_path", "wqbmm_a16w4_msd_noalloc",
    "wqbmm_a16w4_msd_prepass",
    "wqbmm_a16w4_msd_yint", "wqbmm_a16w4_msd_profile_stage", "wqbmm_select_path", "wqbmm_status_string", "wqbmm_version",
    "WqbmmError",
]


def wqbmm_status_string(status: int) -> str:
    return status_string(status)


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _require(t, dtype, ndim, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-D tensor")


def _tiled_shape(K: int, N: int):
    return (N // 16, (K + 127) // 128 * 1024)


def wqbmm_a16w4_tile_weights(w_nd, stream=None):
    """One-time conversion of the ND int4 weights (uint8 [K][N/2]) into the
    tiled layout the kernels read; returns uint8 [N/16][ceil(K/128)*1024]."""
    import torch
    _require(w_nd, torch.uint8, 2, "w_nd")
    K, N = w_nd.shape[0], w_nd.shape[1] * 2
    nbytes = lib().wqbmm_a16w4_tiled_weight_bytes(K, N)
    if nbytes < 0:
        check(WQBMM_ERR_INVALID, "wqbmm_a16w4_tiled_weight_bytes")
    w_tiled = torch.empty(_tiled_shape(K, N), dtype=torch.uint8, device=w_nd.device)
    assert w_tiled.numel() == nbytes
    st = lib().wqbmm_a16w4_tile_weights(w_nd.data_ptr(), K, N, w_tiled.data_ptr(),
                                        _stream_ptr(stream))
    check(st, "wqbmm_a16w4_tile_weights")
    return w_tiled


def wqbmm_a16w4_operand_weights(w_tiled, K: int, stream=None):
    """One-time conversion of tiled weights (for K rows) into their operand
    form for the group-size-128 prefill GEMM; returns uint8
    [wqbmm_a16w4_operand_weight_bytes(K, N)]."""
    import torch
    N = _weight_n(w_tiled, K)
    nbytes = lib().wqbmm_a16w4_operand_weight_bytes(K, N)
    if nbytes < 0:
        check(WQBMM_ERR_INVALID, "wqbmm_a16w4_operand_weight_bytes")
    w_op = torch.empty(nbytes, dtype=torch.uint8, device=w_tiled.device)
    st = lib().wqbmm_a16w4_operand_weights(w_tiled.data_ptr(), K, N, w_op.data_ptr(),
                                           _stream_ptr(stream))
    check(st, "wqbmm_a16w4_operand_weights")
    return w_op


def _operand_ptr(w_operand, K, N):
    import torch
    if w_operand is None:
        return None
    _require(w_operand, torch.uint8, 1, "w_operand")
    if w_operand.numel() != lib().wqbmm_a16w4_operand_weight_bytes(K, N):
        raise ValueError("w_operand must be the wqbmm_a16w4_operand_weights output for this K and N")
    return w_operand.data_ptr()


def _weight_n(w_tiled, K):
    import torch
    _require(w_tiled, torch.uint8, 2, "w_tiled")
    N = w_tiled.shape[0] * 16
    if tuple(w_tiled.shape) != _tiled_shape(K, N):
        raise ValueError("w_tiled must be the wqbmm_a16w4_tile_weights output for this K")
    return N


def wqbmm_a16w4_msd_path(x, w_tiled, antiquant_scale, group_size: int, path: int,
                         y=None, stream=None, w_operand=None):
    import torch
    _require(x, torch.float16, 2, "x")
    _require(antiquant_scale, torch.float16, 2, "antiquant_scale")
    M, K = x.shape
    N = _weight_n(w_tiled, K)
    if antiquant_scale.shape[1] != N or (
            group_size > 0 and antiquant_scale.shape[0] * group_size != K):
        raise ValueError("inconsistent shapes: x [M][K], tiled w for K x N, scale [K/gs][N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _require(y, torch.float16, 2, "y")
        if tuple(y.shape) != (M, N):
            raise ValueError("y must be [M][N]")
    st = lib().wqbmm_a16w4_msd_ex(x.data_ptr(), w_tiled.data_ptr(), _operand_ptr(w_operand, K, N),
                                  antiquant_scale.data_ptr(), int(group_size), M, K, N,
                                  y.data_ptr(), int(path), _stream_ptr(stream))
    check(st, "wqbmm_a16w4_msd")
    return y


def wqbmm_a16w4_msd(x, w_tiled, antiquant_scale, group_size: int, y=None, stream=None,
                    w_operand=None):
    """The operator; returns y (fp16 [M][N]).  Asynchronous on the current
    stream.  w_operand: the weights' optional operand form
    (wqbmm_a16w4_operand_weights)."""
    return wqbmm_a16w4_msd_path(x, w_tiled, antiquant_scale, group_size,
                                WQBMM_PATH_AUTO, y=y, stream=stream, w_operand=w_operand)


def wqbmm_a16w4_msd_noalloc(x, w_tiled, antiquant_scale, group_size: int, y, stream=None):
    """The operator without any device allocation (one fixed scratch array per
    device inside the library); y (fp16 [M][N]) is caller-provided and
    returned.  Calls that overlap in time on one device race."""
    import torch
    _require(x, torch.float16, 2, "x")
    _require(antiquant_scale, torch.float16, 2, "antiquant_scale")
    _require(y, torch.float16, 2, "y")
    M, K = x.shape
    N = _weight_n(w_tiled, K)
    if antiquant_scale.shape[1] != N or (
            group_size > 0 and antiquant_scale.shape[0] * group_size != K) or tuple(y.shape) != (M, N):
        raise ValueError("inconsistent shapes: x [M][K], tiled w for K x N, scale [K/gs][N], y [M][N]")
    st = lib().wqbmm_a16w4_msd_noalloc(x.data_ptr(), w_tiled.data_ptr(), antiquant_scale.data_ptr(),
                                       int(group_size), M, K, N, y.data_ptr(), _stream_ptr(stream))
    check(st, "wqbmm_a16w4_msd_noalloc")
    return y


def wqbmm_a16w4_msd_prepass(x, group_size: int, stream=None):
    """Steps 1-8: returns (a_int int8 [3][M][K], a_max fp32 [M][K/gs])."""
    import torch
    _require(x, torch.float16, 2, "x")
    M, K = x.shape
    a_int = torch.empty((3, M, K), dtype=torch.int8, device=x.device)
    a_max = torch.empty((M, K // max(int(group_size), 1)), dtype=torch.float32, device=x.device)
    st = lib().wqbmm_a16w4_msd_prepass(x.data_ptr(), int(group_size), M, K, a_int.data_ptr(),
                                       a_max.data_ptr(), _stream_ptr(stream))
    check(st, "wqbmm_a16w4_msd_prepass")
    return a_int, a_max


def wqbmm_a16w4_msd_yint(x, w_tiled, group_size: int, g_begin: int, g_end: int,
                         path: int = WQBMM_PATH_AUTO, stream=None):
    """Steps 1-9 for groups [g_begin, g_end): int32 [g_end-g_begin][3][M][N]."""
    import torch
    _require(x, torch.float16, 2, "x")
    M, K = x.shape
    N = _weight_n(w_tiled, K)
    y_int = torch.empty((max(g_end - g_begin, 0), 3, M, N), dtype=torch.int32, device=x.device)
    st = lib().wqbmm_a16w4_msd_yint(x.data_ptr(), w_tiled.data_ptr(), int(group_size),
                                    M, K, N, int(g_begin), int(g_end), y_int.data_ptr(),
                                    int(path), _stream_ptr(stream))
    check(st, "wqbmm_a16w4_msd_yint")
    return y_int


def wqbmm_a16w4_msd_profile_stage(x, w_tiled, antiquant_scale, group_size: int,
                                  stage: int, path: int = 0, y=None, stream=None, w_operand=None):
    """Run one stage of a kernel path (1: operand kernel, 2: contraction on the
    operands the last call of that path on this stream prepared); returns y."""
    import torch
    _require(x, torch.float16, 2, "x")
    _require(antiquant_scale, torch.float16, 2, "antiquant_scale")
    M, K = x.shape
    N = _weight_n(w_tiled, K)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    st = lib().wqbmm_a16w4_msd_profile_stage(x.data_ptr(), w_tiled.data_ptr(),
                                             _operand_ptr(w_operand, K, N),
                                             antiquant_scale.data_ptr(), int(group_size), M, K, N,
                                             y.data_ptr(), int(path), int(stage), _stream_ptr(stream))
    check(st, "wqbmm_a16w4_msd_profile_stage")
    return y
