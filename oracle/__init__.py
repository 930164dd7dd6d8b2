"""ctypes wrapper of the plain C oracle (``msd_oracle.c``).

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
cpu_baseline leg of ``bench.py`` may import this package; the HIP product
path (``weight_only_quantized_msd_amd``) never does.  It shares no code with
the HIP path.

Method source: the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4
PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计" (lpnh.cn/news/2294145), §4.1.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MSD_ORACLE_LIB") or os.path.join(_HERE, "libmsd_oracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from oracle.build import build
        build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.msd_oracle_half_to_float.restype = ctypes.c_float
    lib.msd_oracle_half_to_float.argtypes = [ctypes.c_uint16]
    lib.msd_oracle_float_to_half.restype = ctypes.c_uint16
    lib.msd_oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.msd_oracle_decompose.restype = ctypes.c_int
    lib.msd_oracle_decompose.argtypes = [_p, _i64, _i64, _i64, _p, _p]
    lib.msd_oracle_unpack_w.restype = ctypes.c_int
    lib.msd_oracle_unpack_w.argtypes = [_p, _i64, _i64, _p]
    lib.msd_oracle_yint.restype = ctypes.c_int
    lib.msd_oracle_yint.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p]
    lib.msd_oracle_matmul.restype = ctypes.c_int
    lib.msd_oracle_matmul.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _i64, _p, _p]
    lib.msd_oracle_num_threads.restype = ctypes.c_int
    lib.msd_oracle_num_threads.argtypes = []
    lib.msd_oracle_set_num_threads.restype = None
    lib.msd_oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def num_threads() -> int:
    return int(_load().msd_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of later oracle calls (OpenMP)."""
    _load().msd_oracle_set_num_threads(int(n))


def half_to_float(bits: int) -> float:
    return float(_load().msd_oracle_half_to_float(int(bits) & 0xFFFF))


def float_to_half(v: float) -> int:
    return int(_load().msd_oracle_float_to_half(float(np.float32(v))))


def half_to_float_array(bits: np.ndarray) -> np.ndarray:
    f = np.vectorize(half_to_float, otypes=[np.float32])
    return f(np.asarray(bits, dtype=np.uint16))


def decompose(x: np.ndarray, group_size: int):
    """Steps 1-8.  x: fp16 [M][K] -> (a_int int8 [3][M][K], a_max fp32 [M][G])."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    M, K = x.shape
    a_int = np.empty((3, M, K), np.int8)
    a_max = np.empty((M, K // group_size), np.float32)
    _check(_load().msd_oracle_decompose(_ptr(x.view(np.uint16)), M, K, group_size,
                                        _ptr(a_int), _ptr(a_max)), "decompose")
    return a_int, a_max


def unpack_w(w_packed: np.ndarray, N: int) -> np.ndarray:
    w_packed = np.ascontiguousarray(w_packed, dtype=np.uint8)
    K = w_packed.shape[0]
    assert w_packed.shape[1] * 2 == N
    w = np.empty((K, N), np.int8)
    _check(_load().msd_oracle_unpack_w(_ptr(w_packed), K, N, _ptr(w)), "unpack_w")
    return w


def yint(a_int: np.ndarray, w: np.ndarray, group_size: int, g_begin: int = 0,
         g_end: int | None = None) -> np.ndarray:
    """Step 9 for groups [g_begin, g_end): int32 [g_end-g_begin][3][M][N]."""
    a_int = np.ascontiguousarray(a_int, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    _, M, K = a_int.shape
    N = w.shape[1]
    G = K // group_size
    g_end = G if g_end is None else g_end
    out = np.empty((g_end - g_begin, 3, M, N), np.int32)
    _check(_load().msd_oracle_yint(_ptr(a_int), _ptr(w), M, K, N, group_size,
                                   g_begin, g_end, _ptr(out)), "yint")
    return out


def matmul(x: np.ndarray, w_packed: np.ndarray, scale: np.ndarray, group_size: int,
           rows=None):
    """Steps 1-11.  Returns (y32 fp32 [R][N], y16 fp16 [R][N]) for the given
    rows (all rows if None)."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    w_packed = np.ascontiguousarray(w_packed, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float16)
    M, K = x.shape
    N = w_packed.shape[1] * 2
    if rows is None:
        rows_arr, R, rows_p = None, M, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        R = rows_arr.shape[0]
        rows_p = _ptr(rows_arr)
    y32 = np.empty((R, N), np.float32)
    y16 = np.empty((R, N), np.uint16)
    _check(_load().msd_oracle_matmul(_ptr(x.view(np.uint16)), _ptr(w_packed),
                                     _ptr(scale.view(np.uint16)), group_size, M, K, N,
                                     rows_p, R, _ptr(y32), _ptr(y16)), "matmul")
    return y32, y16.view(np.float16)
