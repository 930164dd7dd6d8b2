"""ctypes binding of libwqbmm.so (the C ABI in include/wqbmm.h).

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the C ABI.  There is no CPU fallback: if the library is not
built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
# WQBMM_LIB selects another build of the same library (the host-sanitized
# build for the sanitizer runs of the boundary tests); default: the product.
LIB_PATH = os.environ.get("WQBMM_LIB") or os.path.join(_HERE, "libwqbmm.so")
INCLUDE_DIR = os.path.join(os.path.dirname(_HERE), "include")
HEADER_PATH = os.path.join(INCLUDE_DIR, "wqbmm.h")

WQBMM_OK = 0
WQBMM_ERR_NULLPTR = 1
WQBMM_ERR_INVALID = 2
WQBMM_ERR_UNSUPPORTED = 3
WQBMM_ERR_LAUNCH = 4
WQBMM_ERR_ALLOC = 5
WQBMM_ERR_CAPTURE = 6
WQBMM_ERR_TOO_LARGE = 7

WQBMM_PATH_AUTO = 0
WQBMM_PATH_DECODE = 1
WQBMM_PATH_PREFILL = 2

_i64 = ctypes.c_int64
_int = ctypes.c_int
_p = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/wqbmm.h
SIGNATURES = {
    "wqbmm_a16w4_tiled_weight_bytes": (_i64, [_i64, _i64]),
    "wqbmm_a16w4_tile_weights": (_int, [_p, _i64, _i64, _p, _p]),
    "wqbmm_a16w4_msd": (_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p]),
    "wqbmm_a16w4_msd_path": (_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _int, _p]),
    "wqbmm_a16w4_operand_weight_bytes": (_i64, [_i64, _i64]),
    "wqbmm_a16w4_operand_weights": (_int, [_p, _i64, _i64, _p, _p]),
    "wqbmm_a16w4_msd_ex": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _int, _p]),
    "wqbmm_a16w4_msd_noalloc": (_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p]),
    "wqbmm_a16w4_msd_prepass": (_int, [_p, _i64, _i64, _i64, _p, _p, _p]),
    "wqbmm_a16w4_msd_yint": (_int, [_p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p, _int, _p]),
    "wqbmm_a16w4_msd_profile_stage": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _int, _int, _p]),
    "wqbmm_select_path": (_int, [_i64, _i64, _i64, _i64]),
    "wqbmm_status_string": (ctypes.c_char_p, [_int]),
    "wqbmm_version": (_int, []),
    # include/wqbmm_probe.h (measurement helper)
    "wqbmm_probe_stream_read": (_int, [_p, _i64, _p, _p]),
    "wqbmm_probe_mfma_valu": (_int, [_int, _int, _p, _p]),
}

_lib = None


class WqbmmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def lib():
    """Load libwqbmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions the headers in include/ declare."""
    names = set()
    for h in sorted(os.listdir(INCLUDE_DIR)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE_DIR, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(wqbmm_\w+)\s*\(", text))
    return sorted(names)


def status_string(status: int) -> str:
    return lib().wqbmm_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != WQBMM_OK:
        raise WqbmmError(status, where)


# ---- raw C entry points (pointers as ints) ------------------------------------

def wqbmm_a16w4_tiled_weight_bytes(K, N) -> int:
    return lib().wqbmm_a16w4_tiled_weight_bytes(K, N)


def wqbmm_a16w4_tile_weights_raw(w_nd, K, N, w_tiled, stream) -> int:
    return lib().wqbmm_a16w4_tile_weights(w_nd, K, N, w_tiled, stream)


def wqbmm_a16w4_msd_raw(x, w, scale, group_size, M, K, N, y, stream) -> int:
    return lib().wqbmm_a16w4_msd(x, w, scale, group_size, M, K, N, y, stream)


def wqbmm_a16w4_msd_path_raw(x, w, scale, group_size, M, K, N, y, path, stream) -> int:
    return lib().wqbmm_a16w4_msd_path(x, w, scale, group_size, M, K, N, y, path, stream)


def wqbmm_a16w4_operand_weight_bytes(K, N) -> int:
    return lib().wqbmm_a16w4_operand_weight_bytes(K, N)


def wqbmm_a16w4_operand_weights_raw(w_tiled, K, N, w_operand, stream) -> int:
    return lib().wqbmm_a16w4_operand_weights(w_tiled, K, N, w_operand, stream)


def wqbmm_a16w4_msd_ex_raw(x, w, w_operand, scale, group_size, M, K, N, y, path, stream) -> int:
    return lib().wqbmm_a16w4_msd_ex(x, w, w_operand, scale, group_size, M, K, N, y, path, stream)


def wqbmm_a16w4_msd_noalloc_raw(x, w, scale, group_size, M, K, N, y, stream) -> int:
    return lib().wqbmm_a16w4_msd_noalloc(x, w, scale, group_size, M, K, N, y, stream)


def wqbmm_a16w4_msd_prepass_raw(x, group_size, M, K, a_int, a_max, stream) -> int:
    return lib().wqbmm_a16w4_msd_prepass(x, group_size, M, K, a_int, a_max, stream)


def wqbmm_a16w4_msd_yint_raw(x, w, group_size, M, K, N, g_begin, g_end, y_int, path, stream) -> int:
    return lib().wqbmm_a16w4_msd_yint(x, w, group_size, M, K, N, g_begin, g_end, y_int, path, stream)


def wqbmm_a16w4_msd_profile_stage_raw(x, w, w_operand, scale, group_size, M, K, N, y, path, stage,
                                      stream) -> int:
    return lib().wqbmm_a16w4_msd_profile_stage(x, w, w_operand, scale, group_size, M, K, N, y, path,
                                               stage, stream)


def wqbmm_probe_stream_read_raw(src, nbytes, sink, stream) -> int:
    return lib().wqbmm_probe_stream_read(src, nbytes, sink, stream)


def wqbmm_probe_mfma_valu_raw(mode, iters, out, stream) -> int:
    return lib().wqbmm_probe_mfma_valu(mode, iters, out, stream)


def wqbmm_select_path(M, K, N, group_size) -> int:
    return lib().wqbmm_select_path(M, K, N, group_size)


def wqbmm_version() -> int:
    return lib().wqbmm_version()
