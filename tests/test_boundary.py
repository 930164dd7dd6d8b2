"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/wqbmm.h declares, and
reject bad arguments on the host with the documented status before touching
the device (the pointers passed here are never dereferenced).  Table-driven
like the parameter-check unit tests the CANN aclnn pages describe
(null pointer -> NULLPTR, empty/invalid shape -> INVALID).
"""
import ctypes

import pytest

from weight_only_quantized_msd_amd import _lib as L

FAKE = 0x1000          # 16-byte aligned, never dereferenced: validation fails first
MIS = 0x1008           # misaligned


@pytest.fixture(autouse=True)
def no_device_visible():
    """These checks pass pointers that are never valid device memory.  They
    run only where no GPU is visible: there a call that validation wrongly
    let through stops at the device check (WQBMM_ERR_UNSUPPORTED) instead of
    launching kernels on the fake pointers."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("fake-pointer validation checks run only without a visible GPU")
    except ImportError:
        pass


def test_library_exports_every_header_symbol():
    names = L.header_functions()
    assert {"wqbmm_a16w4_msd", "wqbmm_a16w4_msd_prepass", "wqbmm_a16w4_msd_yint"} <= set(names)
    handle = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(L.SIGNATURES), "binding and header disagree"


def test_status_strings_and_version():
    for s in range(8):
        assert L.status_string(s).startswith("WQBMM_")
    assert "UNKNOWN" in L.status_string(99)
    assert L.wqbmm_version() >= 10000


def test_select_path():
    assert L.wqbmm_select_path(1, 4096, 4096, 128) == L.WQBMM_PATH_DECODE
    assert L.wqbmm_select_path(16, 4096, 11008, 128) == L.WQBMM_PATH_DECODE
    assert L.wqbmm_select_path(48, 8192, 28672, 64) == L.WQBMM_PATH_DECODE
    assert L.wqbmm_select_path(49, 8192, 28672, 64) == L.WQBMM_PATH_PREFILL
    assert L.wqbmm_select_path(64, 4096, 4096, 128) == L.WQBMM_PATH_DECODE
    assert L.wqbmm_select_path(96, 4096, 4096, 128) == L.WQBMM_PATH_DECODE
    assert L.wqbmm_select_path(97, 4096, 4096, 128) == L.WQBMM_PATH_PREFILL
    assert L.wqbmm_select_path(65, 4096, 4096, 64) == L.WQBMM_PATH_PREFILL
    assert L.wqbmm_select_path(64, 4096, 11008, 128) == L.WQBMM_PATH_DECODE
    assert L.wqbmm_select_path(65, 4096, 11008, 128) == L.WQBMM_PATH_PREFILL
    assert L.wqbmm_select_path(49, 8192, 8192, 128) == L.WQBMM_PATH_PREFILL
    assert L.wqbmm_select_path(48, 8192, 8192, 128) == L.WQBMM_PATH_DECODE
    assert L.wqbmm_select_path(2048, 4096, 4096, 128) == L.WQBMM_PATH_PREFILL


OK_ARGS = dict(x=FAKE, w=FAKE, s=FAKE, gs=128, M=4, K=256, N=256, y=FAKE)

MSD_CASES = [
    ("null x", dict(x=0), L.WQBMM_ERR_NULLPTR),
    ("null w", dict(w=0), L.WQBMM_ERR_NULLPTR),
    ("null scale", dict(s=0), L.WQBMM_ERR_NULLPTR),
    ("null y", dict(y=0), L.WQBMM_ERR_NULLPTR),
    ("null beats bad shape", dict(x=0, K=7), L.WQBMM_ERR_NULLPTR),
    ("M < 0", dict(M=-1), L.WQBMM_ERR_INVALID),
    ("K == 0", dict(K=0), L.WQBMM_ERR_INVALID),
    ("N == 0", dict(N=0), L.WQBMM_ERR_INVALID),
    ("K % gs", dict(K=200), L.WQBMM_ERR_INVALID),
    ("N % 32", dict(N=48), L.WQBMM_ERR_INVALID),
    ("N odd", dict(N=257), L.WQBMM_ERR_INVALID),
    ("gs <= 0", dict(gs=0), L.WQBMM_ERR_INVALID),
    ("M too large", dict(M=(1 << 24) + 1), L.WQBMM_ERR_INVALID),
    ("K too large", dict(K=(1 << 21)), L.WQBMM_ERR_INVALID),
    ("misaligned x", dict(x=MIS), L.WQBMM_ERR_INVALID),
    ("misaligned y", dict(y=MIS), L.WQBMM_ERR_INVALID),
    ("gs 32 unsupported", dict(gs=32), L.WQBMM_ERR_UNSUPPORTED),
    ("gs 256 unsupported", dict(gs=256, K=512), L.WQBMM_ERR_UNSUPPORTED),
    ("empty batch is a no-op", dict(M=0), L.WQBMM_OK),
    ("empty batch allows null x and y", dict(M=0, x=0, y=0), L.WQBMM_OK),
    ("empty batch still needs w", dict(M=0, w=0), L.WQBMM_ERR_NULLPTR),
]


@pytest.mark.parametrize("name,over,want", MSD_CASES, ids=[c[0] for c in MSD_CASES])
def test_msd_validation(name, over, want):
    a = dict(OK_ARGS, **over)
    st = L.wqbmm_a16w4_msd_raw(a["x"], a["w"], a["s"], a["gs"], a["M"], a["K"], a["N"], a["y"], None)
    assert st == want, (name, L.status_string(st))


@pytest.mark.parametrize("path,M,want", [
    (3, 4, L.WQBMM_ERR_INVALID),            # unknown path
    (-1, 4, L.WQBMM_ERR_INVALID),
    (L.WQBMM_PATH_DECODE, 97, L.WQBMM_ERR_INVALID),   # decode kernels cover M <= 96
    (L.WQBMM_PATH_DECODE, 0, L.WQBMM_OK),
    (L.WQBMM_PATH_PREFILL, 0, L.WQBMM_OK),
])
def test_path_validation(path, M, want):
    st = L.wqbmm_a16w4_msd_path_raw(FAKE, FAKE, FAKE, 128, M, 256, 256, FAKE, path, None)
    assert st == want


@pytest.mark.parametrize("over,want", [
    (dict(x=0), L.WQBMM_ERR_NULLPTR),
    (dict(a=0), L.WQBMM_ERR_NULLPTR),
    (dict(m=0), L.WQBMM_ERR_NULLPTR),
    (dict(K=100), L.WQBMM_ERR_INVALID),
    (dict(a=MIS), L.WQBMM_ERR_INVALID),
    (dict(gs=16, K=256), L.WQBMM_ERR_UNSUPPORTED),
    (dict(M=0), L.WQBMM_OK),
])
def test_prepass_validation(over, want):
    a = dict(x=FAKE, gs=64, M=2, K=256, a=FAKE, m=FAKE)
    a.update(over)
    st = L.wqbmm_a16w4_msd_prepass_raw(a["x"], a["gs"], a["M"], a["K"], a["a"], a["m"], None)
    assert st == want


@pytest.mark.parametrize("over,want", [
    (dict(y=0), L.WQBMM_ERR_NULLPTR),
    (dict(gb=-1), L.WQBMM_ERR_INVALID),
    (dict(ge=5), L.WQBMM_ERR_INVALID),          # K/gs = 4 groups
    (dict(gb=2, ge=2), L.WQBMM_ERR_INVALID),    # empty range
    (dict(gb=3, ge=1), L.WQBMM_ERR_INVALID),
    (dict(path=L.WQBMM_PATH_DECODE, M=97), L.WQBMM_ERR_INVALID),
    (dict(M=0), L.WQBMM_OK),
])
def test_yint_validation(over, want):
    a = dict(x=FAKE, w=FAKE, gs=64, M=2, K=256, N=64, gb=0, ge=4, y=FAKE, path=0)
    a.update(over)
    st = L.wqbmm_a16w4_msd_yint_raw(a["x"], a["w"], a["gs"], a["M"], a["K"], a["N"], a["gb"],
                                    a["ge"], a["y"], a["path"], None)
    assert st == want


@pytest.mark.parametrize("over,want", [
    (dict(stage=0), L.WQBMM_ERR_INVALID),
    (dict(stage=3), L.WQBMM_ERR_INVALID),
    (dict(x=0), L.WQBMM_ERR_NULLPTR),
    (dict(w=0), L.WQBMM_ERR_NULLPTR),
    (dict(N=40), L.WQBMM_ERR_INVALID),
    (dict(y=MIS), L.WQBMM_ERR_INVALID),
    (dict(gs=96, K=192), L.WQBMM_ERR_UNSUPPORTED),
    (dict(path=3), L.WQBMM_ERR_INVALID),
    (dict(path=-1), L.WQBMM_ERR_INVALID),
    (dict(path=L.WQBMM_PATH_DECODE, M=97), L.WQBMM_ERR_INVALID),
    (dict(M=0, x=0, y=0), L.WQBMM_OK),
])
def test_profile_stage_validation(over, want):
    a = dict(x=FAKE, w=FAKE, o=None, s=FAKE, gs=64, M=2, K=256, N=64, y=FAKE, path=0, stage=1)
    a.update(over)
    st = L.wqbmm_a16w4_msd_profile_stage_raw(a["x"], a["w"], a["o"], a["s"], a["gs"], a["M"], a["K"],
                                             a["N"], a["y"], a["path"], a["stage"], None)
    assert st == want


@pytest.mark.parametrize("over,want", [
    (dict(o=MIS), L.WQBMM_ERR_INVALID),              # a misaligned operand form
    (dict(o=MIS, stage=2), L.WQBMM_ERR_INVALID),
    (dict(o=FAKE, M=0), L.WQBMM_OK),
    (dict(o=MIS, M=0), L.WQBMM_ERR_INVALID),         # checked even for an empty batch
])
def test_profile_stage_operand_validation(over, want):
    a = dict(x=FAKE, w=FAKE, o=None, s=FAKE, gs=128, M=2, K=256, N=64, y=FAKE, path=2, stage=1)
    a.update(over)
    st = L.wqbmm_a16w4_msd_profile_stage_raw(a["x"], a["w"], a["o"], a["s"], a["gs"], a["M"], a["K"],
                                             a["N"], a["y"], a["path"], a["stage"], None)
    assert st == want


EX_CASES = MSD_CASES + [
    ("misaligned operand form", dict(o=MIS), L.WQBMM_ERR_INVALID),
    ("operand form, empty batch", dict(o=FAKE, M=0), L.WQBMM_OK),
    ("misaligned operand form, empty batch", dict(o=MIS, M=0), L.WQBMM_ERR_INVALID),
    ("operand form does not replace w", dict(o=FAKE, w=0), L.WQBMM_ERR_NULLPTR),
    ("null beats a misaligned operand form", dict(o=MIS, x=0), L.WQBMM_ERR_NULLPTR),
    ("bad shape beats a misaligned operand form", dict(o=MIS, K=200), L.WQBMM_ERR_INVALID),
]


@pytest.mark.parametrize("name,over,want", EX_CASES, ids=[c[0] for c in EX_CASES])
def test_msd_ex_validation(name, over, want):
    a = dict(OK_ARGS, o=None, path=0)
    a.update(over)
    st = L.wqbmm_a16w4_msd_ex_raw(a["x"], a["w"], a["o"], a["s"], a["gs"], a["M"], a["K"], a["N"],
                                  a["y"], a["path"], None)
    assert st == want, (name, L.status_string(st))


@pytest.mark.parametrize("K,N,want", [
    (4096, 4096, (4096 // 32) * 32 * 3072),    # 1.5x the int4 bytes: 6 bits per weight
    (4096, 4128, (4352 // 32) * 32 * 3072),    # columns padded to a multiple of 256
    (8192, 28672, (28672 // 32) * 64 * 3072),
    (192, 64, (256 // 32) * 2 * 3072),         # rows padded to 256
    (1, 32, (256 // 32) * 1 * 3072),
    (0, 64, -1), (64, 0, -1), (64, 48, -1),    # the tiled weights' shape rules
    ((1 << 20) + 1, 64, -1), (64, (1 << 20) + 32, -1),
])
def test_operand_weight_bytes(K, N, want):
    assert L.wqbmm_a16w4_operand_weight_bytes(K, N) == want


@pytest.mark.parametrize("over,want", [
    (dict(t=0), L.WQBMM_ERR_NULLPTR),
    (dict(o=0), L.WQBMM_ERR_NULLPTR),
    (dict(o=0, K=0), L.WQBMM_ERR_NULLPTR),
    (dict(K=0), L.WQBMM_ERR_INVALID),
    (dict(N=48), L.WQBMM_ERR_INVALID),
    (dict(t=MIS), L.WQBMM_ERR_INVALID),
    (dict(o=MIS), L.WQBMM_ERR_INVALID),
])
def test_operand_weights_validation(over, want):
    a = dict(t=FAKE, K=256, N=64, o=FAKE)
    a.update(over)
    st = L.wqbmm_a16w4_operand_weights_raw(a["t"], a["K"], a["N"], a["o"], None)
    assert st == want


@pytest.mark.parametrize("K,N,want", [
    (4096, 4096, 4096 * 4096 // 2),            # K % 128 == 0: exactly K*N/2
    (8192, 28672, 8192 * 28672 // 2),
    (192, 64, (64 // 16) * 2 * 1024),          # rows padded to 256
    (64, 32, 2 * 1024),
    (1, 32, 2 * 1024),
    (0, 64, -1), (64, 0, -1), (64, 48, -1),    # shape rules
    ((1 << 20) + 1, 64, -1), (64, (1 << 20) + 32, -1),
])
def test_tiled_weight_bytes(K, N, want):
    assert L.wqbmm_a16w4_tiled_weight_bytes(K, N) == want


@pytest.mark.parametrize("over,want", [
    (dict(w=0), L.WQBMM_ERR_NULLPTR),
    (dict(t=0), L.WQBMM_ERR_NULLPTR),
    (dict(w=0, K=0), L.WQBMM_ERR_NULLPTR),       # null pointer checked first
    (dict(K=0), L.WQBMM_ERR_INVALID),
    (dict(N=48), L.WQBMM_ERR_INVALID),
    (dict(N=-32), L.WQBMM_ERR_INVALID),
    (dict(w=MIS), L.WQBMM_ERR_INVALID),
    (dict(t=MIS), L.WQBMM_ERR_INVALID),
])
def test_tile_weights_validation(over, want):
    a = dict(w=FAKE, K=256, N=64, t=FAKE)
    a.update(over)
    st = L.wqbmm_a16w4_tile_weights_raw(a["w"], a["K"], a["N"], a["t"], None)
    assert st == want


@pytest.mark.parametrize("mode,iters,out,want", [
    (0, 10, 0, 1),            # null output
    (11, 10, FAKE, 2), (-1, 10, FAKE, 2),
    (0, 0, FAKE, 2), (0, (1 << 20) + 1, FAKE, 2),
])
def test_probe_mfma_valu_validation(mode, iters, out, want):
    assert L.wqbmm_probe_mfma_valu_raw(mode, iters, out, None) == want
