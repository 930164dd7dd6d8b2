"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Method: the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4 PerGroup
伪量化 MatMul 的 MSD 算法与双模板流水设计" (lpnh.cn/news/2294145), §4.1.

Bars:
  * A_int (steps 1-8) byte-identical and A_max bit-identical to the oracle;
  * Y_int (step 9) word-identical to the oracle, on both kernel paths;
  * y (steps 10-11, fp16) against the oracle's fp32 Y32:
        ||y - Y32||_2 / ||Y32||_2 <= 1e-3   and   max|y - Y32| <= 2e-2 * max|Y32|,
    and, element by element, the bound elementwise_bound() derives below:
    half an fp16 ulp (the final rounding) plus what fp32 reassociation of
    steps 10-11 can change;
  * run-to-run bit-identical y.
Inputs are the seeded synthetic workloads of weight_only_quantized_msd_amd.datagen.
"""
import numpy as np
import pytest

import oracle
from parity_bounds import check_y_elementwise, elementwise_bound
from weight_only_quantized_msd_amd import datagen

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS_FRAC = 2e-2

DECODE, PREFILL, AUTO = 1, 2, 0


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_msd_amd as W  # noqa: F401  (loads libwqbmm.so)
    W.lib()
    return torch


def announce(msg):
    print(f"\n[gpu case] {msg}", flush=True)


_cache = {}


def workload(name, M=None):
    key = (name, M)
    if key not in _cache:
        _cache[key] = datagen.make_inputs(name, M=M)
    return _cache[key]


def to_dev(torch, d):
    """x, the TILED weights (converted on the device), scale."""
    import weight_only_quantized_msd_amd as W
    w_tiled = W.wqbmm_a16w4_tile_weights(torch.from_numpy(d["w_packed"]).cuda())
    return (torch.from_numpy(d["x"]).cuda(), w_tiled, torch.from_numpy(d["scale"]).cuda())


def tiled_reference(w, K, N):
    """The tiled weight layout as documented with the C ABI, restated with
    numpy from the unpacked int4 matrix w [K][N]: chunk (nt, kb, lane) holds
    column 16nt + lane%16 at rows 128kb + 64s + 16(lane/16) + 8d + j (low
    nibble of byte 4d + j of step s) and that row + 4 (high nibble); rows
    beyond K are zero."""
    KB = (K + 127) // 128
    wp = np.zeros((KB * 128, N), np.int64)
    wp[:K] = w
    nt, kb, lane, s, d, j = np.meshgrid(np.arange(N // 16), np.arange(KB), np.arange(64),
                                        np.arange(2), np.arange(2), np.arange(4), indexing="ij")
    n = 16 * nt + lane % 16
    k = 128 * kb + 64 * s + 16 * (lane // 16) + 8 * d + j
    byte = (wp[k, n] & 0xF) | ((wp[k + 4, n] & 0xF) << 4)
    return byte.astype(np.uint8).reshape(N // 16, KB * 1024)


def check_y(y, y32, what):
    y = y.astype(np.float64)
    ref = y32.astype(np.float64)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(y - ref) / max(nref, 1e-30)
    mabs = np.abs(y - ref).max() if y.size else 0.0
    lim = MAX_ABS_FRAC * (np.abs(ref).max() if ref.size else 0.0)
    assert rel <= REL_L2 or nref == 0, f"{what}: rel-L2 {rel:.3e}"
    assert mabs <= lim or nref == 0, f"{what}: max-abs {mabs:.3e} > {lim:.3e}"
    if nref == 0:
        assert np.count_nonzero(y) == 0, what


def sample_rows(M, n, seed):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(1, M - 1), n - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], rest]))


ALL = ["tiny", "decode_m1", "decode_m16", "ffn_up_m16", "prefill_m2048", "outlier_m128",
       "pages_sample_m1", "mid_m64", "mid_m256"]


# ------------------------------------------------------------------ weight tiling

@pytest.mark.parametrize("K,N", [(256, 256), (192, 96), (64, 32), (4096, 4096), (8192, 28672 // 8)])
def test_tiled_weights_match_documented_layout(torch_dev, K, N):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = datagen.random_case(1, K, N, 64, seed=K + N)
    announce(f"tile weights K={K} N={N}")
    got = W.wqbmm_a16w4_tile_weights(torch.from_numpy(d["w_packed"]).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), tiled_reference(d["w"].astype(np.int64), K, N))


# ------------------------------------------------------------------ steps 1-8

@pytest.mark.parametrize("name", ALL)
def test_prepass_bit_exact(torch_dev, name):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = workload(name)
    gs = d["group_size"]
    announce(f"prepass {name} M={d['M']} K={d['K']} gs={gs}")
    a_int, a_max = W.wqbmm_a16w4_msd_prepass(torch.from_numpy(d["x"]).cuda(), gs)
    torch.cuda.synchronize()
    ra, rm = oracle.decompose(d["x"], gs)
    assert np.array_equal(a_int.cpu().numpy(), ra)
    assert np.array_equal(a_max.cpu().numpy().view(np.uint32), rm.view(np.uint32))


def adversarial_x(seed, M, K, gs):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[0, :gs] = 0.0                                    # all-zero group
    x[0, gs:2 * gs] *= 1e-5                            # fp16 subnormals
    if M > 1:
        x[1, ::5] *= 500.0                             # outlier channels
        x[1, 2 * gs:3 * gs] = 0.75                     # constant group
    if M > 2:
        x[2] = -np.abs(x[2])
    x = x.astype(np.float16)
    # exact-tie and op-order vectors (element, its group max) at the start of a group
    import json, os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "msd_tie_vectors.json")))
    pairs = fx["vectors"] + fx["order_vectors"]
    for i, v in enumerate(pairs):
        r, g = (i % M), (3 + i // M)
        if (g + 1) * gs > K:
            break
        a = np.uint16(int(v["a"], 16)).view(np.float16)
        m = np.uint16(int(v["amax"], 16)).view(np.float16)
        blk = np.zeros(gs, np.float16)
        blk[0], blk[1] = a, m
        x[r, g * gs:(g + 1) * gs] = blk
    return x


@pytest.mark.parametrize("M,K,gs", [(1, 64, 64), (3, 1024, 64), (5, 2048, 128), (33, 1920, 128)])
def test_prepass_edge_cases(torch_dev, M, K, gs):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    x = adversarial_x(M * 7 + K, M, K, gs)
    announce(f"prepass edge M={M} K={K} gs={gs}")
    a_int, a_max = W.wqbmm_a16w4_msd_prepass(torch.from_numpy(x).cuda(), gs)
    torch.cuda.synchronize()
    ra, rm = oracle.decompose(x, gs)
    assert np.array_equal(a_int.cpu().numpy(), ra)
    assert np.array_equal(a_max.cpu().numpy().view(np.uint32), rm.view(np.uint32))


# ------------------------------------------------------------------ step 9

# Groups sampled at full size: first, middle (G/2), last and one seeded group.
_P_SEEDED = int(np.random.default_rng(4).integers(1, 31))
_O_SEEDED = int(np.random.default_rng(5).integers(1, 127))
YINT_CASES = [
    ("tiny", DECODE, None), ("tiny", PREFILL, None),
    ("decode_m1", DECODE, None), ("decode_m1", PREFILL, (0, 5)),
    ("decode_m16", DECODE, None), ("decode_m16", PREFILL, (7, 12)),
    ("ffn_up_m16", DECODE, (0, 32)),
    ("prefill_m2048", PREFILL, (0, 1)), ("prefill_m2048", PREFILL, (16, 17)),
    ("prefill_m2048", PREFILL, (_P_SEEDED, _P_SEEDED + 1)), ("prefill_m2048", PREFILL, (31, 32)),
    ("outlier_m128", PREFILL, (0, 2)), ("outlier_m128", PREFILL, (64, 65)),
    ("outlier_m128", PREFILL, (_O_SEEDED, _O_SEEDED + 1)), ("outlier_m128", PREFILL, (126, 128)),
    ("pages_sample_m1", DECODE, (0, 64)),
    ("mid_m64", DECODE, None), ("mid_m64", PREFILL, (13, 19)),
    ("mid_m256", PREFILL, (0, 32)),
]


@pytest.mark.parametrize("name,path,grange", YINT_CASES,
                         ids=[f"{c[0]}-{'dec' if c[1] == 1 else 'pre'}-{c[2]}" for c in YINT_CASES])
def test_yint_word_exact(torch_dev, name, path, grange):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = workload(name)
    gs, G = d["group_size"], d["K"] // d["group_size"]
    gb, ge = grange if grange else (0, G)
    x, w, _ = to_dev(torch, d)
    announce(f"yint {name} path={path} groups=[{gb},{ge})")
    yi = W.wqbmm_a16w4_msd_yint(x, w, gs, gb, ge, path=path)
    torch.cuda.synchronize()
    ra, _ = oracle.decompose(d["x"], gs)
    ref = oracle.yint(ra, d["w"], gs, gb, ge)
    got = yi.cpu().numpy()
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} words differ"


# ------------------------------------------------------------------ steps 10-11

Y_CASES = [
    ("tiny", AUTO, None), ("tiny", PREFILL, None),
    ("decode_m1", AUTO, None), ("decode_m1", PREFILL, None),
    ("decode_m16", AUTO, None), ("decode_m16", PREFILL, None),
    ("ffn_up_m16", AUTO, None),
    ("prefill_m2048", AUTO, None),
    ("outlier_m128", AUTO, None),
    ("pages_sample_m1", AUTO, None),
    ("mid_m64", AUTO, None), ("mid_m64", DECODE, None), ("mid_m64", PREFILL, None),
    ("mid_m256", AUTO, None),
]


@pytest.mark.parametrize("name,path,nrows", Y_CASES,
                         ids=[f"{c[0]}-{['auto', 'dec', 'pre'][c[1]]}" for c in Y_CASES])
def test_y_within_tolerance(torch_dev, name, path, nrows):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = workload(name)
    gs = d["group_size"]
    x, w, s = to_dev(torch, d)
    announce(f"y {name} path={path} M={d['M']} K={d['K']} N={d['N']}")
    y = W.wqbmm_a16w4_msd_path(x, w, s, gs, path)
    torch.cuda.synchronize()
    rows = None if nrows is None else sample_rows(d["M"], nrows, 17)
    y32, _ = oracle.matmul(d["x"], d["w_packed"], d["scale"], gs, rows=rows)
    got = y.cpu().numpy()
    got = got if rows is None else got[rows]
    check_y(got, y32, name)
    check_y_elementwise(got, y32, elementwise_bound(d, rows), name)


RAGGED = [  # (M, K, N, gs)
    (1, 64, 32, 64), (2, 128, 96, 128), (3, 192, 160, 64), (4, 640, 288, 128),
    (5, 576, 4128, 64), (13, 1024, 416, 128), (16, 2560, 544, 128), (17, 512, 160, 64),
    (40, 1152, 224, 128), (64, 704, 96, 64), (65, 512, 160, 128), (81, 768, 96, 64),
    (96, 1152, 224, 128),
    (130, 384, 288, 128), (257, 256, 128, 64),
    # M <= 4 with K split over workgroups and a last chunk that ends inside it
    (1, 4736, 96, 64), (3, 6272, 160, 128),
    # prefill with columns padded to the GEMM's column block inside a tile pair
    # range (N = 96: six real 16-column tiles, ten padding tiles at BN = 128)
    (130, 384, 96, 128),
]


@pytest.mark.parametrize("M,K,N,gs", RAGGED, ids=[f"M{c[0]}K{c[1]}N{c[2]}g{c[3]}" for c in RAGGED])
def test_ragged_shapes(torch_dev, M, K, N, gs):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = datagen.random_case(M, K, N, gs, seed=M * 1000 + N)
    d["x"] = adversarial_x(M + K, M, K, gs) if K >= 4 * gs else d["x"]
    x, w, s = to_dev(torch, d)
    y32, _ = oracle.matmul(d["x"], d["w_packed"], d["scale"], gs)
    ra, _ = oracle.decompose(d["x"], gs)
    G = K // gs
    ref_yi = oracle.yint(ra, d["w"], gs, 0, G)
    paths = (DECODE, PREFILL) if M <= 96 else (PREFILL,)
    bound = elementwise_bound(d)
    for p in paths:
        announce(f"ragged M={M} K={K} N={N} gs={gs} path={p}")
        y = W.wqbmm_a16w4_msd_path(x, w, s, gs, p)
        yi = W.wqbmm_a16w4_msd_yint(x, w, gs, 0, G, path=p)
        torch.cuda.synchronize()
        check_y(y.cpu().numpy(), y32, f"path {p}")
        check_y_elementwise(y.cpu().numpy(), y32, bound, f"path {p}")
        assert np.array_equal(yi.cpu().numpy(), ref_yi), f"path {p} Y_int"


# The decode contraction for 4 < M <= 96 (operand kernel + full-K contraction,
# rows in slices of 16): K beyond 4096 (several load rounds per wave), a
# single 128-row block, K not a multiple of 128 at group size 64, Y_int over
# group ranges that start and end inside a 128-row block, and every slice
# count with full and ragged last slices (M = 17, 31, 32, 33, 48, 63, 64, 65,
# 80, 93, 96).
GEMV_CASES = [  # (M, K, N, gs, g_begin, g_end)
    (16, 8192, 512, 128, 0, 64), (8, 12288, 256, 128, 37, 91), (16, 8192, 384, 64, 5, 118),
    (5, 64, 96, 64, 0, 1), (9, 128, 64, 128, 0, 1), (12, 320, 160, 64, 1, 4),
    (17, 4096, 512, 128, 0, 32), (31, 2048, 256, 64, 3, 29), (32, 8192, 384, 128, 11, 60),
    (33, 1024, 288, 128, 0, 8), (48, 4096, 256, 64, 0, 64), (63, 640, 160, 64, 1, 9),
    (64, 4096, 512, 128, 0, 32), (64, 12288, 128, 64, 90, 150),
    (65, 2048, 256, 128, 0, 16), (80, 4096, 160, 64, 7, 53), (93, 640, 96, 64, 1, 9),
    (96, 4096, 512, 128, 0, 32), (96, 8192, 384, 64, 20, 110),
]


@pytest.mark.parametrize("M,K,N,gs,gb,ge", GEMV_CASES,
                         ids=[f"M{c[0]}K{c[1]}N{c[2]}g{c[3]}r{c[4]}-{c[5]}" for c in GEMV_CASES])
def test_decode_contraction_shapes(torch_dev, M, K, N, gs, gb, ge):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = datagen.random_case(M, K, N, gs, seed=M * 31 + K + N)
    if K >= 4 * gs:
        d["x"] = adversarial_x(M + K + 1, M, K, gs)
    x, w, s = to_dev(torch, d)
    announce(f"decode contraction M={M} K={K} N={N} gs={gs} groups=[{gb},{ge})")
    y = W.wqbmm_a16w4_msd_path(x, w, s, gs, DECODE)
    yi = W.wqbmm_a16w4_msd_yint(x, w, gs, gb, ge, path=DECODE)
    torch.cuda.synchronize()
    y32, _ = oracle.matmul(d["x"], d["w_packed"], d["scale"], gs)
    check_y(y.cpu().numpy(), y32, "decode contraction")
    check_y_elementwise(y.cpu().numpy(), y32, elementwise_bound(d), "decode contraction")
    ra, _ = oracle.decompose(d["x"], gs)
    ref = oracle.yint(ra, d["w"], gs, gb, ge)
    got = yi.cpu().numpy()
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} words differ"


# More column tiles than CUs (N/16 > 256): the decode contraction's workgroups
# each cover a run of column tiles with the level chunks held in registers.
# One and two row slices, both group sizes, up to 4 and up to 8 blocks per
# wave, waves without blocks (K = 640, K = 512), and a last workgroup with
# fewer tiles (one, for the odd-count path).  Runs of 5 and 7 tiles (N =
# 16640 and 28672) take the loop over tile pairs several times before the
# run's last tile leaves it.
MULTI_CASES = [  # (M, K, N, gs)
    (16, 4096, 4128, 128), (9, 8192, 5152, 64), (32, 4096, 6144, 128), (20, 2048, 8224, 64),
    (5, 640, 4640, 128), (16, 8192, 4160, 128), (16, 1024, 16640, 128), (12, 512, 28672, 64),
]


@pytest.mark.parametrize("M,K,N,gs", MULTI_CASES, ids=[f"M{c[0]}K{c[1]}N{c[2]}g{c[3]}" for c in MULTI_CASES])
def test_decode_multi_tile_shapes(torch_dev, M, K, N, gs):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = datagen.random_case(M, K, N, gs, seed=M * 17 + K + N)
    if K >= 4 * gs:
        d["x"] = adversarial_x(M + K + 5, M, K, gs)
    x, w, s = to_dev(torch, d)
    announce(f"decode multi-tile M={M} K={K} N={N} gs={gs}")
    y = W.wqbmm_a16w4_msd_path(x, w, s, gs, DECODE)
    y2 = W.wqbmm_a16w4_msd_path(x, w, s, gs, DECODE)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    y32, _ = oracle.matmul(d["x"], d["w_packed"], d["scale"], gs)
    check_y(y.cpu().numpy(), y32, "decode multi-tile")
    check_y_elementwise(y.cpu().numpy(), y32, elementwise_bound(d), "decode multi-tile")


# The group-128 GEMM with few tiles splits K over workgroups and adds the
# splits' fp32 partial sums in split order: single and ragged row blocks,
# ragged columns, split counts from 2 to 8 (uneven last split), and Y_int
# over odd group ranges (each split stores its own groups).
SPLITK_CASES = [  # (M, K, N, gs, g_begin, g_end)
    (1, 1024, 160, 128, 3, 8), (65, 2304, 416, 128, 0, 18), (130, 1024, 288, 128, 1, 8),
    (300, 4096, 544, 128, 5, 30), (97, 4096, 4096, 128, 0, 32),
    # 32 splits: more than the GEMM finishes itself, so the separate reduction runs
    (1, 8192, 128, 128, 10, 50),
]


@pytest.mark.parametrize("M,K,N,gs,gb,ge", SPLITK_CASES,
                         ids=[f"M{c[0]}K{c[1]}N{c[2]}r{c[4]}-{c[5]}" for c in SPLITK_CASES])
def test_prefill_splitk_shapes(torch_dev, M, K, N, gs, gb, ge):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = datagen.random_case(M, K, N, gs, seed=M * 7 + K + N)
    if K >= 4 * gs:
        d["x"] = adversarial_x(M + K + 3, M, K, gs)
    x, w, s = to_dev(torch, d)
    announce(f"prefill split-K M={M} K={K} N={N} gs={gs} groups=[{gb},{ge})")
    y = W.wqbmm_a16w4_msd_path(x, w, s, gs, PREFILL)
    y2 = W.wqbmm_a16w4_msd_path(x, w, s, gs, PREFILL)
    yi = W.wqbmm_a16w4_msd_yint(x, w, gs, gb, ge, path=PREFILL)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    y32, _ = oracle.matmul(d["x"], d["w_packed"], d["scale"], gs)
    check_y(y.cpu().numpy(), y32, "prefill split-K")
    check_y_elementwise(y.cpu().numpy(), y32, elementwise_bound(d), "prefill split-K")
    ra, _ = oracle.decompose(d["x"], gs)
    ref = oracle.yint(ra, d["w"], gs, gb, ge)
    got = yi.cpu().numpy()
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} words differ"


# Group size 64 with many row blocks: the weights are converted by the
# preparation kernel and the GEMM runs 128 x 256 tiles (at least 256 of them);
# K = 192 leaves a last stage of one group.  Sampled rows against the oracle.
WIDE64 = [(512, 192, 16384), (640, 320, 13312)]


@pytest.mark.parametrize("M,K,N", WIDE64, ids=[f"M{c[0]}K{c[1]}N{c[2]}" for c in WIDE64])
def test_group64_wide_tiles(torch_dev, M, K, N):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    gs = 64
    d = datagen.random_case(M, K, N, gs, seed=M + K)
    x, w, s = to_dev(torch, d)
    G = K // gs
    rows = sample_rows(M, 12, 5)
    announce(f"group64 wide M={M} K={K} N={N}")
    y = W.wqbmm_a16w4_msd_path(x, w, s, gs, PREFILL)
    yi = W.wqbmm_a16w4_msd_yint(x, w, gs, G - 1, G, path=PREFILL)
    torch.cuda.synchronize()
    y32, _ = oracle.matmul(d["x"], d["w_packed"], d["scale"], gs, rows=rows)
    check_y(y.cpu().numpy()[rows], y32, "group64 wide")
    check_y_elementwise(y.cpu().numpy()[rows], y32, elementwise_bound(d, rows), "group64 wide")
    ra, _ = oracle.decompose(d["x"][rows], gs)
    ref = oracle.yint(ra, d["w"], gs, G - 1, G)
    got = yi.cpu().numpy()[:, :, rows, :]
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} words differ"


def test_zero_weights_give_exact_zero(torch_dev):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = datagen.random_case(16, 1024, 256, 128, seed=3)
    x = torch.from_numpy(d["x"]).cuda()
    w = W.wqbmm_a16w4_tile_weights(torch.zeros((1024, 128), dtype=torch.uint8, device="cuda"))
    s = torch.from_numpy(d["scale"]).cuda()
    for p in (DECODE, PREFILL):
        announce(f"zero weights path={p}")
        y = W.wqbmm_a16w4_msd_path(x, w, s, 128, p)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y).item() == 0


# ------------------------------------------------------------------ determinism, streams, reuse

@pytest.mark.parametrize("name,path", [("decode_m16", DECODE), ("ffn_up_m16", DECODE),
                                       ("prefill_m2048", PREFILL), ("decode_m1", PREFILL)])
def test_run_to_run_bit_identical(torch_dev, name, path):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = workload(name)
    x, w, s = to_dev(torch, d)
    announce(f"determinism {name} path={path}")
    y1 = W.wqbmm_a16w4_msd_path(x, w, s, d["group_size"], path)
    y2 = W.wqbmm_a16w4_msd_path(x, w, s, d["group_size"], path)
    y3 = W.wqbmm_a16w4_msd_path(x, w, s, d["group_size"], path)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))


def test_side_stream_and_alternating_shapes(torch_dev):
    """The split-K counters re-arm themselves: alternating shapes on one stream
    and a second stream with its own workspace give the same results."""
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    outs = {}
    for name in ("decode_m16", "ffn_up_m16", "decode_m1"):
        d = workload(name)
        x, w, s = to_dev(torch, d)
        announce(f"reference {name}")
        outs[name] = (x, w, s, d["group_size"], W.wqbmm_a16w4_msd(x, w, s, d["group_size"]).clone())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        for name, (x, w, s, gs, ref) in outs.items():
            announce(f"repeat {rep} {name}")
            y = W.wqbmm_a16w4_msd(x, w, s, gs)
            with torch.cuda.stream(side):
                y_side = W.wqbmm_a16w4_msd(x, w, s, gs)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), name
            assert torch.equal(y_side.view(torch.int16), ref.view(torch.int16)), name


# The weights' operand form (wqbmm_a16w4_operand_weights): the group-128
# prefill GEMM then reads its weight tiles from it instead of from the
# preparation kernel.  Both GEMM column-block widths (256 at M = 2048; 128
# with a K-split at M = 256 and at the ragged shapes), columns padded to the
# 128-wide block inside the 256-padded form (N = 4128, N = 96), an odd count
# of 128-row blocks (K = 384), and calls where the form is not read (decode
# path, group size 64).  y must equal the call without the form bit for bit.
OPW_CASES = [  # (name or None, M, K, N, gs, path)
    ("prefill_m2048", None, None, None, None, PREFILL),
    ("mid_m256", None, None, None, None, PREFILL),
    (None, 200, 1024, 4128, 128, PREFILL),
    (None, 130, 384, 96, 128, PREFILL),
    (None, 65, 512, 160, 128, AUTO),
    (None, 300, 2048, 2080, 128, PREFILL),
    # 11 row blocks: 187 tiles of 256 columns (one round, no K-split) beat
    # 363 of 128 (two rounds); the last 256-column block is half padding
    (None, 1300, 512, 4128, 128, PREFILL),
    # 256 tiles of 128 columns (one round, no K-split) beat 128 of 256
    (None, 1024, 512, 4096, 128, PREFILL),
    # group size 64 past two row blocks: 128-column blocks (three rounds of
    # 128-column tiles against two of 256) and 256-column blocks with fewer
    # than 256 tiles (one round against two)
    (None, 384, 256, 28672, 64, PREFILL),
    (None, 640, 512, 8192, 64, PREFILL),
    ("decode_m16", None, None, None, None, AUTO),
    ("outlier_m128", None, None, None, None, PREFILL),
]


@pytest.mark.parametrize("case", OPW_CASES,
                         ids=[c[0] or f"M{c[1]}K{c[2]}N{c[3]}g{c[4]}" for c in OPW_CASES])
def test_operand_weights_bit_identical(torch_dev, case):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    name, M, K, N, gs, path = case
    d = workload(name) if name else datagen.random_case(M, K, N, gs, seed=M + K + N)
    M, K, N, gs = d["M"], d["K"], d["N"], d["group_size"]
    x, w, s = to_dev(torch, d)
    announce(f"operand weights M={M} K={K} N={N} gs={gs} path={path}")
    w_op = W.wqbmm_a16w4_operand_weights(w, K)
    assert w_op.numel() == -(-N // 256) * 8 * -(-K // 128) * 3072
    ref = W.wqbmm_a16w4_msd_path(x, w, s, gs, path)
    got = W.wqbmm_a16w4_msd_path(x, w, s, gs, path, w_operand=w_op)
    again = W.wqbmm_a16w4_msd_path(x, w, s, gs, path, w_operand=w_op)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(again.view(torch.int16), ref.view(torch.int16))
    rows = sample_rows(M, 24, 5)
    y32, _ = oracle.matmul(d["x"], d["w_packed"], d["scale"], gs, rows=rows)
    check_y(got.cpu().numpy()[rows], y32, "with the operand form")
    check_y_elementwise(got.cpu().numpy()[rows], y32, elementwise_bound(d, rows), "with the operand form")


def e2m3_decode(code):
    """Values of 6-bit e2m3 codes (sign, 2 exponent bits with bias 1, 3
    mantissa bits; exponent 0 is subnormal: m/8)."""
    code = np.asarray(code, np.int64)
    sign = np.where(code & 0x20, -1.0, 1.0)
    e, m = (code >> 3) & 3, code & 7
    mag = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * 2.0 ** (e - 1))
    return sign * mag


def operand_reference_values(buf, K, N):
    """The weights' operand form read back as values, restated from its
    documented layout: [256-column block][128-row block][16 column tiles,
    stored as 8 pairs of 3072 bytes: dwords 0-3 of both tiles' lanes (1 KB
    each), then dwords 4-5 (512 bytes each)]; lane l of column tile t holds
    column 16t + l%16 and 32 six-bit slots, slot 2j = k 16(l/16) + j and slot
    2j+1 = k 64 + 16(l/16) + j of the block.  Returns w/2 as [K][N]."""
    NB, KB = -(-N // 256), -(-K // 128)
    b = buf.reshape(NB, KB, 8, 3072)
    lo = np.stack([b[..., 0:1024], b[..., 1024:2048]], axis=3).reshape(NB, KB, 8, 2, 64, 16)
    hi = np.stack([b[..., 2048:2560], b[..., 2560:3072]], axis=3).reshape(NB, KB, 8, 2, 64, 8)
    lane_bytes = np.concatenate([lo, hi], axis=-1)                     # 24 bytes = 192 bits
    bits = np.unpackbits(lane_bytes, axis=-1, bitorder="little").reshape(NB, KB, 8, 2, 64, 32, 6)
    codes = (bits.astype(np.int64) << np.arange(6)).sum(-1)              # [.., lane, slot]
    vals = e2m3_decode(codes)
    out = np.zeros((KB * 128, NB * 256))
    lane = np.arange(64)
    for j in range(16):
        for half in range(2):
            k = 64 * half + 16 * (lane // 16) + j                         # [lane]
            v = vals[..., 2 * j + half]                                     # [NB, KB, pair, p, lane]
            for pr in range(8):
                for p in range(2):
                    col = (2 * pr + p) * 16 + lane % 16
                    for nb in range(NB):
                        for kb in range(KB):
                            out[128 * kb + k, 256 * nb + col] = v[nb, kb, pr, p]
    return out[:K, :N], out


@pytest.mark.parametrize("K,N", [(256, 96), (384, 288), (1024, 544)])
def test_operand_weights_match_documented_layout(torch_dev, K, N):
    """The operand form holds w/2 in e2m3 at the documented positions, and
    zeros in the padding (rows past K, columns past N)."""
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = datagen.random_case(1, K, N, 128, seed=K * 7 + N)
    announce(f"operand form layout K={K} N={N}")
    w_tiled = W.wqbmm_a16w4_tile_weights(torch.from_numpy(d["w_packed"]).cuda())
    w_op = W.wqbmm_a16w4_operand_weights(w_tiled, K)
    torch.cuda.synchronize()
    got, full = operand_reference_values(w_op.cpu().numpy(), K, N)
    assert np.array_equal(got, d["w"].astype(np.float64) / 2.0)
    pad = full.copy()
    pad[:K, :N] = 0.0
    assert not pad.any(), "padding is not zero"


def test_operand_weights_stages(torch_dev):
    """Stages with the operand form compose to the one-call result; stage 2
    refuses operands that a stage 1 prepared with the form when it is called
    without it (the weight tiles were not written), and the other way round."""
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = workload("mid_m256")
    gs = d["group_size"]
    x, w, s = to_dev(torch, d)
    announce("operand weights stages mid_m256")
    w_op = W.wqbmm_a16w4_operand_weights(w, d["K"])
    y1 = W.wqbmm_a16w4_msd_path(x, w, s, gs, PREFILL, w_operand=w_op)
    W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 1, path=PREFILL, w_operand=w_op)
    y2 = W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 2, path=PREFILL, w_operand=w_op)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    with pytest.raises(W.WqbmmError):
        W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 2, path=PREFILL)
    W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 1, path=PREFILL)
    with pytest.raises(W.WqbmmError):
        W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 2, path=PREFILL, w_operand=w_op)
    y3 = W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 2, path=PREFILL)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))


@pytest.mark.parametrize("name,path", [("decode_m16", PREFILL), ("prefill_m2048", PREFILL),
                                       ("outlier_m128", PREFILL), ("decode_m16", DECODE),
                                       ("ffn_up_m16", DECODE), ("decode_m1", DECODE)])
def test_profile_stages_compose_to_path(torch_dev, name, path):
    """Stage 1 (operand kernel) then stage 2 (contraction) give the same bits
    as the one-call path; stage 2 refuses operands prepared for another shape
    or by another path (the fused kernel at M <= 4 needs no operands)."""
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = workload(name)
    gs = d["group_size"]
    x, w, s = to_dev(torch, d)
    announce(f"profile stages {name} path={path}")
    y1 = W.wqbmm_a16w4_msd_path(x, w, s, gs, path)
    W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 1, path=path)
    y2 = W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 2, path=path)
    y3 = W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 2, path=path)   # operands stay prepared
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    if path == DECODE and d["M"] <= 4:
        return
    with pytest.raises(W.WqbmmError):
        W.wqbmm_a16w4_msd_profile_stage(x[: max(1, d["M"] // 2)].contiguous(), w, s, gs, 2, path=path)
    other = PREFILL if path == DECODE else DECODE
    if d["M"] <= 96:   # operands of the other path are not these
        W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 1, path=other)
        with pytest.raises(W.WqbmmError):
            W.wqbmm_a16w4_msd_profile_stage(x, w, s, gs, 2, path=path)


@pytest.mark.parametrize("name,path,opw", [("decode_m16", DECODE, False), ("ffn_up_m16", DECODE, False),
                                           ("tiny", PREFILL, False), ("outlier_m128", PREFILL, False),
                                           ("mid_m256", PREFILL, True), ("prefill_m2048", PREFILL, True)])
def test_graph_replay_matches_eager(torch_dev, name, path, opw):
    """bench.py submits its timed steps as a captured graph: every replay, with
    eager work and synchronizations in between, must reproduce the eager bits
    (the split-K counters re-arm inside the graph; no memset nodes).  With
    opw the captured call reads the weights' operand form."""
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = workload(name)
    gs = d["group_size"]
    x, w, s = to_dev(torch, d)
    w_op = W.wqbmm_a16w4_operand_weights(w, d["K"]) if opw else None
    announce(f"graph {name} path={path} operand form={opw}")
    ref = W.wqbmm_a16w4_msd_path(x, w, s, gs, path)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y = torch.empty_like(ref)
    with torch.cuda.stream(side):
        W.wqbmm_a16w4_msd_path(x, w, s, gs, path, y=y, stream=side, w_operand=w_op)   # warm this stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
        W.wqbmm_a16w4_msd_path(x, w, s, gs, path, y=y, stream=side, w_operand=w_op)
    for rep in range(4):
        y.fill_(7.0)
        other = W.wqbmm_a16w4_msd_path(x, w, s, gs, path)    # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.parametrize("name", ["decode_m16", "decode_m1", "ffn_up_m16"])
def test_splitk_back_to_back_stress(torch_dev, name):
    """Many split-K launches queued back to back (no host sync in between):
    every output equals the first bit for bit, and the first is within
    tolerance of the oracle.  Exercises the per-column-block counters that
    each launch re-arms for the next."""
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = workload(name)
    gs = d["group_size"]
    x, w, s = to_dev(torch, d)
    announce(f"split-K stress {name}")
    outs = [W.wqbmm_a16w4_msd_path(x, w, s, gs, DECODE) for _ in range(64)]
    torch.cuda.synchronize()
    for i, y in enumerate(outs[1:]):
        assert torch.equal(y.view(torch.int16), outs[0].view(torch.int16)), i
    y32, _ = oracle.matmul(d["x"], d["w_packed"], d["scale"], gs)
    check_y(outs[0].cpu().numpy(), y32, name)


def test_empty_batch_is_noop(torch_dev):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    x = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    w = W.wqbmm_a16w4_tile_weights(torch.zeros((256, 64), dtype=torch.uint8, device="cuda"))
    s = torch.ones((4, 128), dtype=torch.float16, device="cuda")
    y = W.wqbmm_a16w4_msd(x, w, s, 64)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 128)
