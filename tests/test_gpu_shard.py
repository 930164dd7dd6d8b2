"""Column (N) sharding, the split the path would use across GPUs: each GPU
holds the tiled weights and scales of a range of columns and computes that
range of y from all of x, with no exchange (the page "WeightQuantBatchMatmulExperiment
算子深度解析：A16W4 PerGroup 伪量化 MatMul 的 MSD 算法与双模板流水设计",
lpnh.cn/news/2294145, §8.1: each core's N offset is baseN times its index).

On one GPU: the operator on column slices of w_tiled (whole 16-column tiles,
a contiguous row range of the tiled layout) and of the scales must give the
matching slices of the full call's y.  Every output's fp32 sum runs over the
same groups in the same order as long as the shard keeps the prefill GEMM's
K-split count; then the slice is bit-identical.  A shard that changes the
split count (fewer tiles, more splits) adds the same group terms in another
association, and is held to the per-element reordering bound instead.
"""
import numpy as np
import pytest

import oracle
from parity_bounds import check_y_elementwise, elementwise_bound
from weight_only_quantized_msd_amd import datagen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_msd_amd as W
    W.lib()
    return torch


CASES = [  # (workload, shards, bit-identical expected)
    ("decode_m1", 4, True), ("decode_m16", 4, True), ("pages_sample_m1", 3, True),
    ("mid_m64", 4, True), ("prefill_m2048", 2, True), ("outlier_m128", 4, True),
    ("mid_m256", 2, False),
]


@pytest.mark.parametrize("name,shards,exact", CASES, ids=[f"{c[0]}-x{c[1]}" for c in CASES])
def test_column_shards_reproduce_the_full_call(torch_dev, name, shards, exact):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    d = datagen.make_inputs(name)
    gs, N = d["group_size"], d["N"]
    print(f"\n[gpu case] shards {name} x{shards}", flush=True)
    x = torch.from_numpy(d["x"]).cuda()
    w = W.wqbmm_a16w4_tile_weights(torch.from_numpy(d["w_packed"]).cuda())
    s = torch.from_numpy(d["scale"]).cuda()
    full = W.wqbmm_a16w4_msd(x, w, s, gs)
    edges = np.linspace(0, N // 32, shards + 1).astype(int) * 32
    parts = []
    for n0, n1 in zip(edges[:-1], edges[1:]):
        ws = w[n0 // 16: n1 // 16]                       # whole column tiles: contiguous rows
        ss = s[:, n0:n1].contiguous()
        parts.append((n0, n1, W.wqbmm_a16w4_msd(x, ws, ss, gs)))
    torch.cuda.synchronize()
    for n0, n1, y in parts:
        ref = full[:, n0:n1]
        if exact:
            assert torch.equal(y.view(torch.int16), ref.contiguous().view(torch.int16)), (n0, n1)
        else:
            dd = dict(d, w=d["w"][:, n0:n1], scale=d["scale"][:, n0:n1])
            y32, _ = oracle.matmul(d["x"], d["w_packed"][:, n0 // 2: n1 // 2],
                                   np.ascontiguousarray(d["scale"][:, n0:n1]), gs)
            check_y_elementwise(y.cpu().numpy(), y32, elementwise_bound(dd), f"shard {n0}:{n1}")
