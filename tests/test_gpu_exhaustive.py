"""Steps 1-8 on every pair of fp16 values that can meet in the decomposition.

Method: the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4 PerGroup
伪量化 MatMul 的 MSD 算法与双模板流水设计" (lpnh.cn/news/2294145), §4.1 steps
1-8.  An element's levels depend only on its own value a and its group's
maximum A_max (with |a| <= A_max), both fp16.  The device divides tmp1 =
rn(7.49*a) by A_max with a refined reciprocal and one remainder correction
rather than a full division; this test shows that it gives the oracle's
correctly rounded quotient for every such pair, by comparing A_int and A_max
over all of them (about 1.0e9 pairs: every positive finite fp16 A_max, every
fp16 a of either sign with |a| <= A_max).

Each group holds A_max itself in element 0 and the values a after it
(zero-padded), one group per row.  The decode kernels and the prepass export
decompose with the same device routine (msd_decompose8); the prefill
preparation kernels pack the same routine's levels into FP6 MFMA operand
tiles.  The prefill path is read back through its Y_int export with identity
weights (K = N = group size, w[k][n] = 1 if k == n else 0), which makes
Y_l[m][n] = A_l[m][n] exactly, so every GPU decomposition is compared with
the oracle over all pairs, at group sizes 128 and 64.  Inputs are built on the
device (they are plain bit patterns), compared on the device against the
oracle's output.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

GS = 128
BMAX = 0x7BFF          # largest finite positive fp16 bit pattern
NCHUNKS = 16


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_msd_amd as W  # noqa: F401
    W.lib()
    return torch


def chunk_bounds():
    # pairs up to pattern b grow like b^2: equal-work chunks
    b = [int(round(1 + BMAX * (i / NCHUNKS) ** 0.5)) for i in range(NCHUNKS + 1)]
    b[-1] = BMAX + 1
    return b


def build_chunk(torch, b0, b1, gs=GS):
    """fp16 [G][gs]: for each A_max pattern b in [b0, b1), the values with
    patterns 0..b and 0x8001..0x8000+b (all a with |a| <= A_max), gs - 1 per
    group after A_max, zero-padded."""
    per = gs - 1
    dev = "cuda"
    bs = torch.arange(b0, b1, device=dev, dtype=torch.int64)
    n = 2 * bs + 1
    g = (n + per - 1) // per
    G = int(g.sum().item())
    slots = g * per
    blk = torch.repeat_interleave(torch.arange(bs.numel(), device=dev), slots)
    off = torch.cumsum(slots, 0) - slots
    r = torch.arange(G * per, device=dev, dtype=torch.int64) - off[blk]
    bb = bs[blk]
    val = torch.where(r <= bb, r, torch.where(r <= 2 * bb, 0x8000 + (r - bb), torch.zeros_like(r)))
    x = torch.empty((G, gs), dtype=torch.int64, device=dev)
    x[:, 0] = torch.repeat_interleave(bs, g)
    x[:, 1:] = val.view(G, per)
    x = torch.where(x >= 0x8000, x - 0x10000, x).to(torch.int16)   # bit patterns as int16
    return x.view(torch.float16).contiguous(), int(n.sum().item())


def test_build_chunk_covers_every_pair(torch_dev):
    """The construction itself, on a small range: every (A_max, a) pair once."""
    torch = torch_dev
    x, total = build_chunk(torch, 1, 40)
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    seen = set()
    for row in xb:
        amax = int(row[0])
        for v in row[1:]:
            seen.add((amax, int(v)))
    want = set()
    for b in range(1, 40):
        for v in list(range(0, b + 1)) + [0x8000 + j for j in range(1, b + 1)]:
            want.add((b, v))
    assert want <= seen and len(want) == total
    assert all((a == b) or (a & 0x7FFF) <= b for (b, a) in seen)   # padding zeros only


def identity_weights(torch, n):
    """Tiled int4 identity of size n x n (w[k][k] = 1)."""
    import weight_only_quantized_msd_amd as W
    w = np.zeros((n, n), np.int16)
    np.fill_diagonal(w, 1)
    u = w & 0xF
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    return W.wqbmm_a16w4_tile_weights(torch.from_numpy(packed).cuda())


@pytest.mark.parametrize("gs", [128, 64])
def test_every_path_decomposes_exhaustively(torch_dev, gs):
    """All (A_max, a) pairs through the prepass export and through the prefill
    path's preparation kernel (read back as Y_int against identity weights),
    both against the oracle."""
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    eye = identity_weights(torch, gs)
    bounds = chunk_bounds()
    pairs = 0
    for ci in range(NCHUNKS):
        b0, b1 = bounds[ci], bounds[ci + 1]
        x, n = build_chunk(torch, b0, b1, gs)
        ra, rm = oracle.decompose(x.cpu().numpy(), gs)
        ref = torch.from_numpy(ra).cuda()
        a_int, a_max = W.wqbmm_a16w4_msd_prepass(x, gs)
        yi = W.wqbmm_a16w4_msd_yint(x, eye, gs, 0, 1, path=W.WQBMM_PATH_PREFILL)
        torch.cuda.synchronize()
        same_pre = torch.equal(a_int, ref)
        same_max = torch.equal(a_max.view(torch.int32), torch.from_numpy(rm.view(np.int32)).cuda())
        same_fill = torch.equal(yi[0], ref.to(torch.int32))
        pairs += n
        print(f"[exhaustive gs={gs}] A_max patterns [{b0:#06x}, {b1:#06x}): {n} pairs, prepass "
              f"{'equal' if same_pre else 'DIFFER'}, prefill {'equal' if same_fill else 'DIFFER'}", flush=True)
        if not same_fill:
            diff = (yi[0] != ref.to(torch.int32)).nonzero()[:5].cpu().numpy()
            xs = x.view(torch.int16).cpu().numpy().view(np.uint16)
            cases = [(hex(int(xs[r, 0])), hex(int(xs[r, c]))) for (_, r, c) in diff]
            pytest.fail(f"prefill A_int differs, e.g. (A_max, a) = {cases}")
        assert same_pre and same_max
        del x, a_int, a_max, yi, ref
    assert pairs == sum(2 * b + 1 for b in range(1, BMAX + 1))
