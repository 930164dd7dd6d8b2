"""Per-element bound on the fp16 output y against the oracle's fp32 Y32.

The GPU kernels compute steps 10-11 of the MSD definition (the page
"WeightQuantBatchMatmulExperiment 算子深度解析：A16W4 PerGroup 伪量化 MatMul 的
MSD 算法与双模板流水设计", lpnh.cn/news/2294145, §4.1) from the same exact
integer level sums Y_l as the oracle, in another fp32 order, and round to
fp16.  elementwise_bound() is what that reordering can change; the parity
tests require every element of y to lie within it, beside the rel-L2 and
max-abs bars.
"""
import numpy as np

U32 = 2.0 ** -24   # unit roundoff of fp32


def fp16_half_ulp(v):
    """Half the fp16 spacing at |v| (2^-25 in the subnormal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(a)) - 11)


def elementwise_bound(d, rows=None):
    """Per-element bound on |y - Y32| for a kernel that computes steps 10-11
    from the exact Y_l in another fp32 order than the oracle, then rounds to
    fp16 with RNE.

    Both sides form each group's term from the same exact integers Y_l with a
    handful of fp32 roundings (the kernels fold 1/7.49, 1/(7.49*14.98),
    1/(7.49*14.98^2) and A_max into per-row weights, use fused multiply-adds,
    and sum K-slices in another order), and each sums G terms in fp32.  With
    T = sum_g A_max[m][g] * |s[g][n]| * sum_{k in g} |w[k][n]|, which bounds
    sum_g |Y_group| because sum_l |A_l|/(7.49*14.98^(l-1)) <= 7*(1 + 1/14.98
    + 1/14.98^2)/7.49 < 1, each side's fp32 result is within (G + 12)*u*T of
    the exact value of its own expression (u = 2^-24: at most G - 1 additions
    and about 12 roundings per term), so the two fp32 sums differ by at most
    2*(G + 12)*u*T.  The fused decode kernel adds its K-splits as 2^-24
    fixed-point integers: at most 32 partials, 2^-20 in all.  The kernel's
    fp16 store adds half an fp16 ulp of its own result."""
    import oracle as O
    x, w, s, gs = d["x"], d["w"], d["scale"], d["group_size"]
    if rows is not None:
        x = x[rows]
    G = x.shape[1] // gs
    _, a_max = O.decompose(np.ascontiguousarray(x), gs)
    absw = np.abs(w.astype(np.float64)).reshape(G, gs, -1).sum(axis=1)          # [G][N]
    T = a_max.astype(np.float64) @ (np.abs(s.astype(np.float64)) * absw)       # [R][N]
    delta = 2.0 * (G + 12) * U32 * T + 2.0 ** -20
    return delta


def check_y_elementwise(y, y32, bound, what):
    """|y - Y32| <= half an fp16 ulp of (|Y32| + bound) + bound, everywhere."""
    y = y.astype(np.float64)
    ref = y32.astype(np.float64)
    lim = fp16_half_ulp(np.abs(ref) + bound) + bound
    err = np.abs(y - ref)
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the per-element bound, e.g. "
                             f"[{i[0]}, {i[1]}]: y {y[tuple(i)]!r} Y32 {ref[tuple(i)]!r} bound {lim[tuple(i)]:.3e}")
