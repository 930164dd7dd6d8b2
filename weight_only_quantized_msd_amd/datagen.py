"""Seeded synthetic inputs for the A16W4 per-group MSD matmul.

This module is the ONLY code shared by the CPU oracle (``oracle/``) and the
HIP path: it draws inputs and lays them out in the boundary's storage format.
It holds none of the method's arithmetic (no A_max, no decomposition, no
contraction, no combine) -- just numpy random draws and the int4 storage
packing that the operator's input format prescribes.

Workloads follow the operator spec of the WeightQuantBatchMatmulExperiment
page ("WeightQuantBatchMatmulExperiment 算子深度解析：A16W4 PerGroup 伪量化
MatMul 的 MSD 算法与双模板流水设计", lpnh.cn/news/2294145):

* §4.2 (算子规格): x1 is M x K fp16, x2 is K x N int4, antiquant_scale is
  GroupNum x N fp16 (groups run along K), y is M x N fp16, all ND (row-major).
* §4.3 (样例的默认运行规格): int4 weights are stored two per byte.  The page
  does not say which nibble holds which column; we store column 2j in the low
  nibble and column 2j+1 in the high nibble of byte (k, j), two's complement.

Draw recipe (per config, numpy ``default_rng(seed)``, PCG64), in this order:
X, then W, then scale, then (outlier config only) the outlier channels.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    group_size: int
    seed: int
    x_dist: str = "normal"          # "normal" -> N(0,1); "uniform3" -> U[-3,3]
    w_low: int = -8                 # inclusive
    w_high: int = 7                 # inclusive
    scale_dist: tuple = ("uniform", 0.005, 0.02)
    outlier_frac: float = 0.0       # fraction of K channels multiplied by outlier_mult
    outlier_mult: float = 50.0
    note: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.K // self.group_size


# The five measured workloads, two points in the middle of the M range and
# the page's own sample shape (§4.3).
WORKLOADS = {
    "tiny": Workload("tiny", 4, 256, 256, 64, seed=0,
                     note="smallest parity case, several groups and tiles"),
    "decode_m1": Workload("decode_m1", 1, 4096, 4096, 128, seed=1,
                          note="GEMV-like decode, HBM-bound on int4 weight bytes"),
    "decode_m16": Workload("decode_m16", 16, 4096, 4096, 128, seed=2,
                           note="batched decode, HBM-bound"),
    "ffn_up_m16": Workload("ffn_up_m16", 16, 4096, 11008, 128, seed=3,
                           note="FFN up-projection decode"),
    "prefill_m2048": Workload("prefill_m2048", 2048, 4096, 4096, 128, seed=4,
                              note="prefill, MFMA-bound (3M effective rows)"),
    "outlier_m128": Workload("outlier_m128", 128, 8192, 28672, 64, seed=5,
                             scale_dist=("lognormal", -4.5, 0.3),
                             outlier_frac=0.01, outlier_mult=50.0,
                             note="1% of K channels x50; lognormal scales"),
    # The middle of the M = 1..2048 range at the decode shape (same
    # distributions as decode_m16): where the kernel paths meet.
    "mid_m64": Workload("mid_m64", 64, 4096, 4096, 128, seed=7,
                        note="64 rows, K = N = 4096: the row-sliced decode contraction"),
    "mid_m256": Workload("mid_m256", 256, 4096, 4096, 128, seed=8,
                         note="256 rows, K = N = 4096: two 128-row blocks of the prefill GEMM"),
    # The page's sample: M=1, N=12288, K=8192, groupSize=128, x ~ U[-3,3],
    # w in [-7,7], scale ~ U[-3,3] (negative scales allowed).
    "pages_sample_m1": Workload("pages_sample_m1", 1, 8192, 12288, 128, seed=6,
                                x_dist="uniform3", w_low=-7, w_high=7,
                                scale_dist=("uniform", -3.0, 3.0),
                                note="the WeightQuantBatchMatmulExperiment page's §4.3 sample shape"),
}


def pack_int4(w: np.ndarray) -> np.ndarray:
    """int8 [K][N] with values in [-8,7] -> uint8 [K][N/2] storage format.

    Byte (k, j) holds column 2j in bits 0..3 and column 2j+1 in bits 4..7,
    each as a 4-bit two's-complement field.
    """
    w = np.asarray(w)
    if w.ndim != 2 or w.shape[1] % 2:
        raise ValueError("pack_int4 expects a 2-D array with an even column count")
    if w.min(initial=0) < -8 or w.max(initial=0) > 7:
        raise ValueError("int4 values must lie in [-8, 7]")
    u = w.astype(np.int16) & 0xF
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def make_inputs(wl: Workload | str, seed: int | None = None, M: int | None = None):
    """Draw (x fp16 [M][K], w int8 [K][N], w_packed uint8 [K][N/2], scale fp16 [G][N]).

    ``seed`` overrides the workload's seed; ``M`` overrides the row count
    (used for reduced-size parity cases that keep the workload's K, N, gs and
    value distributions).
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    M = wl.M if M is None else int(M)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    G = wl.K // wl.group_size

    if wl.x_dist == "normal":
        x32 = rng.standard_normal((M, wl.K), dtype=np.float32)
    elif wl.x_dist == "uniform3":
        x32 = rng.uniform(-3.0, 3.0, (M, wl.K)).astype(np.float32)
    else:
        raise ValueError(wl.x_dist)

    w = rng.integers(wl.w_low, wl.w_high + 1, (wl.K, wl.N), dtype=np.int8)

    kind, p0, p1 = wl.scale_dist
    if kind == "uniform":
        scale = rng.uniform(p0, p1, (G, wl.N)).astype(np.float16)
    elif kind == "lognormal":
        scale = rng.lognormal(p0, p1, (G, wl.N)).astype(np.float16)
    else:
        raise ValueError(kind)

    if wl.outlier_frac > 0:
        n_out = int(round(wl.outlier_frac * wl.K))
        idx = rng.choice(wl.K, n_out, replace=False)
        x32[:, idx] *= np.float32(wl.outlier_mult)   # before the fp16 cast

    x = x32.astype(np.float16)
    return dict(x=x, w=w, w_packed=pack_int4(w), scale=scale,
                M=M, K=wl.K, N=wl.N, group_size=wl.group_size, name=wl.name)


def random_case(M: int, K: int, N: int, group_size: int, seed: int,
                x_scale: float = 1.0):
    """Unnamed seeded case with the default distributions (N(0,1) x, int4 w,
    U[0.005,0.02] scale).  Used for ragged and edge-case shapes."""
    wl = Workload("adhoc", M, K, N, group_size, seed)
    d = make_inputs(wl)
    if x_scale != 1.0:
        d["x"] = (d["x"].astype(np.float32) * np.float32(x_scale)).astype(np.float16)
    return d
