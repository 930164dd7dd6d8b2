#!/usr/bin/env python3
"""Throughput of the A16W4 per-group MSD matmul on one MI355X.

One step = one call of the whole operator (steps 1-11: decomposition of x,
integer contraction on MFMA, fp32 combine/accumulate, fp16 store) on one
synthetic batch that is already resident in HBM, with the weights already in
the library's tiled layout and, where the group-size-128 prefill path runs,
also in their operand form (FP6 MFMA operand tiles; both converted once per
weight, outside any timed region).  Those workloads also report the step
without the operand form ("without_operand_weights").  Steps cycle through enough distinct buffer sets (x, w, scale, y)
that their footprint exceeds 512 MiB, twice the 256 MiB MALL, so every step
streams its weights from HBM.  The K timed steps are captured once into a HIP
graph; the headline replays it once between synchronizations.  The steps'
time is taken with HIP events on the launch stream (ms_per_step); the host
wall clock around the same replay is reported beside it.

The headline workload is prefill_m2048 (M = 2048, K = N = 4096, group size
128), the largest configuration of the metric's M = 1..2048 range.  Every
other workload is measured in the same run and nested under "workloads",
each with its own step time, the roofline of its dominant kernel (timed
alone, in its own graph over the same rotating buffer sets) and its
preparation kernel.  The weight-streaming workloads also carry a plain read
of the same byte count (the achievable-bandwidth reference).

Prints ONE JSON line.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload NAME] [--only] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "A16W4 MSD matmul effective TOPS + weight GB/s (% roofline) at M=1..2048"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
I8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (5.0 POP/s)
FP6_PEAK_TOPS = 10100.0      # MI355X dense FP6 MFMA, published (10.1 PFLOP/s): the GEMMs' own dtype
# fp32 vector rate in lane-operations: the published 157.3 TFLOP/s counts an FMA
# as two flops, i.e. 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz operations per second
VALU_F32_OPS_PEAK_T = 256 * 4 * 32 * 2.4e9 / 1e12
MALL_COLD_BYTES = 512 << 20
HEADLINE = "prefill_m2048"
NESTED = ["decode_m1", "decode_m16", "ffn_up_m16", "mid_m64", "mid_m256", "outlier_m128",
          "pages_sample_m1", "tiny"]
REPLAYS = 11                 # extra timed replays of the K-step graph for median / p10 / p90


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_quantized_msd_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic(M, K, N, gs):
    G = K // gs
    w_bytes = K * N // 2
    bytes_total = w_bytes + 2 * G * N + 2 * M * K + 2 * M * N   # W + scale + x + y, once each
    return dict(w_bytes=w_bytes, bytes=bytes_total, eff_ops=2 * M * N * K, exec_i8_ops=6 * M * N * K)


def kernels_of(path, M, K, N, gs):
    """The kernels the library launches for this shape and path: (preparation
    kernel or None, dominant kernel).  Mirrors the dispatch in msd_api.cpp and
    the launchers (msd_decode.hip, msd_decode_gemv.hip, msd_prefill*.hip)."""
    if path == 1:
        if M <= 4:
            return None, "msd_decode_kernel"
        # more column tiles than CUs: workgroups of several tiles (one or two
        # row slices, at most 8 or 4 blocks of 128 rows per wave)
        R, kbw = -(-M // 16), -(-(-(-K // 128)) // 8)
        if N // 16 > 256 and ((R == 1 and kbw <= 8) or (R == 2 and kbw <= 4)):
            return "msd_decode_operands_kernel", "msd_decode_gemv_multi_kernel"
        return "msd_decode_operands_kernel", "msd_decode_gemv_kernel"
    if gs == 128:
        return "msd_prep_kernel", ("msd_gemm_kernel" if prefill_splits(M, K, N) == 1
                                   else "msd_gemm_kernel + msd_splitk_reduce_kernel")
    mblocks = -(-M // 128)
    return "msd_prep64_kernel", ("msd_gemm64w_kernel" if mblocks <= 2 else "msd_gemm64_kernel")


def prefill_bn(M, N):
    """Column block of the group-128 GEMM (msd_prefill.hip prefill_layout):
    64 for at most 32 tiles of 128 columns; else 256 when its rounds of 256
    workgroups cost less, a 256-column tile counting 7/4 of a 128-column one."""
    mb = -(-M // 128)
    t256, t128 = mb * -(-N // 256), mb * -(-N // 128)
    if t128 <= 32:
        return 64
    return 256 if (t128 >= 256 and -(-t256 // 256) * 7 < -(-t128 // 256) * 4) else 128


def prefill64_bn(M, N):
    """Column block of the group-64 GEMM (msd_prefill64.hip prefill64_layout):
    128 with the in-GEMM weight conversion (up to two row blocks), else 256
    when its rounds of 256 workgroups cost less, a 256-column tile counting
    15/8 of a 128-column one."""
    mb = -(-M // 128)
    t256, t128 = mb * -(-N // 256), mb * -(-N // 128)
    return 256 if (mb > 2 and -(-t256 // 256) * 15 < -(-t128 // 256) * 8) else 128


def prefill_splits(M, K, N):
    """K-splits of the group-128 GEMM (msd_prefill.hip set_splits): enough to
    bring the workgroups to about 256 when the tiles alone are fewer, each
    split at least two groups long."""
    G = K // 128
    mb = -(-M // 128)
    bn = prefill_bn(M, N)
    tiles = mb * -(-N // bn)
    s = 1 if tiles >= 256 else 256 // tiles
    s = min(s, max(1, G // 2))
    gps = -(-G // s)
    return -(-G // gps)


def prefill_prep_bytes(M, K, N, gs, operand_weights=False):
    """Algorithmic bytes of the prefill preparation kernel: it reads x and
    writes the level operand tiles (1536 bytes each: 16 rows x 128 k at group
    size 128, 32 rows x 64 k at group size 64) and the level weights (fp32 per
    row and group: A_max * w_1 alone at group size 128, all three at 64); unless the GEMM converts the weights itself (group
    size 64 with at most two 128-row blocks) or reads the weights' operand form
    (group size 128, operand_weights), it also reads the tiled int4 weights and
    writes their operand tiles (columns padded to 256 at group size 128, to
    the GEMM's column block at group size 64)."""
    G = K // gs
    per = 16 if gs == 128 else 32
    mpad = -(-M // 128) * 128
    w_in_gemm = gs == 64 and mpad // 128 <= 2
    if gs == 128:
        npad = -(-N // 256) * 256                  # the weight tiles' 256-column blocks
    else:
        npad = -(-N // prefill64_bn(M, N)) * prefill64_bn(M, N)
    b = 2 * M * K + 1536 * (3 * mpad // per) * G + (4 if gs == 128 else 12) * mpad * G
    if not w_in_gemm and not (operand_weights and gs == 128):
        b += K * N // 2 + 1536 * (npad // per) * G
    return b


def uses_operand_weights(path, gs):
    """The weights' operand form is read by the group-128 prefill path only."""
    return path == 2 and gs == 128


def make_sets(torch, W, M, K, N, gs, nsets, seed, dist, operand_weights=False):
    """Seeded synthetic buffer sets with the workload's distributions, drawn on
    the GPU: x ~ N(0,1) (or U[-3,3]) fp16, int4 weights uniform over their
    range packed two per byte and then converted once into the library's
    tiled layout (outside any timed region, as a deployment converts its
    static weights at load time), and with operand_weights also into their
    operand form; per-group scales uniform / lognormal fp16."""
    gen = torch.Generator(device="cuda")
    sets = []
    G = K // gs
    for i in range(nsets):
        gen.manual_seed(seed * 1000003 + i)
        if dist["x"] == "normal":
            x = torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32)
        else:
            x = (torch.rand((M, K), generator=gen, device="cuda") * 6.0 - 3.0)
        if dist.get("outlier_frac", 0) > 0:
            idx = torch.randperm(K, generator=gen, device="cuda")[: int(round(dist["outlier_frac"] * K))]
            x[:, idx] *= dist["outlier_mult"]
        x = x.to(torch.float16)
        lo, hi = dist["w"]
        wv = torch.randint(lo, hi + 1, (K, N), generator=gen, device="cuda", dtype=torch.int16)
        wu = wv & 0xF
        w_nd = (wu[:, 0::2] | (wu[:, 1::2] << 4)).to(torch.uint8).contiguous()
        w = W.wqbmm_a16w4_tile_weights(w_nd)
        del w_nd
        w_op = W.wqbmm_a16w4_operand_weights(w, K) if operand_weights else None
        kind, p0, p1 = dist["scale"]
        if kind == "uniform":
            s = torch.rand((G, N), generator=gen, device="cuda") * (p1 - p0) + p0
        else:
            s = torch.exp(torch.randn((G, N), generator=gen, device="cuda") * p1 + p0)
        s = s.to(torch.float16)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        sets.append(dict(x=x, w=w, o=w_op, s=s, y=y))
        del wv, wu
    return sets


class Timed:
    """`steps` calls (cycling fn_list) captured into one graph on `stream`
    after `warmup` eager calls, then replayed untimed for at least 0.2 s.
    replay_ms() times one replay with HIP events
    on that stream (per call), between synchronizations, and also returns the
    host wall clock of the same replay."""

    def __init__(self, torch, stream, fn_list, steps, warmup):
        self.torch, self.stream, self.steps = torch, stream, steps
        with torch.cuda.stream(stream):
            for i in range(warmup):
                fn_list[i % len(fn_list)]()
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g, stream=stream, capture_error_mode="relaxed"):
            for i in range(steps):
                fn_list[i % len(fn_list)]()
        # untimed replays: the first uploads the graph; the rest, for at least
        # 0.2 s, bring the clocks to their steady state
        t0 = time.perf_counter()
        for _ in range(1000):
            self.g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= 0.2:
                break

    def replay_ms(self):
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            self.g.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return e0.elapsed_time(e1) / self.steps, (t1 - t0) * 1e3 / self.steps

    def spread(self, n):
        v = sorted(self.replay_ms()[0] for _ in range(n))
        q = lambda p: v[min(len(v) - 1, max(0, int(round(p * (len(v) - 1)))))]
        return {"replays": n, "p10_ms": round(q(0.1), 6), "median_ms": round(statistics.median(v), 6),
                "p90_ms": round(q(0.9), 6)}


def host_cpu():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"model": model, "machine": platform.machine(), "logical_cpus": os.cpu_count(),
            "usable_cpus": usable}


def cpu_baseline(name, M, K, N, gs, seconds):
    """The CPU oracle (plain C, OpenMP over rows) on a bounded sample of the
    workload: a prefix of rows, all of K and N; timed at all usable cores and
    at one thread, about `seconds` each."""
    import numpy as np
    import oracle
    from weight_only_quantized_msd_amd import datagen
    d = datagen.make_inputs(name)
    rows = np.arange(M) if M <= 16 else np.arange(min(M, 16))

    def run(threads):
        oracle.set_num_threads(threads)
        used = oracle.num_threads()
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.matmul(d["x"], d["w_packed"], d["scale"], gs, rows=rows)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 10000:
                break
        return 2.0 * len(rows) * N * K * reps / el / 1e12, used, reps, el

    cpu = host_cpu()
    v_all, used_all, reps_all, el_all = run(cpu["usable_cpus"])
    v_one, _, reps_one, el_one = run(1)
    oracle.set_num_threads(cpu["usable_cpus"])
    return {"value": v_all, "unit": "TOPS", "cores": used_all, "kind": "oracle",
            "sample": (f"{name}: rows {len(rows)} of {M}, all of K={K}, N={N}; "
                       f"{reps_all} oracle call(s) in {el_all:.1f} s at {used_all} threads"),
            "one_thread": {"value": v_one, "unit": "TOPS", "cores": 1,
                           "sample": f"same rows; {reps_one} oracle call(s) in {el_one:.1f} s"},
            "host_cpu": cpu}


def read_traffic(workload, sha):
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None, None
    t = json.load(open(p))
    if t.get("kernel_sources_sha") != sha:
        return None, "stale: kernel sources changed since the counters were taken"
    return t.get("hbm_bytes_per_launch"), t


def plain_read(torch, W, nbytes, steps, warmup):
    """The achievable-bandwidth reference: a plain streaming read of `nbytes`
    (wqbmm_probe_stream_read), over rotating buffers of >= 512 MiB in all."""
    from weight_only_quantized_msd_amd import _lib as L
    nb = -(-nbytes // 16) * 16
    nbuf = max(2, min(256, math.ceil(MALL_COLD_BYTES / nb)))
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    for b in bufs:
        b.fill_(1)
    sink = torch.empty(2048, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    sp = int(stream.cuda_stream)

    def call(b):
        def f():
            rc = L.wqbmm_probe_stream_read_raw(b.data_ptr(), nb, sink.data_ptr(), sp)
            if rc:
                raise RuntimeError(f"wqbmm_probe_stream_read: {rc}")
        return f

    t = Timed(torch, stream, [call(b) for b in bufs], steps, warmup)
    ms, _ = t.replay_ms()
    del bufs
    return {"kernel": "msd_probe_read_kernel", "bytes": nb, "avg_kernel_us": round(ms * 1e3, 3),
            "GBps": round(nb / (ms * 1e-3) / 1e9, 1), "frac_of_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def measure(torch, W, name, args, path_override=0):
    """Everything about one workload: step time (event and wall clock, spread,
    warm-cache), each kernel alone, its roofline."""
    from weight_only_quantized_msd_amd import datagen
    wl = datagen.WORKLOADS[name]
    M, K, N, gs = wl.M, wl.K, wl.N, wl.group_size
    alg = algorithmic(M, K, N, gs)
    path = path_override or W.wqbmm_select_path(M, K, N, gs)
    dist = {"x": wl.x_dist, "w": (wl.w_low, wl.w_high), "scale": wl.scale_dist,
            "outlier_frac": wl.outlier_frac, "outlier_mult": wl.outlier_mult}
    opw = uses_operand_weights(path, gs)
    nsets = max(2, min(256, math.ceil(MALL_COLD_BYTES / alg["bytes"])))
    sets = make_sets(torch, W, M, K, N, gs, nsets, wl.seed, dist, operand_weights=opw)
    stream = torch.cuda.Stream()
    lib = W.lib()
    sptr = int(stream.cuda_stream)
    print(f"[bench] {name}: M={M} K={K} N={N} gs={gs} path={path} sets={nsets} operand_weights={opw}",
          file=sys.stderr, flush=True)

    def optr(st, use):
        return st["o"].data_ptr() if use and st["o"] is not None else None

    def call(st, use_op=True):
        def f():
            rc = lib.wqbmm_a16w4_msd_ex(st["x"].data_ptr(), st["w"].data_ptr(), optr(st, use_op),
                                        st["s"].data_ptr(), gs, M, K, N, st["y"].data_ptr(), path, sptr)
            if rc:
                raise W.WqbmmError(rc, "wqbmm_a16w4_msd_ex")
        return f

    def stage(st, k, use_op=True):
        def f():
            rc = lib.wqbmm_a16w4_msd_profile_stage(st["x"].data_ptr(), st["w"].data_ptr(),
                                                   optr(st, use_op), st["s"].data_ptr(), gs, M, K, N,
                                                   st["y"].data_ptr(), path, k, sptr)
            if rc:
                raise W.WqbmmError(rc, "wqbmm_a16w4_msd_profile_stage")
        return f

    steps, warmup = args.steps, args.warmup
    full = Timed(torch, stream, [call(st) for st in sets], steps, warmup)
    ev_ms, wall_ms = full.replay_ms()
    spread = full.spread(REPLAYS)
    del full
    warm = Timed(torch, stream, [call(sets[0])], steps, warmup)
    warm_ms, _ = warm.replay_ms()
    del warm

    prep_name, main_name = kernels_of(path, M, K, N, gs)
    prep_ms = None
    if prep_name:
        t = Timed(torch, stream, [stage(st, 1) for st in sets], steps, warmup)
        prep_ms, _ = t.replay_ms()
        del t
    t = Timed(torch, stream, [stage(st, 2) for st in sets], steps, warmup)
    kern_ms, _ = t.replay_ms()
    del t
    without = None
    if opw and not args.no_operand_compare:
        # the same workload without the operand form: the preparation kernel
        # converts the tiled weights on every call
        t = Timed(torch, stream, [call(st, False) for st in sets], steps, warmup)
        wo_ms, _ = t.replay_ms()
        del t
        t = Timed(torch, stream, [stage(st, 1, False) for st in sets], steps, warmup)
        wo_prep_ms, _ = t.replay_ms()
        del t
        t = Timed(torch, stream, [stage(st, 2, False) for st in sets], steps, warmup)
        wo_kern_ms, _ = t.replay_ms()
        del t
        without = {"ms_per_step": round(wo_ms, 6),
                   "effective_TOPS": round(alg["eff_ops"] / (wo_ms * 1e-3) / 1e12, 3),
                   "prep_avg_kernel_us": round(wo_prep_ms * 1e3, 3),
                   "prep_algorithmic_bytes_per_launch": prefill_prep_bytes(M, K, N, gs),
                   "main_avg_kernel_us": round(wo_kern_ms * 1e3, 3)}

    G = K // gs
    sha = kernel_sources_sha()
    traffic, tinfo = read_traffic(name, sha)
    extra = {}
    if path == 1:
        if M > 4:
            # contraction kernel: tiled int4 weights, scales, the level operands
            # (three int4 levels per row slice) and level weights once, y
            # R = ceil(M/16) slices of 16 rows, each three int4 levels of every k
            kb = -(-K // 128)
            R = -(-M // 16)
            kbytes = alg["w_bytes"] + 2 * G * N + R * (3 * 1024 * kb + 192 * G) + 2 * M * N
            extra["prep"] = {"kernel": prep_name, "avg_kernel_us": round(prep_ms * 1e3, 3),
                             "algorithmic_bytes_per_launch": 2 * M * K + R * (3 * 1024 * kb + 192 * G)}
        else:
            kbytes = alg["bytes"]
        achieved = kbytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": main_name, "avg_kernel_us": round(kern_ms * 1e3, 3),
                "algorithmic_bytes_per_launch": kbytes}
        if not args.no_plain_read:
            pr = plain_read(torch, W, alg["bytes"], steps, warmup)
            pr["note"] = "plain streaming read of the workload's algorithmic bytes (W + scale + x + y)"
            extra["plain_read_reference"] = pr
            roof["frac_of_plain_read"] = round(pr["avg_kernel_us"] / (kern_ms * 1e3), 4)
    else:
        # The GEMM contracts on FP6 (e2m3) MFMAs, so its roofline peak is the
        # dense FP6 rate; the fraction of the int8 rate is reported beside it.
        # It is timed alone over the rotating sets with the operand tiles as
        # the preparation kernel of the same shape left them (MALL-resident,
        # as in a full step, where the GEMM follows its preparation kernel).
        # (with a K-split the timed stage is the GEMM and its reduction)
        achieved = alg["exec_i8_ops"] / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP6_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP6_PEAK_TOPS, 4), "traffic": traffic,
                "kernel": main_name, "mfma_dtype": "fp6 e2m3",
                "avg_kernel_us": round(kern_ms * 1e3, 3),
                "algorithmic_ops_per_launch": alg["exec_i8_ops"],
                "frac_of_i8_peak": round(achieved / I8_PEAK_TOPS, 4),
                "operands": "MALL-resident operand tiles, as the preparation kernel leaves them"}
        # The GEMMs spend more SIMD time on the fp32 combine of step 10 than on
        # the MFMA: 4 fp32 operations per (row, column, group) -- three for
        # the level weights, one for the scale and the running sum.
        combine_ops = 4 * M * N * G
        alu = combine_ops / (kern_ms * 1e-3) / 1e12
        extra["alu_view"] = {"bound": "alu", "ops_per_launch": combine_ops, "achieved": round(alu, 2),
                             "peak": round(VALU_F32_OPS_PEAK_T, 2), "unit": "T fp32 op/s",
                             "frac": round(alu / VALU_F32_OPS_PEAK_T, 4)}
        prep_bytes = prefill_prep_bytes(M, K, N, gs, opw)
        extra["prep"] = {"kernel": prep_name, "avg_kernel_us": round(prep_ms * 1e3, 3),
                         "algorithmic_bytes_per_launch": prep_bytes,
                         "achieved_GBps": round(prep_bytes / (prep_ms * 1e-3) / 1e9, 1)}
        if opw:
            roof["operands"] = ("x level tiles MALL-resident, as the preparation kernel leaves them; "
                                "weight tiles from the weights' operand form in HBM")
            if without:
                extra["without_operand_weights"] = without
    if isinstance(tinfo, dict):
        extra["traffic_detail"] = {k: tinfo[k] for k in tinfo if k not in ("kernel_sources_sha", "commands")}
    elif isinstance(tinfo, str):
        extra["traffic_detail"] = tinfo
    t_s = ev_ms * 1e-3
    res = {
        "config": {"workload": f"{name}: M={M} K={K} N={N} group_size={gs}", "M": M, "K": K, "N": N,
                   "group_size": gs, "path": {1: "decode", 2: "prefill"}[path],
                   "weights": ("tiled int4 + operand form (FP6), both converted once before timing"
                               if opw else "tiled int4, converted once before timing"),
                   "buffer_sets": nsets, "footprint_MiB": round(nsets * alg["bytes"] / 2 ** 20, 1)},
        "ms_per_step": round(ev_ms, 6),
        "wall_ms_per_step": round(wall_ms, 6),
        "step_spread": spread,
        "warm_cache_ms_per_step": round(warm_ms, 6),
        "effective_TOPS": round(alg["eff_ops"] / t_s / 1e12, 3),
        "weight_GBps": round(alg["w_bytes"] / t_s / 1e9, 1),
        "weight_GBps_frac_of_hbm": round(alg["w_bytes"] / t_s / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_algorithmic_GBps": round(alg["bytes"] / t_s / 1e9, 1),
        "exec_i8_TOPS": round(alg["exec_i8_ops"] / t_s / 1e12, 2),
        "step_frac_of_i8_peak": round(alg["exec_i8_ops"] / t_s / 1e12 / I8_PEAK_TOPS, 4),
        "roofline": roof,
    }
    res.update(extra)
    del sets
    torch.cuda.synchronize()
    return res


def probe_overlap(torch, steps, warmup, iters=2000):
    """The MFMA / VALU co-issue probe (wqbmm_probe_mfma_valu): the time of
    each mode per launch (HIP events over a graph of `steps` launches, median
    of 5 replays), and the ratios that say whether the two kinds of work
    overlap on a SIMD: 1.0 for `both_in_each_wave` / (mfma + fma) means no
    overlap."""
    from weight_only_quantized_msd_amd import _lib as L
    out = torch.empty(262144, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    sp = int(stream.cuda_stream)
    res = {}
    for mode, name in [(0, "mfma_only"), (1, "fma_only"), (2, "both_in_each_wave"), (3, "one_kind_per_wave"),
                       (4, "both_in_each_wave_barrier_per_round"), (6, "one_wave_per_simd_mfma_only"),
                       (7, "one_wave_per_simd_fma_only"), (5, "one_wave_per_simd_both"),
                       (9, "four_waves_per_simd_mfma_only"), (10, "four_waves_per_simd_fma_only"),
                       (8, "four_waves_per_simd_both")]:
        def f(mode=mode):
            rc = L.wqbmm_probe_mfma_valu_raw(mode, iters, out.data_ptr(), sp)
            if rc:
                raise RuntimeError(f"wqbmm_probe_mfma_valu: {rc}")
        t = Timed(torch, stream, [f], steps, warmup)
        res[name] = round(t.spread(5)["median_ms"] * 1e3, 2)
        del t
    alone = res["mfma_only"] + res["fma_only"]
    return {"unit": "us per launch", "rounds": iters,
            "round": "12 FP6 16x16x128 MFMAs and/or 64 fp32 FMAs per wave, 2 waves per SIMD",
            "us": res,
            "both_in_each_wave_over_sum": round(res["both_in_each_wave"] / alone, 3),
            "one_kind_per_wave_over_sum": round(res["one_kind_per_wave"] / alone, 3),
            "both_in_each_wave_barrier_per_round_over_sum":
                round(res["both_in_each_wave_barrier_per_round"] / alone, 3),
            "one_wave_per_simd_both_over_sum":
                round(res["one_wave_per_simd_both"] / (res["one_wave_per_simd_mfma_only"]
                                                      + res["one_wave_per_simd_fma_only"]), 3),
            "four_waves_per_simd_both_over_sum":
                round(res["four_waves_per_simd_both"] / (res["four_waves_per_simd_mfma_only"]
                                                        + res["four_waves_per_simd_fma_only"]), 3)}


SHAPES_DEFAULT = [(128, 4096, 4096, 128), (256, 4096, 4096, 128), (512, 4096, 4096, 128),
                  (1024, 4096, 4096, 128), (1536, 4096, 4096, 128), (2048, 4096, 4096, 128),
                  (3072, 4096, 4096, 128), (512, 4096, 11008, 128), (256, 4096, 8192, 128),
                  (384, 8192, 28672, 64), (1024, 4096, 11008, 64)]


def shapes(torch, W, shape_list, steps, warmup):
    """Prefill-path step time (median of 5 replays, MALL-cold) at arbitrary
    shapes, each kernel alone beside it, with the weights' operand form and,
    at group size 128, without it.  Returns a list of rows."""
    rows = []
    lib = W.lib()
    for M, K, N, gs in shape_list:
        alg = algorithmic(M, K, N, gs)
        nsets = max(2, min(64, math.ceil(MALL_COLD_BYTES / alg["bytes"])))
        dist = {"x": "normal", "w": (-8, 7), "scale": ("uniform", 0.005, 0.02)}
        sets = make_sets(torch, W, M, K, N, gs, nsets, 7, dist, operand_weights=gs == 128)
        stream = torch.cuda.Stream()
        sptr = int(stream.cuda_stream)
        row = {"M": M, "K": K, "N": N, "group_size": gs,
               "column_block": prefill_bn(M, N) if gs == 128 else prefill64_bn(M, N),
               "k_splits": prefill_splits(M, K, N) if gs == 128 else 1}
        for use in ((True, False) if gs == 128 else (False,)):
            def call(st, k=0, use=use):
                def f():
                    op = st["o"].data_ptr() if use else None
                    if k == 0:
                        rc = lib.wqbmm_a16w4_msd_ex(st["x"].data_ptr(), st["w"].data_ptr(), op,
                                                    st["s"].data_ptr(), gs, M, K, N, st["y"].data_ptr(),
                                                    2, sptr)
                    else:
                        rc = lib.wqbmm_a16w4_msd_profile_stage(st["x"].data_ptr(), st["w"].data_ptr(), op,
                                                               st["s"].data_ptr(), gs, M, K, N,
                                                               st["y"].data_ptr(), 2, k, sptr)
                    if rc:
                        raise W.WqbmmError(rc, "shapes")
                return f
            print(f"[shapes] M={M} K={K} N={N} gs={gs} operand_form={use}", file=sys.stderr, flush=True)
            t = Timed(torch, stream, [call(st) for st in sets], steps, warmup)
            step = t.spread(5)["median_ms"]
            del t
            t = Timed(torch, stream, [call(st, 1) for st in sets], steps, warmup)
            prep = t.replay_ms()[0]
            del t
            t = Timed(torch, stream, [call(st, 2) for st in sets], steps, warmup)
            main = t.replay_ms()[0]
            del t
            key = "with_operand_form" if use else ("without_operand_form" if gs == 128 else "step")
            row[key] = {"step_us": round(step * 1e3, 2), "prep_us": round(prep * 1e3, 2),
                        "gemm_us": round(main * 1e3, 2),
                        "effective_TOPS": round(alg["eff_ops"] / (step * 1e-3) / 1e12, 1)}
        rows.append(row)
        del sets
        torch.cuda.synchronize()
    return rows


SWEEP_M = [8, 12, 16, 24, 32, 48, 64, 80, 96, 128]
SWEEP_SHAPES = [("K4096_N4096_g128", 4096, 4096, 128), ("K4096_N11008_g128", 4096, 11008, 128),
                ("K8192_N28672_g64", 8192, 28672, 64)]


def sweep(torch, W, args):
    """Decode-vs-prefill split: the step time of each kernel path at
    M = 8..128 on the decode shape (K = N = 4096, group size 128), a wider
    group-128 shape (K = 4096, N = 11008) and the outlier shape (K = 8192,
    N = 28672, group size 64), MALL-cold as above,
    with each path's kernels timed alone (the group-128 prefill path with the
    weights' operand form).  Returns a list of rows."""
    from weight_only_quantized_msd_amd import datagen  # noqa: F401
    rows = []
    lib = W.lib()
    for label, K, N, gs in SWEEP_SHAPES:
        for M in SWEEP_M:
            alg = algorithmic(M, K, N, gs)
            nsets = max(2, min(64, math.ceil(MALL_COLD_BYTES / alg["bytes"])))
            dist = {"x": "normal", "w": (-8, 7), "scale": ("uniform", 0.005, 0.02)}
            sets = make_sets(torch, W, M, K, N, gs, nsets, 7, dist, operand_weights=gs == 128)
            stream = torch.cuda.Stream()
            sptr = int(stream.cuda_stream)
            for path in (1, 2):
                st0 = sets[0]
                rc = lib.wqbmm_a16w4_msd_path(st0["x"].data_ptr(), st0["w"].data_ptr(), st0["s"].data_ptr(),
                                              gs, M, K, N, st0["y"].data_ptr(), path, sptr)
                if rc == W.WQBMM_ERR_INVALID:      # the decode path's row limit
                    continue
                if rc:
                    raise W.WqbmmError(rc, "sweep")
                def call(st, k=0):
                    def f():
                        op = st["o"].data_ptr() if st["o"] is not None else None
                        if k == 0:
                            rc = lib.wqbmm_a16w4_msd_ex(st["x"].data_ptr(), st["w"].data_ptr(), op,
                                                        st["s"].data_ptr(), gs, M, K, N,
                                                        st["y"].data_ptr(), path, sptr)
                        else:
                            rc = lib.wqbmm_a16w4_msd_profile_stage(st["x"].data_ptr(), st["w"].data_ptr(), op,
                                                                   st["s"].data_ptr(), gs, M, K, N,
                                                                   st["y"].data_ptr(), path, k, sptr)
                        if rc:
                            raise W.WqbmmError(rc, "sweep")
                    return f
                print(f"[sweep] {label} M={M} path={path}", file=sys.stderr, flush=True)
                t = Timed(torch, stream, [call(st) for st in sets], args.steps, args.warmup)
                step_ms = t.spread(5)["median_ms"]
                del t
                prep_name, main_name = kernels_of(path, M, K, N, gs)
                prep_ms = None
                if prep_name:
                    t = Timed(torch, stream, [call(st, 1) for st in sets], args.steps, args.warmup)
                    prep_ms = t.replay_ms()[0]
                    del t
                t = Timed(torch, stream, [call(st, 2) for st in sets], args.steps, args.warmup)
                main_ms = t.replay_ms()[0]
                del t
                rows.append({"shape": label, "M": M, "K": K, "N": N, "group_size": gs,
                             "path": {1: "decode", 2: "prefill"}[path],
                             "selected": W.wqbmm_select_path(M, K, N, gs) == path,
                             "step_us": round(step_ms * 1e3, 3),
                             "effective_TOPS": round(alg["eff_ops"] / (step_ms * 1e-3) / 1e12, 2),
                             "weight_GBps": round(alg["w_bytes"] / (step_ms * 1e-3) / 1e9, 1),
                             "prep_kernel": prep_name,
                             "prep_us": None if prep_ms is None else round(prep_ms * 1e3, 3),
                             "main_kernel": main_name, "main_us": round(main_ms * 1e3, 3)})
            del sets
            torch.cuda.synchronize()
    return rows


def main():
    from weight_only_quantized_msd_amd import datagen
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(datagen.WORKLOADS),
                    help="the headline workload (default prefill_m2048)")
    ap.add_argument("--only", action="store_true", help="measure the headline workload alone")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 decode, 2 prefill (headline only)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plain-read", action="store_true")
    ap.add_argument("--no-operand-compare", action="store_true",
                    help="skip the group-128 prefill step without the weights' operand form")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: the decode-vs-prefill M sweep (one JSON line)")
    ap.add_argument("--shapes", nargs="?", const="default", default=None,
                    help="instead of the bench line: the prefill path at shapes 'M,K,N,gs;...' "
                         "(default: a built-in list), with and without the weights' operand form")
    ap.add_argument("--probe-overlap", action="store_true",
                    help="instead of the bench line: the MFMA / VALU co-issue probe (one JSON line)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}). Run with --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import weight_only_quantized_msd_amd as W
    torch.cuda.init()

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.shapes:
        lst = SHAPES_DEFAULT if args.shapes == "default" else [
            tuple(int(v) for v in item.split(",")) for item in args.shapes.split(";") if item]
        print(json.dumps({"shapes": shapes(torch, W, lst, args.steps, args.warmup), "steps": args.steps,
                          "kernel_sources_sha": kernel_sources_sha()}), flush=True)
        return

    if args.probe_overlap:
        print(json.dumps({"probe_overlap": probe_overlap(torch, args.steps, args.warmup),
                          "kernel_sources_sha": kernel_sources_sha()}), flush=True)
        return

    if args.sweep:
        print(json.dumps({"sweep": sweep(torch, W, args), "steps": args.steps,
                          "kernel_sources_sha": kernel_sources_sha()}), flush=True)
        return

    head = measure(torch, W, args.workload, args, args.path)
    nested = {}
    if not args.only:
        for name in NESTED + ([HEADLINE] if args.workload != HEADLINE else []):
            if name != args.workload:
                nested[name] = measure(torch, W, name, args)

    wl = datagen.WORKLOADS[args.workload]
    alg = algorithmic(wl.M, wl.K, wl.N, wl.group_size)
    out = {
        "metric": METRIC,
        "value": head["effective_TOPS"],
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if head["config"]["path"] == "decode" else "fp6",
        "data": "synthetic",
        "config": dict(head["config"], submission="captured HIP graph of the K steps; ms_per_step from "
                       "HIP events on the launch stream, wall_ms_per_step from the host clock"),
        "timing": {"ms_per_step": "HIP events around one replay of the K-step graph, per step",
                   "wall_ms_per_step": "host clock around the same replay, between synchronizations",
                   "step_spread": f"per-step time of {REPLAYS} further replays: p10 / median / p90",
                   "warm_cache_ms_per_step": "K steps on one buffer set (weights MALL-resident), labelled warm"},
        "kernel_sources_sha": kernel_sources_sha(),
    }
    for k, v in head.items():
        if k not in ("config", "ms_per_step"):
            out[k] = v
    out["value"] = round(alg["eff_ops"] / (head["ms_per_step"] * 1e-3) / 1e12, 3)
    if nested:
        out["workloads"] = nested
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, wl.M, wl.K, wl.N, wl.group_size, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
