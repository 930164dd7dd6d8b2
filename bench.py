#!/usr/bin/env python3
"""Throughput of the A16W4 per-group MSD matmul on one MI355X.

One step = one call of the whole operator (steps 1-11: decomposition of x,
integer contraction on MFMA, fp32 combine/accumulate, fp16 store) on one
synthetic batch that is already resident in HBM, with weights already in the
library's tiled layout (converted once per weight, outside the timed region).  Steps cycle through enough distinct buffer sets
(x, w, scale, y) that their footprint exceeds 512 MiB, twice the 256 MiB
MALL, so every step streams its weights from HBM.  The K timed steps are
captured once into a HIP graph and replayed, so the GPU runs them back to
back without Python launch overhead in between; the kernels are the same as
in an eager call.

Prints ONE JSON line:  metric / value (effective TOPS = 2*M*N*K per step per
second) / ms_per_step / roofline of the dominant kernel (HIP events on the
launch stream) / cpu_baseline (the CPU oracle on the host cores).

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "A16W4 MSD matmul effective TOPS + weight GB/s (% roofline) at M=1..2048"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
I8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (5.0 POP/s)
FP6_PEAK_TOPS = 10100.0      # MI355X dense FP6 MFMA, published (10.1 PFLOP/s): the GEMM's own dtype
# fp32 vector rate in lane-operations: the published 157.3 TFLOP/s counts an FMA
# as two flops, i.e. 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz operations per second
VALU_F32_OPS_PEAK_T = 256 * 4 * 32 * 2.4e9 / 1e12
MALL_COLD_BYTES = 512 << 20


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


def make_sets(torch, W, M, K, N, gs, nsets, seed, dist):
    """Seeded synthetic buffer sets with the workload's distributions, drawn on
    the GPU: x ~ N(0,1) (or U[-3,3]) fp16, int4 weights uniform over their
    range packed two per byte and then converted once into the library's
    tiled layout (outside any timed region, as a deployment converts its
    static weights at load time), per-group scales uniform / lognormal fp16."""
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
        kind, p0, p1 = dist["scale"]
        if kind == "uniform":
            s = torch.rand((G, N), generator=gen, device="cuda") * (p1 - p0) + p0
        else:
            s = torch.exp(torch.randn((G, N), generator=gen, device="cuda") * p1 + p0)
        s = s.to(torch.float16)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        sets.append(dict(x=x, w=w, s=s, y=y))
        del wv, wu
    return sets


def timed_graph(torch, stream, fn_list, steps, warmup):
    """Eager warmup, capture `steps` calls (cycling fn_list) into one graph,
    replay once untimed, then time one replay: wall clock between
    synchronizations, and HIP events on the launch stream."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn_list[i % len(fn_list)]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream, capture_error_mode="relaxed"):
        for i in range(steps):
            fn_list[i % len(fn_list)]()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def prefill_prep_bytes(M, K, N, gs):
    """Algorithmic bytes of the prefill preparation kernel: it reads x and
    writes the level operand tiles (1536 bytes each: 16 rows x 128 k at group
    size 128, 32 rows x 64 k at group size 64) and the level weights (fp32,
    three per row and group); unless the GEMM converts the weights itself (group
    size 64 with at most two 128-row blocks), it also reads the tiled int4
    weights and writes their operand tiles (columns padded to the GEMM's
    column block of 256, or 128 when 256 would give fewer than 256 tiles)."""
    G = K // gs
    per = 16 if gs == 128 else 32
    mpad = -(-M // 128) * 128
    w_in_gemm = gs == 64 and mpad // 128 <= 2
    bn = 256 if (not w_in_gemm and (mpad // 128) * -(-N // 256) >= 256) else 128
    npad = -(-N // bn) * bn
    b = 2 * M * K + 1536 * (3 * mpad // per) * G + 12 * mpad * G
    if not w_in_gemm:
        b += K * N // 2 + 1536 * (npad // per) * G
    return b


def cpu_baseline(name, M, K, N, gs, seconds):
    import numpy as np
    import oracle
    from weight_only_quantized_msd_amd import datagen
    d = datagen.make_inputs(name)
    # bounded sample: all rows for small M, else a prefix of rows
    rows = np.arange(M) if M <= 16 else np.arange(min(M, 8))
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.matmul(d["x"], d["w_packed"], d["scale"], gs, rows=rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 10000:
            break
    ops = 2.0 * len(rows) * N * K * reps
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": ops / el / 1e12, "unit": "TOPS", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{name}: rows {len(rows)} of {M}, all of K={K}, N={N}; {reps} oracle call(s) in {el:.1f} s",
            "host_cpu": cpu, "seconds": round(el, 2)}


def read_traffic(workload, sha):
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None, None
    t = json.load(open(p))
    if t.get("kernel_sources_sha") != sha:
        return None, "stale: kernel sources changed since the counters were taken"
    return t.get("hbm_bytes_per_launch"), t


def main():
    from weight_only_quantized_msd_amd import datagen
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_m16", choices=sorted(datagen.WORKLOADS))
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 decode, 2 prefill")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    wl = datagen.WORKLOADS[args.workload]
    M, K, N, gs = wl.M, wl.K, wl.N, wl.group_size
    alg = algorithmic(M, K, N, gs)
    path = args.path or W.wqbmm_select_path(M, K, N, gs)
    dist = {"x": wl.x_dist, "w": (wl.w_low, wl.w_high), "scale": wl.scale_dist,
            "outlier_frac": wl.outlier_frac, "outlier_mult": wl.outlier_mult}
    set_bytes = alg["bytes"]
    nsets = max(2, min(256, math.ceil(MALL_COLD_BYTES / set_bytes)))
    torch.cuda.init()
    sets = make_sets(torch, W, M, K, N, gs, nsets, wl.seed, dist)
    stream = torch.cuda.Stream()
    lib = W.lib()
    sptr = int(stream.cuda_stream)

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def call(st):
        def f():
            rc = lib.wqbmm_a16w4_msd_path(st["x"].data_ptr(), st["w"].data_ptr(), st["s"].data_ptr(),
                                          gs, M, K, N, st["y"].data_ptr(), path, sptr)
            if rc:
                raise W.WqbmmError(rc, "wqbmm_a16w4_msd_path")
        return f

    ms_step, ev_step = timed_graph(torch, stream, [call(st) for st in sets], args.steps, args.warmup)
    t_s = ms_step * 1e-3
    value = alg["eff_ops"] / t_s / 1e12

    extra = {}
    sha = kernel_sources_sha()
    traffic, tinfo = read_traffic(args.workload, sha)

    # The path's kernels timed alone, each in its own graph over the rotating
    # sets (MALL-cold): stage 1 = the operand kernel, stage 2 = the
    # contraction on the operands the last stage 1 left in this stream's
    # workspace (rotating scale, y and, for the weights, w).  The fused decode
    # kernel (M <= 4) is stage 2 alone.
    def stage(st, k):
        def f():
            rc = lib.wqbmm_a16w4_msd_profile_stage(st["x"].data_ptr(), st["w"].data_ptr(),
                                                   st["s"].data_ptr(), gs, M, K, N,
                                                   st["y"].data_ptr(), path, k, sptr)
            if rc:
                raise W.WqbmmError(rc, "wqbmm_a16w4_msd_profile_stage")
        return f

    G = K // gs
    two_kernels = path == 2 or M > 4
    prep_ms = None
    if two_kernels:
        _, prep_ms = timed_graph(torch, stream, [stage(st, 1) for st in sets], args.steps, args.warmup)
    _, kern_ms = timed_graph(torch, stream, [stage(st, 2) for st in sets], args.steps, args.warmup)
    if path == 1:
        if M > 4:
            # contraction kernel: tiled int4 weights, scales, the 16-row level
            # operands (three int4 levels) and level weights once, y
            kb = -(-K // 128)
            kbytes = alg["w_bytes"] + 2 * G * N + 3 * 1024 * kb + 192 * G + 2 * M * N
            kname = "msd_decode_gemv_kernel"
            extra["prep"] = {"kernel": "msd_decode_operands_kernel", "avg_kernel_us": round(prep_ms * 1e3, 3),
                             "algorithmic_bytes_per_launch": 2 * M * K + 3 * 1024 * kb + 192 * G}
        else:
            kbytes = alg["bytes"]
            kname = "msd_decode_kernel"
        achieved = kbytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kname, "avg_kernel_us": round(kern_ms * 1e3, 3),
                "algorithmic_bytes_per_launch": kbytes}
    else:
        # The GEMM contracts on FP6 (e2m3) MFMAs, so its roofline peak is the
        # dense FP6 rate; the fraction of the int8 rate is reported beside it.
        achieved = alg["exec_i8_ops"] / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP6_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP6_PEAK_TOPS, 4), "traffic": traffic,
                "kernel": "msd_gemm_kernel", "mfma_dtype": "fp6 e2m3",
                "avg_kernel_us": round(kern_ms * 1e3, 3),
                "algorithmic_ops_per_launch": alg["exec_i8_ops"],
                "frac_of_i8_peak": round(achieved / I8_PEAK_TOPS, 4)}
        # The GEMM spends more SIMD time on the fp32 combine of step 10 than on
        # the MFMA (and the two do not overlap): 4 fp32 operations per (row,
        # column, group) -- three for the level weights, one for the scale and
        # the running sum.
        combine_ops = 4 * M * N * G
        alu = combine_ops / (kern_ms * 1e-3) / 1e12
        extra["alu_view"] = {"bound": "alu", "ops_per_launch": combine_ops, "achieved": round(alu, 2),
                             "peak": round(VALU_F32_OPS_PEAK_T, 2), "unit": "T fp32 op/s",
                             "frac": round(alu / VALU_F32_OPS_PEAK_T, 4)}
        prep_bytes = prefill_prep_bytes(M, K, N, gs)
        extra["prep"] = {"kernel": "msd_prep_kernel", "avg_kernel_us": round(prep_ms * 1e3, 3),
                         "achieved_GBps": round(prep_bytes / (prep_ms * 1e-3) / 1e9, 1)}
    if tinfo is not None and not isinstance(tinfo, str):
        extra["traffic_detail"] = {k: tinfo[k] for k in tinfo if k != "kernel_sources_sha"}
    elif isinstance(tinfo, str):
        extra["traffic_detail"] = tinfo

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if path == 1 else "fp6",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: M={M} K={K} N={N} group_size={gs}",
                   "M": M, "K": K, "N": N, "group_size": gs,
                   "path": {1: "decode", 2: "prefill"}[path],
                   "buffer_sets": nsets, "footprint_MiB": round(nsets * set_bytes / 2 ** 20, 1),
                   "submission": "captured HIP graph of the K steps"},
        "weight_GBps": round(alg["w_bytes"] / t_s / 1e9, 1),
        "weight_GBps_frac_of_hbm": round(alg["w_bytes"] / t_s / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_algorithmic_GBps": round(alg["bytes"] / t_s / 1e9, 1),
        "exec_i8_TOPS": round(alg["exec_i8_ops"] / t_s / 1e12, 2),
        "event_ms_per_step": round(ev_step, 6),
        "roofline": roof,
        "kernel_sources_sha": sha,
    }
    out.update(extra)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, M, K, N, gs, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
