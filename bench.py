"""Benchmark: fused GMM E-step + sufficient statistics on one MI355X.

A step is one EM iteration through the C-ABI (gmm_em_iterate with iters=1):
parameter precompute, the fused E-step with statistics, the deterministic
partial reduction and the M-step, on the "ref" blob workload
(N=1,048,576 points, d=128, K=256 diagonal components, fp32) with X resident
in HBM. Every step (warm-up and timed) starts from the same initial
parameters (K data points as means, unit variances, equal weights), restored
by three small device copies inside the step, so that all steps do identical
work. `value` = N*K / (wall-clock seconds per step).

Prints one JSON line with, besides the required keys,
  roofline     - the fused E-step kernel's flops per launch / its average
                 duration (HIP events recorded around the kernel on its own
                 stream), against the FP32 MFMA peak, plus its algorithmic
                 HBM rate; `traffic` comes from committed rocprofv3 counter
                 readings when they were taken on the current kernel source
  cpu_baseline - the float64 oracle's E-step on a bounded row sample of the
                 same workload, on this host, single-threaded
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "E-step+stats points×components/s (N=1M,d=128,K=256); % of MFMA/HBM peak"
UNIT = "points×components/s"
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_FP64_MFMA_TFLOPS = 78.6
PEAK_HBM_GBPS = 8000.0
VAR_FLOOR = 1e-6
KERNEL_SRC = os.path.join(ROOT, "soft_clustering_gmm_amd", "csrc", "gmm_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ref_estep_stats.json")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, if still current."""
    if workload != "ref" or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(X, mu, var, logw, rows: int):
    """The oracle's E-step (as it stands) on the first `rows` rows, one thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    x = np.ascontiguousarray(X[:rows])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.estep(x, mu, var, logw)
        dt = time.perf_counter() - t0
    K = mu.shape[0]
    return {"value": rows * K / dt, "unit": UNIT, "cores": 1, "kind": "oracle",
            "sample": f"float64 oracle E-step + statistics (difference form, materialised R) on the first "
                      f"{rows} of {X.shape[0]} rows, same parameters; {dt:.2f} s on 1 host thread"}


def host_streamed(args, w, X, mu, var, logw, torch, gmm, dev):
    """One step = the row-chunked E-step over X in pinned host memory (copies of
    chunk i+1 overlap the scoring of chunk i) plus the M-step, from the initial
    parameters. Prints one JSON line with the PCIe-inclusive rate."""
    N, d, K = X.shape[0], X.shape[1], mu.shape[0]
    Xh = torch.from_numpy(X).pin_memory()
    mu0, var0, lw0 = (torch.from_numpy(a.copy()).to(dev) for a in (mu, var, logw))
    mud, vard, lwd = mu0.clone(), var0.clone(), lw0.clone()
    xt = gmm.GMM_F16 if X.dtype == np.float16 else gmm.GMM_F32
    ws = gmm.workspace_chunked(N, d, K, args.chunk_rows, xt, dev)

    def step():
        mud.copy_(mu0)
        vard.copy_(var0)
        lwd.copy_(lw0)
        Nk, Sx, Sxx, _, _ = gmm.estep_stats_chunked(Xh, mud, vard, lwd, args.chunk_rows, ws=ws)
        gmm.mstep(Nk, Sx, Sxx, N, VAR_FLOOR, mud, vard, lwd)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    xbytes = X.nbytes
    out = {
        "metric": METRIC + " [X streamed from pinned host memory]", "value": N * K / (ms * 1e-3), "unit": UNIT,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: N={N} d={d} K={K} {w.x_dtype}; X in pinned host memory, "
                               f"{args.chunk_rows} rows per chunk; step = chunked E-step + M-step",
                   "N": N, "d": d, "K": K, "x_dtype": w.x_dtype, "chunk_rows": args.chunk_rows},
        "host_to_device_GBps": round(xbytes / (ms * 1e-3) / 1e9, 2),
    }
    print(json.dumps(out), flush=True)
    return 0


def border_lists_bench(args, w, torch, gmm, dev):
    """One step = the inverted-list build (gmm_border_lists) over a synthetic
    top-2 assignment of the workload's N points and K lists, inputs in HBM.
    HBM roofline on the algorithmic bytes: read idx and resp (16 B per point),
    write one int32 per list entry and the K + 1 offsets."""
    from soft_clustering_gmm_amd import datagen
    N, K = w.N, w.K
    idx, resp = datagen.random_top2(11, N, K)
    idx_d, resp_d = torch.from_numpy(idx).to(dev), torch.from_numpy(resp).to(dev)
    members = torch.empty(2 * N, dtype=torch.int32, device=dev)
    ws = torch.empty(int(gmm.lib().gmm_border_lists_workspace_bytes(N, K)), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        off, _ = gmm.border_lists(idx_d, resp_d, K, args.border_threshold, ws=ws, members=members)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        off, _ = gmm.border_lists(idx_d, resp_d, K, args.border_threshold, ws=ws, members=members)
        b.record()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    entries = int(off[-1].item())
    alg = N * 16 + entries * 4 + (K + 1) * 8
    gbps = alg / (k_ms * 1e-3) / 1e9
    out = {
        "metric": "border-vector inverted-list build, points/s", "value": N / (ms * 1e-3), "unit": "points/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"{w.name} shape: N={N} K={K}, synthetic top-2 (seed 11), threshold "
                               f"{args.border_threshold}, {entries} list entries", "N": N, "K": K},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": alg, "avg_launch_ms": round(k_ms, 4)},
    }
    print(json.dumps(out), flush=True)
    return 0


def top2_bench(args, w, X, mu, var, logw, torch, gmm, dev):
    """One step = gmm_assign_top2 (each point's two most responsible components
    and their responsibilities, from the fp64 score pass) on the workload's X
    and initial parameters, all resident in HBM. Roofline: the pass's 4NKd
    score flops on the FP64 MFMA peak, timed with events around the call."""
    N, d, K = X.shape[0], X.shape[1], mu.shape[0]
    Xd = torch.from_numpy(X).to(dev)
    mud, vard, lwd = (torch.from_numpy(a.copy()).to(dev) for a in (mu, var, logw))
    ws = gmm.workspace(N, d, K, dev)
    for _ in range(args.warmup):
        gmm.assign_top2(Xd, mud, vard, lwd, ws=ws)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        gmm.assign_top2(Xd, mud, vard, lwd, ws=ws)
        b.record()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    flops = 4.0 * N * K * d
    ach = flops / (k_ms * 1e-3) / 1e12
    out = {
        "metric": "top-2 assignment, points x components/s", "value": N * K / (ms * 1e-3),
        "unit": "points×components/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"{w.name} recipe: N={N} d={d} K={K} {w.x_dtype}; initial parameters; "
                               f"step = gmm_assign_top2", "N": N, "d": d, "K": K},
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_FP64_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_FP64_MFMA_TFLOPS, 4), "traffic": None,
                     "kernel": "estep_lse_kernel (top-2)", "flops_per_launch": flops,
                     "avg_call_ms": round(k_ms, 4)},
    }
    print(json.dumps(out), flush=True)
    return 0


def kmeans_bench(args, w, torch, gmm, dev):
    """One step = one Lloyd iteration (nearest-centre assignment: fp32 scores on
    the matrix cores, exact fp64 distances for the candidates; then the
    list-based centre update) from the workload's initial means, X in HBM.
    Roofline: the assignment's 4NKd score flops on the FP32 MFMA peak, timed
    with events around the assignment call."""
    from soft_clustering_gmm_amd import datagen
    X, mu, _, _ = datagen.make_workload(args.workload)
    N, d, K = X.shape[0], X.shape[1], mu.shape[0]
    Xd = torch.from_numpy(X).to(dev)
    C0 = torch.from_numpy(mu.copy()).to(dev)
    C = C0.clone()
    ws = gmm.kmeans_workspace(N, d, K, dev)
    assign = torch.empty(N, dtype=torch.int32, device=dev)
    lib = gmm.lib()
    stream = gmm._stream(dev)

    def step(ev=None):
        C.copy_(C0)
        if ev:
            ev[0].record()
        gmm._check("gmm_kmeans_assign", lib.gmm_kmeans_assign(
            gmm._ptr(Xd), gmm._xtype(Xd), N, d, gmm._ptr(C), K, gmm._ptr(assign), None, None, gmm._ptr(ws),
            ws.numel(), stream))
        if ev:
            ev[1].record()
        gmm.kmeans_update(Xd, assign, C, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    a_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    flops = 4.0 * N * K * d
    ach = flops / (a_ms * 1e-3) / 1e12
    out = {
        "metric": "k-means Lloyd iteration, points x centres/s", "value": N * K / (ms * 1e-3),
        "unit": "points×centres/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32+f64", "data": "synthetic",
        "config": {"workload": f"{w.name} recipe: N={N} d={d} K={K} {w.x_dtype}; centres = the K initial means; "
                               f"step = assignment + update", "N": N, "d": d, "K": K},
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": None,
                     "kernel": "kmeans_assign_kernel", "flops_per_launch": flops,
                     "avg_assign_ms": round(a_ms, 4)},
    }
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ref", choices=["tiny", "ref", "smallk", "largek", "ivf"])
    ap.add_argument("--cpu-rows", type=int, default=131072, help="row sample for the oracle baseline (0: skip)")
    ap.add_argument("--x-on-host", action="store_true",
                    help="keep X in pinned host memory and stream it through the row-chunked E-step "
                         "(PCIe-inclusive rate; not the HBM-resident headline)")
    ap.add_argument("--chunk-rows", type=int, default=1 << 18, help="rows per chunk with --x-on-host")
    ap.add_argument("--border-lists", action="store_true",
                    help="time the border-vector inverted-list build on the workload's N and K from a "
                         "synthetic top-2 assignment resident in HBM")
    ap.add_argument("--border-threshold", type=float, default=0.05)
    ap.add_argument("--top2", action="store_true",
                    help="time gmm_assign_top2 on the workload's X and initial parameters")
    ap.add_argument("--kmeans", action="store_true",
                    help="time Lloyd iterations of k-means on the workload's X with its K initial means as centres")
    ap.add_argument("--stats-precision", default="fp32", choices=["fp32", "split-bf16"],
                    help="statistics contraction (split-bf16: split products on the bf16 matrix cores)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this E-step build runs on a "
              f"single MI355X; see the design notes for how it would shard over N.", file=sys.stderr)
        return 2

    import torch
    from soft_clustering_gmm_amd import datagen, gmm
    gmm.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    gmm.set_stats_precision(gmm.STATS_SPLIT_BF16 if args.stats_precision == "split-bf16" else gmm.STATS_FP32)

    w = datagen.WORKLOADS[args.workload]
    if args.border_lists:
        return border_lists_bench(args, w, torch, gmm, dev)
    if args.kmeans:
        return kmeans_bench(args, w, torch, gmm, dev)
    X, mu, var, logw = datagen.make_workload(args.workload)
    if args.x_on_host:
        return host_streamed(args, w, X, mu, var, logw, torch, gmm, dev)
    if args.top2:
        return top2_bench(args, w, X, mu, var, logw, torch, gmm, dev)
    N, d, K = X.shape[0], X.shape[1], mu.shape[0]
    Xd = torch.from_numpy(X).to(dev)
    mu0, var0, lw0 = (torch.from_numpy(a.copy()).to(dev) for a in (mu, var, logw))
    mud, vard, lwd = mu0.clone(), var0.clone(), lw0.clone()
    ws = gmm.workspace(N, d, K, dev)
    torch.cuda.synchronize()

    def step():
        mud.copy_(mu0)
        vard.copy_(var0)
        lwd.copy_(lw0)
        gmm.em_iterate(Xd, mud, vard, lwd, 1, VAR_FLOOR, ws=ws)

    for _ in range(args.warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:  # materialise the events
        a.record()
        b.record()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        gmm.set_timing_events(*evs[i])
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_step = 1e3 * wall / args.steps
    k_ms = [a.elapsed_time(b) for a, b in evs]
    k_avg = float(np.mean(k_ms))
    flops = 8.0 * N * K * d
    xbytes = N * d * X.itemsize + K * (2 * d + 1) * 4
    achieved = flops / (k_avg * 1e-3) / 1e12
    small = K <= 16 and d <= 64
    single = K <= 256
    regime = "small-K" if small else "single-sweep" if single else "two-pass"
    ctype = {"f32": "float", "f16": "_Float16"}[w.x_dtype]
    sp = str(args.stats_precision == "split-bf16").lower()
    kernel = (f"estep_small_kernel<{-(-d // 16)},{ctype},{sp}> (small K)" if small
              else f"estep_stats_kernel<{-(-d // 32)},0,{ctype},{sp}> (single sweep)" if single
              else f"estep_lse_kernel + estep_stats_kernel<{-(-d // 32)},1,{ctype},{sp}> (two-pass)")
    roof = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": committed_traffic(args.workload),
        "kernel": kernel,
        "flops_per_launch": flops, "avg_launch_ms": round(k_avg, 4),
        "p90_launch_ms": round(float(np.percentile(k_ms, 90)), 4),
        "hbm_algorithmic_bytes_per_launch": xbytes,
        "hbm_achieved_GBps": round(xbytes / (k_avg * 1e-3) / 1e9, 1),
        "hbm_frac": round(xbytes / (k_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "credit": ("dense 8NKd flops; the fp32 statistics loop skips points whose responsibilities for a "
                   "wave's 32 components are all exactly zero (exact, data-dependent), so executed "
                   "matrix-core work can be below the credited flops" if not small and sp == "false"
                   else "dense 8NKd flops, all executed"),
    }
    out = {
        "metric": METRIC, "value": N * K / (ms_step * 1e-3), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32+bf16x3" if args.stats_precision == "split-bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: N={N} d={d} K={K} {w.x_dtype} Gaussian blobs (seed {w.seed}); "
                               f"step = one EM iteration from the initial parameters (precompute, fused E-step+stats, "
                               f"reduction, M-step)",
                   "N": N, "d": d, "K": K, "x_dtype": w.x_dtype, "regime": regime,
                   "stats_precision": args.stats_precision},
        "roofline": roof,
    }
    if args.cpu_rows > 0:
        out["cpu_baseline"] = cpu_baseline(X, mu, var, logw, min(args.cpu_rows, N))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
