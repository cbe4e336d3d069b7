"""Benchmark: fused GMM E-step + sufficient statistics on one MI355X.

A step is one EM iteration through the C-ABI (gmm_em_iterate with iters=1):
parameter precompute, the fused E-step with statistics, the deterministic
partial reduction and the M-step, on the "ref" blob workload
(N=1,048,576 points, d=128, K=256 diagonal components, fp32) with X resident
in HBM. Every step (warm-up and timed) starts from the same initial
parameters (K data points as means, unit variances, equal weights), restored
by one device copy of the flat parameter buffer inside the step, so that all
steps do identical work. `value` = N*K / (wall-clock seconds per step).
Unless --warmup is given, the untimed warm-up runs at least 3 steps and
200 ms, past the GPU's clock ramp (the first ~30 ms of back-to-back E-steps
run up to ~12% slower); the line reports how many warm-up steps ran.

Prints one JSON line with, besides the required keys,
  roofline     - the fused E-step kernel's flops per launch / its average
                 duration (HIP events recorded around the kernel on its own
                 stream), against the FP32 MFMA peak, plus its algorithmic
                 HBM rate; `traffic` comes from committed rocprofv3 counter
                 readings when they were taken on the current kernel source
  cpu_baseline - the float64 oracle's E-step (expanded form: two BLAS
                 products per row chunk) on the same workload, on every
                 host core this process may use, at full N where that takes
                 under ~20 s, else on a leading row sample
  measured peaks - the FP32 matrix-core issue rate and the HBM read rate
                 this GPU sustains (the library's peak probes), so that the
                 roofline fraction is also quoted against measured peaks
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
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
# Rough fp64 work the oracle's expanded form does per second on one modern
# host core (two GEMMs of 2d per point x component, plus the exponentials):
# only used to choose the row sample so that the baseline takes ~20 s.
CPU_BUDGET_POINT_COMP_D = 2.5e10


WARMUP_MIN_STEPS = 3
WARMUP_MIN_MS = 200.0


def warm_up(step, args, torch) -> int:
    """Untimed steps before the timed ones; returns how many ran. With --warmup W exactly W.
    By default at least WARMUP_MIN_STEPS steps and WARMUP_MIN_MS of wall time, each step
    synchronised: on a GPU that has just become busy the first ~30 ms of back-to-back E-steps
    run up to ~12% slower while its clock ramps up (rocprofv3 traces of 300 launches), and the
    timed steps should measure the steady state."""
    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        return args.warmup
    n = 0
    t0 = time.perf_counter()
    while n < WARMUP_MIN_STEPS or 1e3 * (time.perf_counter() - t0) < WARMUP_MIN_MS:
        step()
        torch.cuda.synchronize()
        n += 1
    return n


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_counters(workload: str, stats_precision: str):
    """rocprofv3 counter readings committed for this workload's fused E-step (HBM
    bytes and executed MFMA flops per launch), if taken on the current kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return {}
    with open(COUNTERS_FILE) as f:
        table = json.load(f)
    t = table.get(f"{workload}/{stats_precision}", {})
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return {}
    return t


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(X, mu, var, logw, max_rows: int | None = None):
    """The oracle's E-step (as it stands, expanded form) on every core this process may use:
    full N when it fits the time budget, else the leading rows, scaled to the metric's unit."""
    import oracle
    from threadpoolctl import threadpool_limits
    N, d = X.shape
    K = mu.shape[0]
    cores = len(os.sched_getaffinity(0))
    rows = int(min(N, max(4096, CPU_BUDGET_POINT_COMP_D * cores / (K * d))))
    if max_rows:
        rows = min(rows, max_rows)
    x = np.ascontiguousarray(X[:rows])
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        oracle.estep(x, mu, var, logw, form="expanded", row_chunk=8192)
        dt = time.perf_counter() - t0
    what = "all" if rows == N else f"the first {rows} of"
    return {"value": rows * K / dt, "unit": UNIT, "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"float64 oracle E-step + statistics, expanded form (scores from two BLAS products, "
                      f"materialised R per 8192-row chunk), on {what} {N} rows, same parameters; {dt:.2f} s "
                      f"with BLAS on {cores} threads ({cpu_model()})"}


def measured_peaks(torch, gmm, dev, reps: int = 5):
    """FP32 matrix-core issue rate and HBM read rate of this GPU from the library's
    peak probes (best of `reps` launches each, timed with events on the probes' stream)."""
    out = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    res = {}
    for name, launch in (
            ("mfma_f32_tflops", lambda: gmm.peak_mfma(gmm.PEAK_FP32, 20000, 2048, out)),
            ("mfma_f64_tflops", lambda: gmm.peak_mfma(gmm.PEAK_FP64, 10000, 2048, out)),
            ("hbm_read_gbps", lambda: gmm.peak_hbm_read(buf, 2048, out))):
        launch()  # warm-up
        best = 0.0
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            work = launch()
            b.record()
            b.synchronize()
            rate = work / (a.elapsed_time(b) * 1e-3)
            best = max(best, rate)
        res[name] = round(best / (1e12 if "tflops" in name else 1e9), 1)
    del buf
    # fp32 matrix and vector work alone, together in each wave, and in separate waves of one SIMD
    co = torch.empty(1024 * 512, dtype=torch.float32, device=dev)
    t = []
    for mode in range(4):
        gmm.peak_coissue(mode, 2000, 1024, co)  # warm-up
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gmm.peak_coissue(mode, 20000, 1024, co)
            b.record()
            b.synchronize()
            best = min(best, a.elapsed_time(b))
        t.append(best)
    res["coissue_ms"] = {"mfma_only": round(t[0], 3), "valu_only": round(t[1], 3), "both_per_wave": round(t[2], 3),
                         "split_waves": round(t[3], 3),
                         "both_per_wave_over_sum": round(t[2] / (t[0] + t[1]), 3),
                         "split_waves_over_half_sum": round(t[3] / ((t[0] + t[1]) / 2), 3)}
    res["probes"] = ("gmm_peak_mfma: 2048 blocks x 4 waves, 8 independent MFMAs per trip (32x32x2 fp32 / "
                     "16x16x4 fp64); gmm_peak_hbm_read: 4 GiB read once, 16-byte loads, 2048 blocks x 256")
    return res


def param_buffers(torch, mu, var, logw, dev):
    """The initial parameters P0 and the working parameters P on the device,
    each one flat buffer [mu | var | logw], and mu, var, logw as views of P:
    a step resets all three with one device copy."""
    K, d = mu.shape
    flat = np.concatenate([mu.ravel(), var.ravel(), logw.ravel()]).astype(np.float32)
    P0 = torch.from_numpy(flat).to(dev)
    P = P0.clone()
    return P0, P, P[:K * d].view(K, d), P[K * d:2 * K * d].view(K, d), P[2 * K * d:]


def host_streamed(args, w, X, mu, var, logw, torch, gmm, dev):
    """One step = the row-chunked E-step over X in pinned host memory (copies of
    chunk i+1 overlap the scoring of chunk i) plus the M-step, from the initial
    parameters. Prints one JSON line with the PCIe-inclusive rate."""
    N, d, K = X.shape[0], X.shape[1], mu.shape[0]
    Xh = torch.from_numpy(X).pin_memory()
    P0, P, mud, vard, lwd = param_buffers(torch, mu, var, logw, dev)
    xt = gmm.GMM_F16 if X.dtype == np.float16 else gmm.GMM_F32
    ws = gmm.workspace_chunked(N, d, K, args.chunk_rows, xt, dev)

    def step():
        P.copy_(P0)
        Nk, Sx, Sxx, _, _ = gmm.estep_stats_chunked(Xh, mud, vard, lwd, args.chunk_rows, ws=ws)
        gmm.mstep(Nk, Sx, Sxx, N, VAR_FLOOR, mud, vard, lwd)

    warmup = warm_up(step, args, torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    xbytes = X.nbytes
    out = {
        "metric": METRIC + " [X streamed from pinned host memory]", "value": N * K / (ms * 1e-3), "unit": UNIT,
        "n_gpus": 1, "steps": args.steps, "warmup": warmup, "ms_per_step": round(ms, 4),
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
    warmup = warm_up(lambda: gmm.border_lists(idx_d, resp_d, K, args.border_threshold, ws=ws, members=members),
                     args, torch)
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
        "n_gpus": 1, "steps": args.steps, "warmup": warmup, "ms_per_step": round(ms, 4),
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
    warmup = warm_up(lambda: gmm.assign_top2(Xd, mud, vard, lwd, ws=ws), args, torch)
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
        "unit": "points×components/s", "n_gpus": 1, "steps": args.steps, "warmup": warmup,
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

    warmup = warm_up(step, args, torch)
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
        "unit": "points×centres/s", "n_gpus": 1, "steps": args.steps, "warmup": warmup,
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
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3 and at least 200 ms of them)")
    ap.add_argument("--workload", default="ref", choices=["tiny", "ref", "smallk", "largek", "ivf"])
    ap.add_argument("--rows", type=int, default=None,
                    help="draw the workload's recipe at this many rows instead of its own N (E-step, top-2 "
                         "and host-streamed benches); the committed counter figures are then not reported")
    ap.add_argument("--cpu-rows", type=int, default=-1,
                    help="row cap for the oracle baseline (-1: as many as fit ~20 s, full N where possible; 0: skip)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak probes")
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
    ap.add_argument("--stats-precision", default="auto", choices=["auto", "fp32", "split-bf16"],
                    help="statistics contraction: auto (the library's default: fp32 products, exact fp16 "
                         "splits in the second pass over half-precision X), fp32, or split-bf16 products")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this E-step build runs on a "
              f"single MI355X; see the design notes for how it would shard over N.", file=sys.stderr)
        return 2

    import torch
    from soft_clustering_gmm_amd import datagen, gmm
    gmm.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    gmm.set_stats_precision({"auto": gmm.STATS_AUTO, "fp32": gmm.STATS_FP32,
                             "split-bf16": gmm.STATS_SPLIT_BF16}[args.stats_precision])

    w = datagen.WORKLOADS[args.workload]
    if args.border_lists:
        return border_lists_bench(args, w, torch, gmm, dev)
    if args.kmeans:
        return kmeans_bench(args, w, torch, gmm, dev)
    if args.rows is not None and args.rows < max(w.K, 1):
        print(f"--rows must be at least K = {w.K} for the {w.name} recipe", file=sys.stderr)
        return 2
    X, mu, var, logw = datagen.make_workload(args.workload, N=args.rows)
    if args.x_on_host:
        return host_streamed(args, w, X, mu, var, logw, torch, gmm, dev)
    if args.top2:
        return top2_bench(args, w, X, mu, var, logw, torch, gmm, dev)
    N, d, K = X.shape[0], X.shape[1], mu.shape[0]
    Xd = torch.from_numpy(X).to(dev)
    P0, P, mud, vard, lwd = param_buffers(torch, mu, var, logw, dev)
    ws = gmm.workspace(N, d, K, dev)
    torch.cuda.synchronize()

    def step():
        P.copy_(P0)
        gmm.em_iterate(Xd, mud, vard, lwd, 1, VAR_FLOOR, ws=ws)

    warmup = warm_up(step, args, torch)
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
    # the second pass over half-precision X in the default mode: exact fp16 splits (rows with |x| < 15)
    f16split = args.stats_precision == "auto" and regime == "two-pass" and w.x_dtype == "f16"
    s2 = "2" if f16split else ("1" if sp == "true" else "0")
    kernel = (f"estep_small_kernel<{-(-d // 16)},{ctype},{sp}> (small K)" if small
              else f"estep_stats_kernel<{-(-d // 32)},0,{ctype},{int(sp == 'true')}> (single sweep)" if single
              else f"estep_stats_kernel<{-(-d // 32)},2,{ctype},0> + lse_merge_kernel + estep_lse_kernel "
                   f"(fallback rows) + estep_stats_kernel<{-(-d // 32)},1,{ctype},{s2}> (two-pass)")
    # the committed counters were taken at the recipe's own N
    ctr = committed_counters(args.workload, args.stats_precision) if N == w.N else {}
    executed = ctr.get("executed_flops_per_launch")
    roof = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": ctr.get("hbm_bytes_per_launch"),
        "executed_frac": (round(executed / (k_avg * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4)
                          if executed else None),
        "executed_flops_per_launch": executed,
        "kernel": kernel,
        "flops_per_launch": flops, "avg_launch_ms": round(k_avg, 4),
        "p90_launch_ms": round(float(np.percentile(k_ms, 90)), 4),
        "hbm_algorithmic_bytes_per_launch": xbytes,
        "hbm_achieved_GBps": round(xbytes / (k_avg * 1e-3) / 1e9, 1),
        "hbm_frac": round(xbytes / (k_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "credit": "dense 8NKd flops (4NKd scores + 4NKd statistics)"
                  + ("; the fp32 statistics loop leaves out points whose responsibilities for a wave's 32 "
                     "components are all at most 2^-20/N/max(1,|x|^2) (at most ~1e-6 of any statistic, "
                     "data-dependent)" if not small and sp == "false" else ", all statistics executed")
                  + ("; the first pass scores every pair once more (4NKd, not credited)" if regime == "two-pass"
                     else "")
                  + "; executed_flops_per_launch counts what the matrix cores ran",
    }
    out = {
        "metric": METRIC, "value": N * K / (ms_step * 1e-3), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("f32+bf16x3" if args.stats_precision == "split-bf16" else
                  "f32+f16x2" if f16split else "f32"),
        "data": "synthetic",
        "config": {"workload": f"{w.name}: N={N} d={d} K={K} {w.x_dtype} Gaussian blobs (seed {w.seed}); "
                               f"step = one EM iteration from the initial parameters (precompute, fused E-step+stats, "
                               f"reduction, M-step)",
                   "N": N, "d": d, "K": K, "x_dtype": w.x_dtype, "regime": regime,
                   "stats_precision": args.stats_precision},
        "roofline": roof,
    }
    if not args.no_peaks:
        pk = measured_peaks(torch, gmm, dev)
        roof["measured_peak"] = pk
        roof["frac_of_measured_peak"] = round(achieved / pk["mfma_f32_tflops"], 4)
        roof["hbm_frac_of_measured_peak"] = round(xbytes / (k_avg * 1e-3) / 1e9 / pk["hbm_read_gbps"], 4)
    if args.cpu_rows != 0:
        out["cpu_baseline"] = cpu_baseline(X, mu, var, logw, args.cpu_rows if args.cpu_rows > 0 else None)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
