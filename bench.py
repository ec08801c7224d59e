"""Benchmark of the LoGRA sketch hot path on one MI355X.

One step = one update over the whole layer set of the workload:
  A. project every selected matrix's input, every microbatch, straight into
     the packed operand form the accumulate reads (XAt = X A^T; one
     persistent launch per microbatch over every matrix of every layer)
  B. accumulate every sketch, every microbatch (one persistent launch per
     microbatch over every matrix of every layer)
  C. RowAdam for every sketch in one grouped call (writing the update straight in the merge's
     packed operand form), predicted-KL q over the context set, alpha on
     the device
  D. merge every matrix, W <- round(W - eta*alpha U A) (grouped: the seven
     matrices of one layer per launch)
Inputs are synthetic and resident in HBM before timing starts (distinct
buffers for every layer and microbatch, so the 256 MB Infinity Cache cannot
serve them).  The metric is HBM GB/s of phases B + D: their algorithmic bytes
(accumulate 2Td + 4Tr + 8dr per matrix and microbatch, merge 4dk + 4dr per
matrix) divided by their HIP-event time on the stream the kernels run on.

The step is the call sequence of rank_gradient_sketching_logra_amd.update,
the same one the full-size parity tests run.  Phase times are medians over
the timed steps.  The read and copy ceilings of the part are measured in the
same process with the library's streaming probe, and every phase is reported
against them as well as against the published peaks.

Modes:
  (default)              the benchmark; prints one JSON line
  --counter-run          a short run for rocprofv3 --pmc: a copy of known size
                         (the calibration) and one step of the workload
  --summarize-traffic F W  read the FETCH_SIZE (F) and WRITE_SIZE (W) counter
                         CSVs of two --counter-run passes and print the
                         calibrated HBM bytes per launch of the accumulate and
                         of the merge
--gpus above 1 is refused: this measures one GPU.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published
PEAK_MFMA_BF16_TFS = 2500.0   # MI355X dense bf16 matrix peak, published
CALIB_BYTES = 1 << 30   # plain copy used to calibrate the byte counters
POOL_LIMIT_BYTES = 160e9  # distinct input sets up to this size, else a pool
POOL_SETS = 17            # input sets in a pool (27B set: 17 x 0.74 GB)
BALLAST_BYTES = {"dense-27b-set-r256": 10 * 10**9}
DEFAULT_WORKLOAD = "qwen2.5-7b-set-r64"
# Microbatches per projection and accumulate launch.  Several at r = 64 (four on the 7B set,
# two on the 1.5B set): their inputs are stored together, so each tile's fixed cost (ring fill,
# class-sum exchange, S read and write) is paid once per launch.  One at r = 256, where pairing
# saved 2.5%.
PER_LAUNCH = {"qwen2.5-7b-set-r64": 4, "qwen2.5-1.5b-set-r64": 2}
# Layers per grouped merge launch (at most 16 matrices a launch): two layers halve the
# launches and give each block twice the units over which to spread its start (sign
# generation, ring fill).
MERGE_PER_LAUNCH = {"qwen2.5-7b-set-r64": 2, "qwen2.5-1.5b-set-r64": 2, "dense-27b-set-r256": 2}
ACC_KERNEL = "acc_bf16_table_kernel"
MERGE_KERNEL = "merge_bf16_kernel"
CALIB_KERNEL = "probe_copy_kernel"
CSRC = "rank_gradient_sketching_logra_amd/csrc/"
# the committed counter summaries, and the sources each kernel is built from
TRAFFIC_FILES = {ACC_KERNEL: "profiles/acc_bf16_table_kernel.{w}.traffic.md",
                 MERGE_KERNEL: "profiles/merge_bf16_kernel.{w}.traffic.md"}
KERNEL_SOURCES = {ACC_KERNEL: [CSRC + "kernels_sketch.hip", CSRC + "device_common.h"],
                  MERGE_KERNEL: [CSRC + "kernels_merge.hip", CSRC + "device_common.h"]}
PROBE_BYTES = 4 << 30     # the read probe streams 4 GiB; the copy probe moves 2 GiB each way


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rounding", default=None, choices=[None, "nearest", "stochastic"])
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=None, help="use fewer layers (profiling runs only)")
    ap.add_argument("--microbatches-per-launch", type=int, default=None,
                    help="microbatches whose inputs are stored together and projected and "
                         "accumulated by one launch each (default: per workload)")
    ap.add_argument("--merge-layers-per-launch", type=int, default=None,
                    help="layers per grouped merge launch (default: per workload)")
    ap.add_argument("--counter-run", action="store_true")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-counters", metavar="COUNTER_CSV",
                    help="per-dispatch means of every counter in a rocprofv3 --pmc csv, for the "
                         "accumulate and merge kernels")
    return ap.parse_args()


def acc_bytes(T, d, r):
    return 2 * T * d + 4 * T * r + 8 * d * r


def merge_bytes(d, k, r):
    return 4 * d * k + 4 * d * r


def project_bytes(T, k, r):
    return 2 * T * k + 4 * T * r


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload, tokens_per_launch, layers_per_launch):
    """Calibrated HBM bytes per launch of `kernel` from the committed counter summary, or None
    when it is missing, was taken on other kernel sources or on launches of another size (the
    accumulate's tokens, the merge's layers)."""
    try:
        with open(os.path.join(ROOT, TRAFFIC_FILES[kernel].format(w=workload))) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    t = json.loads(line[len("traffic-json: "):])
                    same = (t.get("tokens_per_launch") == tokens_per_launch if kernel == ACC_KERNEL
                            else t.get("layers_per_launch", 1) == layers_per_launch)
                    if t.get("kernel_sources") == kernel_source_hash(kernel) and same:
                        return t
    except OSError:
        pass
    return None


def summarize_traffic(fetch_csv, write_csv, workload, tokens_per_launch, layers_per_launch):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the calibration copy, the accumulate and
    the merge; each counter is scaled by bytes-moved / counter-reading of the copy.  Returns
    one summary per kernel."""
    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = next((k for k in (ACC_KERNEL, MERGE_KERNEL, CALIB_KERNEL) if k in name), None)
            if key is None:
                continue
            vals.setdefault(key, {}).setdefault(row["Dispatch_Id"], 0.0)
            vals[key][row["Dispatch_Id"]] += float(row["Counter_Value"])
        return {k: sorted(v.values()) for k, v in vals.items()}
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    fcopy, wcopy = max(f[CALIB_KERNEL]), max(w[CALIB_KERNEL])
    ffac = CALIB_BYTES / (fcopy * 1024.0)
    wfac = CALIB_BYTES / (wcopy * 1024.0)
    out = []
    for kernel in (ACC_KERNEL, MERGE_KERNEL):
        if kernel not in f or kernel not in w:
            continue
        fk = sum(f[kernel]) / len(f[kernel]) * 1024.0 * ffac
        wk = sum(w[kernel]) / len(w[kernel]) * 1024.0 * wfac
        out.append({"kernel": kernel, "workload": workload,
                    "fetch_bytes_per_launch": round(fk), "write_bytes_per_launch": round(wk),
                    "traffic_bytes_per_launch": round(fk + wk),
                    "fetch_calibration": round(ffac, 4), "write_calibration": round(wfac, 4),
                    "copy_fetch_kib": fcopy, "copy_write_kib": wcopy,
                    "dispatches": len(f[kernel]), "kernel_sources": kernel_source_hash(kernel),
                    **({"tokens_per_launch": tokens_per_launch} if kernel == ACC_KERNEL
                       else {"layers_per_launch": layers_per_launch})})
    return out


def summarize_counters(path):
    """Mean per dispatch of every counter in one rocprofv3 counter csv, with the mean dispatch
    duration, for the accumulate and the merge kernels (the counters summed over the dimensions
    rocprofv3 reports them in)."""
    per = {}
    for row in csv.DictReader(open(path)):
        key = next((k for k in (ACC_KERNEL, MERGE_KERNEL) if k in row["Kernel_Name"]), None)
        if key is None:
            continue
        d = per.setdefault(key, {}).setdefault(row["Dispatch_Id"], {"counters": {}})
        d["ns"] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
        c = d["counters"]
        c[row["Counter_Name"]] = c.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    out = []
    for kernel, disp in per.items():
        n = len(disp)
        names = sorted({c for d in disp.values() for c in d["counters"]})
        out.append({"kernel": kernel, "dispatches": n,
                    "mean_us": round(sum(d["ns"] for d in disp.values()) / n / 1e3, 2),
                    "mean": {c: sum(d["counters"].get(c, 0.0) for d in disp.values()) / n for c in names},
                    "kernel_sources": kernel_source_hash(kernel)})
    return out


def cpu_baseline(w, rounding):
    """The oracle, untuned, on a bounded sample: layer 0's seven accumulates for one
    microbatch and its seven merges.  Returns the sample's algorithmic GB/s."""
    import numpy as np
    import oracle
    from oracle import philox
    from rank_gradient_sketching_logra_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    mats = w.matrices(layers=[0])
    inputs = []
    for (layer, kind, mid, d, k) in mats:
        inputs.append((mid, d, k, synth.output_grad(w, layer, kind, 0),
                       synth.fp32_matrix((w.T, w.r), 7.5, (w.index, mid, 0, 0, 0)),
                       synth.weight(w, layer, kind),
                       synth.fp32_matrix((d, w.r), 1.0, (w.index, mid, 0, 0, 7))))
    nbytes = 0
    t0 = time.perf_counter()
    for (mid, d, k, db, XAt, wb, U) in inputs:
        S = oracle.accumulate(np.zeros((d, w.r)), oracle.bf16_bits_to_f64(db), XAt.astype(np.float64))
        A = oracle.regen_A(w.seed, mid, w.step, w.r, k)
        u = philox.sr_draws(w.sr_seed, mid, w.step, d, k) if rounding == "stochastic" else None
        oracle.merge(oracle.bf16_bits_to_f64(wb), U.astype(np.float64), A, w.eta, w_dtype="bf16",
                     mode=rounding, u_draws=u)
        nbytes += acc_bytes(w.T, d, w.r) + merge_bytes(d, k, w.r)
        del S
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layer 0 of {w.name}: 7 accumulates (1 microbatch, T={w.T}) + 7 merges ({rounding}),"
                      f" numpy fp64, {nbytes / 1e9:.2f} GB algorithmic in {dt:.1f} s"}


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def measure_ceilings(B, torch, dev):
    """Read and copy ceilings of the part, with the library's streaming probe: the best of a
    few launch shapes, each timed over three back-to-back launches."""
    src = torch.empty((PROBE_BYTES,), dtype=torch.uint8, device=dev)
    src.fill_(7)
    sink = torch.empty((4096,), dtype=torch.uint8, device=dev)
    half = PROBE_BYTES // 2
    dst = torch.empty((half,), dtype=torch.uint8, device=dev)
    best = {"read": (0.0, 0), "copy": (0.0, 0)}
    for mode in ("read", "copy"):
        for bpc in (1, 2, 4, 8):
            a = src if mode == "read" else src[:half]
            o = sink if mode == "read" else dst
            B.bandwidth_probe(mode, a, o, bpc)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                B.bandwidth_probe(mode, a, o, bpc)
            e1.record()
            torch.cuda.synchronize()
            moved = 3 * (PROBE_BYTES if mode == "read" else 2 * half)
            gbs = moved / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if gbs > best[mode][0]:
                best[mode] = (gbs, bpc)
    del src, dst, sink
    return {"read_gbs": round(best["read"][0], 1), "copy_gbs": round(best["copy"][0], 1),
            "read_blocks_per_cu": best["read"][1], "copy_blocks_per_cu": best["copy"][1],
            "bytes": PROBE_BYTES, "probe": "logra_bandwidth_probe (16-byte accesses, non-temporal loads, grid-strided)"}


def roofline(name, per_launch_bytes, per_launch_flops, launch_us):
    """Roofline entry of one kernel from its algorithmic bytes and flops per launch: the bound is
    whichever of HBM (8 TB/s) and dense bf16 matrix work (2.5 PFLOP/s) takes longer."""
    t_hbm = per_launch_bytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = per_launch_flops / (PEAK_MFMA_BF16_TFS * 1e12)
    sec = launch_us * 1e-6
    if t_hbm >= t_mfma:
        ach = per_launch_bytes / sec / 1e9
        return {"bound": "hbm", "kernel": name, "achieved": round(ach, 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    ach = per_launch_flops / sec / 1e12
    return {"bound": "mfma", "kernel": name, "achieved": round(ach, 2), "peak": PEAK_MFMA_BF16_TFS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_MFMA_BF16_TFS, 4)}


def main():
    args = parse()
    if args.summarize_traffic:
        from rank_gradient_sketching_logra_amd import synth
        w = synth.BY_NAME[args.workload]
        tpl = w.T * (args.microbatches_per_launch or PER_LAUNCH.get(w.name, 1))
        mpl = args.merge_layers_per_launch or MERGE_PER_LAUNCH.get(w.name, 1)
        for t in summarize_traffic(*args.summarize_traffic, args.workload, tpl, mpl):
            print("traffic-json: " + json.dumps(t))
        return
    if args.summarize_counters:
        for t in summarize_counters(args.summarize_counters):
            print("counters-json: " + json.dumps(t))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from rank_gradient_sketching_logra_amd import binding as B
    from rank_gradient_sketching_logra_amd import synth
    from rank_gradient_sketching_logra_amd import update as U

    w = synth.BY_NAME[args.workload]
    rounding = args.rounding or w.rounding
    layers = args.layers or w.layers
    if args.counter_run:
        args.steps, args.warmup = 1, 0
    T, r, M = w.T, w.r, w.microbatches
    # G microbatches per launch: their inputs are stored as one [G T x width] block per matrix,
    # so one launch of G T tokens projects or accumulates them all (S is read and written
    # once per G microbatches).  From here on T and M count tokens per launch and launches.
    G = args.microbatches_per_launch or PER_LAUNCH.get(w.name, 1)
    if G < 1 or M % G:
        print(f"--microbatches-per-launch must divide the {M} microbatches", file=sys.stderr)
        sys.exit(2)
    T_mb = T
    T, M = G * T, M // G
    ML = args.merge_layers_per_launch or MERGE_PER_LAUNCH.get(w.name, 1)
    if ML < 1 or ML * len(w.kinds) > 16:
        print("--merge-layers-per-launch: at most 16 matrices per launch", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()
    g = torch.Generator(device=dev)
    g.manual_seed(1234)

    def randn(shape, std, dtype=torch.bfloat16):
        t = torch.empty(shape, dtype=dtype, device=dev)
        t.normal_(0.0, std, generator=g)
        return t

    if args.counter_run:
        # the calibration: the library's copy probe over CALIB_BYTES
        src = torch.empty((CALIB_BYTES,), dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        B.bandwidth_probe("copy", src, dst, 4)
        torch.cuda.synchronize()
        del src, dst

    mats = w.matrices(layers=range(layers))
    kinds = tuple(w.kinds)
    xw = {"att": w.shapes["q"][1], "o": w.shapes["o"][1], "mlp": w.shapes["gate"][1], "down": w.shapes["down"][1]}
    pbytes = B.packed_input_bytes(T, r)
    # One input set (X and D of every matrix) per (layer, microbatch).  When the distinct
    # sets would not fit beside the weights, the step rotates through a pool of sets,
    # consecutive launches on consecutive sets, the pool far larger than the 256 MB Infinity
    # Cache.  The packed projected inputs are outputs of the projection phase and inputs of
    # the accumulate phase, so every (layer, microbatch, matrix) has its own.
    set_bytes = T * 2 * (sum(xw.values()) + sum(d for (_, d) in w.shapes.values()))
    nsets = layers * M if layers * M * set_bytes <= POOL_LIMIT_BYTES else POOL_SETS
    sid = {(l, mb): (mb * layers + l) % nsets for l in range(layers) for mb in range(M)}
    X = {(i, s): randn((T, xw[s]), 1.0) for i in range(nsets) for s in xw}
    D = {(i, kind): randn((T, d), 1e-3) for i in range(nsets) for kind, (d, k) in w.shapes.items()}
    PL = {(l, mb, kind): torch.empty((pbytes,), dtype=torch.uint8, device=dev)
          for l in range(layers) for mb in range(M) for kind in w.shapes}
    W = {(l, kind): randn((d, k), 0.02) for (l, kind, mid, d, k) in mats}
    S = {(l, kind): torch.zeros((d, r), dtype=torch.float32, device=dev) for (l, kind, mid, d, k) in mats}
    UP = {(l, kind): torch.empty((B.packed_update_bytes(d, r),), dtype=torch.uint8, device=dev)
          for (l, kind, mid, d, k) in mats}
    V = {(l, kind): torch.zeros((d,), dtype=torch.float32, device=dev) for (l, kind, mid, d, k) in mats}
    keys = {(l, kind): B.key(w.seed, mid, w.step) for (l, kind, mid, d, k) in mats}
    ra_ws = B.workspace(B.rowadam_grouped_ws_bytes(len(mats), sum(d for (_, _, _, d, _) in mats)), dev)
    acc_ws = B.workspace(B.sketch_accumulate_table_ws_bytes(len(mats)), dev)
    proj_ws = B.workspace(B.project_input_table_ws_bytes(len(mats)), dev)
    # the rest of the model's weights, resident but untouched (27B set: the projections are
    # 43.6 GB of the model's ~54 GB)
    ballast = torch.empty((BALLAST_BYTES.get(w.name, 0),), dtype=torch.uint8, device=dev)
    P, Vv = (w.P or 64), (w.V or 152064)
    z = randn((P, Vv), 4.0)
    zd = randn((P, Vv), 1.0)
    kl_ws = B.workspace(B.predicted_kl_q_ws_bytes(P, Vv), dev)
    q = torch.empty((1,), dtype=torch.float32, device=dev)
    alpha = torch.empty((1,), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    acc_total = sum(acc_bytes(T, d, r) for (_, _, _, d, _) in mats) * M
    merge_total = sum(merge_bytes(d, k, r) for (_, _, _, d, k) in mats)
    proj_total = sum(project_bytes(T, k, r) for (_, _, _, d, k) in mats) * M
    acc_flops = sum(2 * T * d * r for (_, _, _, d, _) in mats) * M
    merge_flops = sum(2 * d * k * r for (_, _, _, d, k) in mats)
    layer_list = list(range(layers))
    sketches = [(S[key_], V[key_], UP[key_]) for key_ in S]
    t_step = 0

    def step(ev):
        nonlocal t_step
        t_step += 1
        for s_ in S.values():
            s_.zero_()
        ev[0].record()
        for mb in range(M):                          # A: forward-side projections
            U.project(layer_list, kinds, lambda l, kd: keys[(l, kd)],
                      lambda l, kd, mb=mb: X[(sid[(l, mb)], U.SHARED_INPUT[kd])],
                      lambda l, kd, mb=mb: PL[(l, mb, kd)], r, proj_ws)
        ev[1].record()
        for mb in range(M):                          # B: backward-side sketch accumulation
            U.accumulate(layer_list, kinds, lambda l, kd, mb=mb: D[(sid[(l, mb)], kd)],
                         lambda l, kd, mb=mb: PL[(l, mb, kd)], lambda l, kd: S[(l, kd)], r, acc_ws)
        ev[2].record()
        U.optimise(sketches, r, t_step, w.beta, w.eps, ra_ws)     # C: optimiser, q, alpha
        U.step_size(z, zd, w.tau, w.delta, w.alpha_max, q, alpha, kl_ws)
        ev[3].record()
        U.merge(layer_list, kinds, lambda l, kd: keys[(l, kd)], lambda l, kd: W[(l, kd)],   # D: merge
                lambda l, kd: UP[(l, kd)], r, w.eta, alpha, rounding, w.sr_seed, per_launch=ML)
        ev[4].record()

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    for _ in range(args.warmup):
        step(events())
    torch.cuda.synchronize()
    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.counter_run:
        print("counter run done", flush=True)
        return
    K = args.steps
    ph = [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(4)]   # ms per phase per step
    med = [median(p) for p in ph]
    acc_ms, merge_ms = med[1], med[3]
    value = (acc_total + merge_total) / ((acc_ms + merge_ms) * 1e-3) / 1e9
    acc_gbs = acc_total / (acc_ms * 1e-3) / 1e9
    merge_gbs = merge_total / (merge_ms * 1e-3) / 1e9
    proj_gbs = proj_total / (med[0] * 1e-3) / 1e9
    acc_launch_us = acc_ms * 1e3 / M
    merge_launches = (layers + ML - 1) // ML
    merge_launch_us = merge_ms * 1e3 / merge_launches
    metric = ("sketch-accumulate + merge HBM GB/s (% of peak), Qwen-7B layer set, r=64"
              if w.name == DEFAULT_WORKLOAD else
              f"sketch-accumulate + merge HBM GB/s (% of peak), {w.name}")
    full = layers == w.layers
    acc_traffic = read_traffic(ACC_KERNEL, w.name, T, ML) if full else None
    merge_traffic = read_traffic(MERGE_KERNEL, w.name, T, ML) if full else None
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs of the workload's shapes, resident in HBM)",
        "config": {"workload": w.name, "layers": layers, "matrices": len(mats), "r": r, "T": T_mb,
                   "microbatches": M * G, "microbatches_per_launch": G, "merge_layers_per_launch": ML,
                   "rounding": rounding, "optimizer": w.optimizer,
                   "contexts": P, "vocab": Vv, "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2)},
    }
    # Roofline of the dominant kernel (the accumulate) from the method's own work per launch
    # (one microbatch of every matrix): 2Td + 4Tr + 8dr bytes and 2Tdr flops per matrix.
    rf = roofline(ACC_KERNEL, acc_total // M, acc_flops // M, acc_launch_us)
    rf.update({"traffic": acc_traffic["traffic_bytes_per_launch"] if acc_traffic else None,
               "bytes_per_launch": acc_total // M, "flops_per_launch": acc_flops // M,
               "launches": M * K, "avg_launch_us": round(sum(ph[1]) * 1e3 / (M * K), 3),
               "median_launch_us": round(acc_launch_us, 3)})
    # The matrix cores execute twice the method's flops (XAt enters as bf16 hi + lo); reported
    # beside the roofline, not used for it.
    rf["mfma_executed_tflops"] = round(2 * (acc_flops // M) / (acc_launch_us * 1e-6) / 1e12, 1)
    out["roofline"] = rf
    mrf = roofline(MERGE_KERNEL, merge_total // merge_launches, merge_flops // merge_launches,
                   merge_launch_us)
    mrf.update({"traffic": merge_traffic["traffic_bytes_per_launch"] if merge_traffic else None,
                "bytes_per_launch": merge_total // merge_launches, "launches": merge_launches * K,
                "median_launch_us": round(merge_launch_us, 3)})
    out["roofline_merge"] = mrf
    out["phases_ms"] = {"project": round(med[0], 3), "accumulate": round(acc_ms, 3),
                        "rowadam_q_alpha": round(med[2], 3), "merge": round(merge_ms, 3),
                        "statistic": f"median of {K} steps"}
    out["phases_ms_mean"] = {n_: round(sum(p) / K, 3) for n_, p in
                             zip(("project", "accumulate", "rowadam_q_alpha", "merge"), ph)}
    out["kernels_gbs"] = {"accumulate": round(acc_gbs, 1), "merge": round(merge_gbs, 1),
                          "project": round(proj_gbs, 1)}
    out["algorithmic_gb"] = {"accumulate": round(acc_total / 1e9, 3), "merge": round(merge_total / 1e9, 3),
                             "project": round(proj_total / 1e9, 3)}
    # Time bound of each phase: the larger of its HBM time at 8 TB/s and its matrix time at the
    # dense bf16 peak, both from the method's own bytes and flops.
    acc_bound = max(acc_total / PEAK_HBM_GBS / 1e6, acc_flops / PEAK_MFMA_BF16_TFS / 1e9)
    merge_bound = max(merge_total / PEAK_HBM_GBS / 1e6, merge_flops / PEAK_MFMA_BF16_TFS / 1e9)
    out["bound_ms"] = {"accumulate": round(acc_bound, 3), "merge": round(merge_bound, 3),
                       "accumulate_frac": round(acc_bound / acc_ms, 4),
                       "merge_frac": round(merge_bound / merge_ms, 4),
                       "accumulate_hilo_mfma_ms": round(2 * acc_flops / PEAK_MFMA_BF16_TFS / 1e9, 3)}
    # The part's own read and copy ceilings, measured here, and each phase against them (the
    # accumulate mostly reads; the merge reads and writes W in equal measure, like a copy).
    ceil = measure_ceilings(B, torch, dev)
    ceil["accumulate_frac_of_read"] = round(acc_gbs / ceil["read_gbs"], 4)
    ceil["merge_frac_of_copy"] = round(merge_gbs / ceil["copy_gbs"], 4)
    out["copy_ceiling"] = ceil
    # The reconstruction-cosine diagnostic on one dense gradient of the largest projection
    # (outside the timed step; the method itself never forms G).
    (_, dkind, dmid, dd, dk) = max(mats, key=lambda m: m[3] * m[4])
    G = randn((dd, dk), 1e-2)
    cws = B.workspace(B.reconstruction_cosine_ws_bytes(dd, dk, r), dev)
    cout = torch.empty((4,), dtype=torch.float64, device=dev)
    B.reconstruction_cosine(keys[(0, dkind)], G, r, out=cout, ws=cws)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        B.reconstruction_cosine(keys[(0, dkind)], G, r, out=cout, ws=cws)
    c1.record()
    torch.cuda.synchronize()
    cus = c0.elapsed_time(c1) * 1e3 / 5
    # the same gradient under the Gaussian projection variant (the pages' ablation)
    Ag = B.regen_A_gaussian(keys[(0, dkind)], r, dk, dev)
    Agp = B.pack_projection(Ag)
    gout = B.reconstruction_cosine_explicit(G, Ag, Agp, ws=cws)
    torch.cuda.synchronize()
    out["diagnostics"] = {"reconstruction_cosine": {
        "matrix": f"{dkind} {dd}x{dk} bf16", "r": r, "cos": round(float(cout[0].item()), 6),
        "cos_gaussian": round(float(gout[0].item()), 6),
        "us": round(cus, 1), "g_read_gbs": round(2 * dd * dk / (cus * 1e-6) / 1e9, 1)}}
    del Ag, Agp, G
    # The merge phase in the other rounding mode (the metric uses the workload's own), on
    # copies of the weights so the timed steps above are unaffected: median of five passes.
    other = "stochastic" if rounding == "nearest" else "nearest"
    Wc = {key_: t.clone() for key_, t in W.items()}
    times = []
    for rep in range(6):
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record()
        U.merge(layer_list, kinds, lambda l, kd: keys[(l, kd)], lambda l, kd: Wc[(l, kd)],
                lambda l, kd: UP[(l, kd)], r, w.eta, alpha, other, w.sr_seed, per_launch=ML)
        m1.record()
        torch.cuda.synchronize()
        if rep:
            times.append(m0.elapsed_time(m1))
    other_ms = median(times)
    out["merge_other_rounding"] = {"rounding": other, "ms": round(other_ms, 3),
                                   "gbs": round(merge_total / (other_ms * 1e-3) / 1e9, 1),
                                   "pct_of_peak": round(100 * merge_total / (other_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
    del Wc
    # The finite-difference check of the predicted KL at the step the update took.
    a_dev = float(alpha.item())
    ekl = B.exact_kl(z, zd, a_dev, w.tau)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    B.exact_kl(z, zd, a_dev, w.tau, out=ekl)
    e1.record()
    torch.cuda.synchronize()
    out["diagnostics"]["exact_kl"] = {
        "contexts": P, "vocab": Vv, "alpha": round(a_dev, 6), "predicted": float(a_dev * a_dev * q.item()),
        "exact": float(ekl.item()), "us": round(e0.elapsed_time(e1) * 1e3, 1)}
    if not args.skip_cpu_baseline and full and w.name == DEFAULT_WORKLOAD:
        out["cpu_baseline"] = cpu_baseline(w, rounding)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
