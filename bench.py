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

Modes:
  (default)              the benchmark; prints one JSON line
  --counter-run          a short run for rocprofv3 --pmc: a plain copy of known
                         size (the calibration) and one step of the workload
  --summarize-traffic F W  read the FETCH_SIZE (F) and WRITE_SIZE (W) counter
                         CSVs of two --counter-run passes and print the
                         calibrated HBM bytes per accumulate launch
--gpus above 1 is refused: this measures one GPU.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
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
ACC_KERNEL = "acc_bf16_table_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "acc_bf16_table_kernel.qwen2.5-7b-set-r64.traffic.md")
KERNEL_SOURCES = ["rank_gradient_sketching_logra_amd/csrc/kernels_sketch.hip",
                  "rank_gradient_sketching_logra_amd/csrc/kernels.h",
                  "rank_gradient_sketching_logra_amd/csrc/device_common.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rounding", default=None, choices=[None, "nearest", "stochastic"])
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=None, help="use fewer layers (profiling runs only)")
    ap.add_argument("--counter-run", action="store_true")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    return ap.parse_args()


def acc_bytes(T, d, r):
    return 2 * T * d + 4 * T * r + 8 * d * r


def merge_bytes(d, k, r):
    return 4 * d * k + 4 * d * r


def project_bytes(T, k, r):
    return 2 * T * k + 4 * T * r


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Calibrated HBM bytes per accumulate launch from the committed counter summary, or None
    when it is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    t = json.loads(line[len("traffic-json: "):])
                    if t.get("kernel_sources") == kernel_source_hash():
                        return t
    except OSError:
        pass
    return None


def summarize_traffic(fetch_csv, write_csv):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the copy and of the accumulate kernel;
    scale each counter by bytes-moved / counter-reading of the copy."""
    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = "acc" if ACC_KERNEL in name else "copy" if re.search(r"copy", name) else None
            if key is None:
                continue
            vals.setdefault(key, {}).setdefault(row["Dispatch_Id"], 0.0)
            vals[key][row["Dispatch_Id"]] += float(row["Counter_Value"])
        return {k: sorted(v.values()) for k, v in vals.items()}
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    # the calibration copy is the largest copy dispatch
    fcopy, wcopy = max(f["copy"]), max(w["copy"])
    ffac = CALIB_BYTES / (fcopy * 1024.0)
    wfac = CALIB_BYTES / (wcopy * 1024.0)
    facc = sum(f["acc"]) / len(f["acc"]) * 1024.0 * ffac
    wacc = sum(w["acc"]) / len(w["acc"]) * 1024.0 * wfac
    return {"kernel": ACC_KERNEL, "workload": "qwen2.5-7b-set-r64",
            "fetch_bytes_per_launch": round(facc), "write_bytes_per_launch": round(wacc),
            "traffic_bytes_per_launch": round(facc + wacc),
            "fetch_calibration": round(ffac, 4), "write_calibration": round(wfac, 4),
            "copy_fetch_kib": fcopy, "copy_write_kib": wcopy,
            "acc_dispatches": len(f["acc"]), "kernel_sources": kernel_source_hash()}


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


def main():
    args = parse()
    if args.summarize_traffic:
        t = summarize_traffic(*args.summarize_traffic)
        print("traffic-json: " + json.dumps(t))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from rank_gradient_sketching_logra_amd import binding as B
    from rank_gradient_sketching_logra_amd import synth

    w = synth.BY_NAME[args.workload]
    rounding = args.rounding or w.rounding
    layers = args.layers or w.layers
    if args.counter_run:
        args.steps, args.warmup = 1, 0
    T, r, M = w.T, w.r, w.microbatches
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
        # the calibration: a plain copy of CALIB_BYTES
        src = torch.empty((CALIB_BYTES // 2,), dtype=torch.bfloat16, device=dev).normal_(generator=g)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    mats = w.matrices(layers=range(layers))
    # Inputs X: q/k/v share the attention input, gate/up the MLP input.
    shared = {"q": "att", "k": "att", "v": "att", "o": "o", "gate": "mlp", "up": "mlp", "down": "down"}
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

    by_layer = {}
    for (l, kind, mid, d, k) in mats:
        by_layer.setdefault(l, []).append((kind, d, k))
    acc_total = sum(acc_bytes(T, d, r) for (_, _, _, d, _) in mats) * M
    merge_total = sum(merge_bytes(d, k, r) for (_, _, _, d, k) in mats)
    proj_total = sum(project_bytes(T, k, r) for (_, _, _, d, k) in mats) * M
    n_acc_launch = M
    acc_per_launch = acc_total // n_acc_launch
    t_step = 0

    def step(ev):
        nonlocal t_step
        t_step += 1
        for s in S.values():
            s.zero_()
        ev[0].record()
        for mb in range(M):                          # A: forward-side projections
            # one persistent launch per microbatch over every matrix of every layer
            B.project_input_table([(keys[(l, kind)], X[(sid[(l, mb)], shared[kind])], None,
                                    PL[(l, mb, kind)])
                                   for l in range(layers) for (kind, d, k) in by_layer[l]],
                                  r, ws=proj_ws)
        ev[1].record()
        for mb in range(M):                          # B: backward-side sketch accumulation
            # one persistent launch per microbatch over every matrix of every layer
            B.sketch_accumulate_table([(D[(sid[(l, mb)], kind)], PL[(l, mb, kind)], S[(l, kind)])
                                       for l in reversed(range(layers)) for (kind, d, k) in by_layer[l]],
                                      r, ws=acc_ws)
        ev[2].record()
        # C: optimiser (U in the merge's packed form), every sketch in one grouped call
        B.rowadam_packed_grouped([(S[key_], V[key_], UP[key_]) for key_ in S], r, t_step, w.beta,
                                 w.eps, ws=ra_ws)
        B.predicted_kl_q(z, zd, w.tau, out=q, ws=kl_ws)
        B.step_alpha_dev(q, w.delta, w.alpha_max, out=alpha)
        ev[3].record()
        for l in range(layers):                      # D: merge (one launch per layer)
            B.merge_grouped_packed([(keys[(l, kind)], W[(l, kind)], UP[(l, kind)]) for (kind, d, k) in by_layer[l]],
                                   r, w.eta, scale_dev=alpha, mode=rounding, sr_seed=w.sr_seed)
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
    ph = [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(4)]   # ms per phase per step
    tot = [sum(p) for p in ph]
    K = args.steps
    acc_ms, merge_ms = tot[1] / K, tot[3] / K
    value = (acc_total + merge_total) / ((acc_ms + merge_ms) * 1e-3) / 1e9
    acc_gbs = acc_total / (acc_ms * 1e-3) / 1e9
    merge_gbs = merge_total / (merge_ms * 1e-3) / 1e9
    proj_gbs = proj_total / (tot[0] / K * 1e-3) / 1e9
    avg_launch_us = acc_ms * 1e3 / n_acc_launch
    traffic = read_traffic() if w.name == DEFAULT_WORKLOAD else None
    metric = ("sketch-accumulate + merge HBM GB/s (% of peak), Qwen-7B layer set, r=64"
              if w.name == DEFAULT_WORKLOAD else
              f"sketch-accumulate + merge HBM GB/s (% of peak), {w.name}")
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
        "config": {"workload": w.name, "layers": layers, "matrices": len(mats), "r": r, "T": T,
                   "microbatches": M, "rounding": rounding, "optimizer": w.optimizer,
                   "contexts": P, "vocab": Vv, "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2)},
        "roofline": {"bound": "hbm", "kernel": ACC_KERNEL,
                     "achieved": round(acc_per_launch / (avg_launch_us * 1e-6) / 1e9, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(acc_per_launch / (avg_launch_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
                     "bytes_per_launch": acc_per_launch, "launches": n_acc_launch * K,
                     "avg_launch_us": round(avg_launch_us, 3)},
        "phases_ms": {"project": round(tot[0] / K, 3), "accumulate": round(acc_ms, 3),
                      "rowadam_q_alpha": round(tot[2] / K, 3), "merge": round(merge_ms, 3)},
        "kernels_gbs": {"accumulate": round(acc_gbs, 1), "merge": round(merge_gbs, 1),
                        "project": round(proj_gbs, 1)},
        "algorithmic_gb": {"accumulate": round(acc_total / 1e9, 3), "merge": round(merge_total / 1e9, 3),
                           "project": round(proj_total / 1e9, 3)},
    }
    # Time bound of each phase: the larger of its HBM time at 8 TB/s and its matrix time at
    # the dense bf16 peak, the matrix work counted twice (XAt and U enter as bf16 hi + lo).
    acc_flops = sum(2 * T * d * r for (_, _, _, d, _) in mats) * M
    merge_flops = sum(2 * d * k * r for (_, _, _, d, k) in mats)
    acc_bound = max(acc_total / PEAK_HBM_GBS / 1e6, 2 * acc_flops / PEAK_MFMA_BF16_TFS / 1e9)
    merge_bound = max(merge_total / PEAK_HBM_GBS / 1e6, 2 * merge_flops / PEAK_MFMA_BF16_TFS / 1e9)
    out["bound_ms"] = {"accumulate": round(acc_bound, 3), "merge": round(merge_bound, 3),
                       "accumulate_frac": round(acc_bound / acc_ms, 4),
                       "merge_frac": round(merge_bound / merge_ms, 4),
                       "accumulate_mfma_tflops_executed": round(2 * acc_flops / (acc_ms * 1e-3) / 1e12, 1)}
    if w.name != DEFAULT_WORKLOAD and 2 * acc_flops / PEAK_MFMA_BF16_TFS / 1e9 > acc_total / PEAK_HBM_GBS / 1e6:
        # matrix-bound accumulate (r = 256): its roofline is the matrix peak, in the
        # algorithmic flops 2Tdr per matrix
        fl = acc_flops // n_acc_launch
        out["roofline"].update({"bound": "mfma", "achieved": round(fl / (avg_launch_us * 1e-6) / 1e12, 2),
                                "peak": PEAK_MFMA_BF16_TFS, "unit": "TFLOP/s",
                                "frac": round(fl / (avg_launch_us * 1e-6) / 1e12 / PEAK_MFMA_BF16_TFS, 4),
                                "flops_per_launch": fl})
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
    del Ag, Agp
    # The merge phase in the other rounding mode (the metric uses the workload's own), on
    # copies of the weights so the timed steps above are unaffected.
    other = "stochastic" if rounding == "nearest" else "nearest"
    Wc = {key_: t.clone() for key_, t in W.items()}
    for rep in range(2):
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record()
        for l in range(layers):
            B.merge_grouped_packed([(keys[(l, kind)], Wc[(l, kind)], UP[(l, kind)]) for (kind, d, k) in by_layer[l]],
                                   r, w.eta, scale_dev=alpha, mode=other, sr_seed=w.sr_seed)
        m1.record()
        torch.cuda.synchronize()
    other_ms = m0.elapsed_time(m1)
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
    if not args.skip_cpu_baseline and layers == w.layers and w.name == DEFAULT_WORKLOAD:
        out["cpu_baseline"] = cpu_baseline(w, rounding)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
