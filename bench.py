#!/usr/bin/env python3
"""Benchmark of the tensor-parallel MLP shard forward on one MI355X.

One step = one call of tp_mlp_shard_forward: for each of the k shards the
column GEMM + bias + GeLU and the row GEMM, then the on-device shard sum, over
one batch of seeded synthetic inputs already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--variant literal|fused]

Prints ONE JSON line (metric, value in TFLOP/s, ms_per_step, roofline of the
dominant kernel, CPU-oracle baseline) on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TP-shard MLP forward TFLOP/s (bf16) and % of MI355X MFMA peak"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # dense MFMA: 256 CU x 2.4 GHz x (4096 | 256) flop/clk
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt2_small")
    ap.add_argument("--variant", choices=["literal", "fused"], default="literal")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (0 disables the CPU leg)")
    ap.add_argument("--kernel-steps", type=int, default=None,
                    help="steps of the per-kernel timing pass (default: --steps)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain float32 copy kernel (y = x * 1) over MIB MiB, 5 times: "
                         "the known-size reference for the HBM byte counters")
    return ap.parse_args()


def kernel_bytes(kind, w, elt):
    M, H, Fk, k = w.M, w.H, w.Fk, w.k
    if kind == "col_gelu":
        return (M * H + H * Fk + Fk + M * Fk) * elt
    if kind == "row_partial":
        return (M * Fk + Fk * H) * elt + M * H * 4
    if kind == "row_partial_accum":
        return (M * Fk + Fk * H) * elt + 2 * M * H * 4
    if kind == "shard_reduce":
        return (k + 1) * M * H * 4
    raise KeyError(kind)


def kernel_flops(kind, w):
    if kind.startswith("col_gelu") or kind.startswith("row_partial"):
        return 2 * w.M * w.H * w.Fk
    return (w.k - 1) * w.M * w.H


def main():
    args = parse()
    if args.gpus != 1:
        log("bench.py measures one GPU only: this build has no multi-GPU path "
            "(the k shards run back to back on one device); run with --gpus 1")
        sys.exit(2)

    import numpy as np
    import torch
    import tensor_transformer_mlp_amd as tpm
    from tensor_transformer_mlp_amd import inputs

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                          "launches": 5}), flush=True)
        return

    tpm.lib()  # raises if the HIP library is not built: there is no fallback
    w = inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fused = args.variant == "fused"
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    elt = 2 if w.dtype == "bf16" else 4

    log("workload %s: M=%d H=%d F=%d k=%d dtype=%s variant=%s" % (w.name, w.M, w.H, w.F, w.k, w.dtype,
                                                                 args.variant))
    t = time.time()
    inp = inputs.make_inputs(w)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    X = up(inp["X"])
    Wd, bd, Vd = up(inp["W"]), up(inp["b"]), up(inp["V"])
    Fk = w.Fk
    Ws = [Wd[:, i * Fk:(i + 1) * Fk].contiguous() for i in range(w.k)]
    bs = [bd[i * Fk:(i + 1) * Fk].contiguous() for i in range(w.k)]
    Vs = [Vd[i * Fk:(i + 1) * Fk, :].contiguous() for i in range(w.k)]
    del Wd, bd, Vd
    Z = torch.empty(w.M, w.H, dtype=torch.float32, device=dev)
    flags = tpm.TP_FUSED_ACCUM if fused else 0
    ws_bytes = tpm.tp_mlp_workspace_bytes(w.k, w.M, w.H, Fk, tpm.TP_BF16 if w.dtype == "bf16" else tpm.TP_F32,
                                          flags)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log("inputs ready in %.1f s (workspace %.1f MB)" % (time.time() - t, ws_bytes / 1e6))

    def step():
        tpm.tp_mlp_shard_forward(X, Ws, bs, Vs, Z=Z, workspace=ws, fused=fused)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    tflops = w.flop / (ms * 1e-3) / 1e12
    log("timed %d steps: %.4f ms/step, %.1f TFLOP/s (%.1f%% of %s peak)" % (
        args.steps, ms, tflops, 100 * tflops / PEAK_TFLOPS[w.dtype], w.dtype))
    if not bool(torch.isfinite(Z).all()):
        raise RuntimeError("non-finite output")

    # Per-kernel pass: the kernels of one step through the per-kernel entry
    # points, in the same launch configuration; each kind's launches of the
    # step run back to back between one HIP event pair on the stream they are
    # launched on, and a spin kernel queued first keeps the GPU busy while the
    # host enqueues, so no host gap falls inside a pair.
    stream = torch.cuda.current_stream()
    ks = args.kernel_steps or args.steps
    Y = torch.empty(w.M, Fk, dtype=tdt, device=dev)
    parts = [torch.empty(w.M, w.H, dtype=torch.float32, device=dev) for _ in range(w.k)]
    kinds = ["col_gelu", "row_partial"] + (["row_partial_accum"] if fused and w.k > 1 else []) + \
        (["shard_reduce"] if not fused and w.k > 1 else [])
    durs = {kd: [] for kd in kinds}
    nlaunch = {"col_gelu": w.k, "row_partial": 1 if fused else w.k, "row_partial_accum": w.k - 1,
               "shard_reduce": 1}

    def launch(kind):
        if kind == "col_gelu":
            for i in range(w.k):
                tpm.tp_mlp_col_gelu(X, Ws[i], bs[i], Y_i=Y)
        elif kind == "row_partial":
            for i in range(nlaunch["row_partial"]):
                tpm.tp_mlp_row_partial(Y, Vs[i], Z_i=Z if fused else parts[i])
        elif kind == "row_partial_accum":
            for i in range(1, w.k):
                tpm.tp_mlp_row_partial(Y, Vs[i], Z_i=Z, accumulate=True)
        else:
            tpm.tp_shard_reduce(parts, Z=Z)

    spin = getattr(torch.cuda, "_sleep", None)
    for it in range(args.warmup + ks):
        if spin is not None:
            spin(3_000_000)
        rec = []
        for kind in kinds:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch(kind)
            b.record(stream)
            rec.append((kind, a, b))
        torch.cuda.synchronize()
        if it >= args.warmup:
            for kind, a, b in rec:
                durs[kind].append(a.elapsed_time(b) / nlaunch[kind])
    kern = {}
    for kind, d in durs.items():
        if not d:
            continue
        avg = float(np.mean(d))
        per_step = avg * nlaunch[kind]
        kern[kind] = {"launches_per_step": nlaunch[kind], "avg_ms": avg, "ms_per_step": per_step,
                      "flop": kernel_flops(kind, w), "bytes": kernel_bytes(kind, w, elt)}
        log("  %-18s %2d/step  avg %.4f ms  (%.4f ms/step)  %.1f TFLOP/s  %.0f GB/s" % (
            kind, nlaunch[kind], avg, per_step, kernel_flops(kind, w) / avg / 1e9,
            kernel_bytes(kind, w, elt) / avg / 1e6))
    dom = max(kern, key=lambda k_: kern[k_]["ms_per_step"])
    d = kern[dom]
    peak_f = PEAK_TFLOPS[w.dtype]
    t_mfma = d["flop"] / (peak_f * 1e12)
    t_hbm = d["bytes"] / (PEAK_HBM_GBS * 1e9)
    if dom != "shard_reduce" and t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": d["flop"] / (d["avg_ms"] * 1e-3) / 1e12, "peak": peak_f,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": d["bytes"] / (d["avg_ms"] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name, args.variant, dom)
    roof["kernel"] = dom
    roof["avg_ms"] = d["avg_ms"]

    cpu = None
    if args.cpu_baseline_seconds > 0:
        cpu = cpu_baseline(w, inp, args.cpu_baseline_seconds)

    out = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded Philox normals, random-init weights)",
        "pct_of_peak": round(100 * tflops / PEAK_TFLOPS[w.dtype], 2),
        "config": dict(w.describe(), variant=args.variant, parallelism="tp%d shards on 1 GPU" % w.k),
        "roofline": roof,
        "kernels": {k_: {"avg_ms": round(v["avg_ms"], 5), "per_step": v["launches_per_step"]}
                    for k_, v in kern.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def measured_traffic(workload, variant, kind):
    """HBM bytes per launch of `kind` from the committed counter summary
    (profiles/traffic.json), or None if that summary does not cover this
    kernel or was taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "tensor_transformer_mlp_amd", "csrc", "tp_mlp_kernels.hip")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    e = rec.get("entries", {}).get("%s/%s/%s" % (workload, variant, kind))
    if not e:
        return None
    return e["hbm_bytes_per_launch"]


def cpu_baseline(w, inp, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    the first rows of the batch (all k shards, full W and V), or, when the whole
    batch takes less than the target time, whole-batch passes repeated up to it."""
    import numpy as np
    import oracle

    oracle.build_oracle()
    X64 = oracle.widen(inp["X"])
    W64, b64, V64 = oracle.widen(inp["W"]), oracle.widen(inp["b"]), oracle.widen(inp["V"])
    probe = min(w.M, 32)
    t = time.perf_counter()
    oracle.forward_rows(X64, W64, b64, V64, w.k, np.arange(probe))
    tp = time.perf_counter() - t
    rows = int(min(w.M, max(probe, probe * target_s / max(tp, 1e-6))))
    passes, dt = 0, 0.0
    while passes == 0 or (rows == w.M and dt < target_s and passes < 100):
        t = time.perf_counter()
        oracle.forward_rows(X64, W64, b64, V64, w.k, np.arange(rows))
        dt += time.perf_counter() - t
        passes += 1
    flop = 4 * rows * w.H * w.F * passes
    val = flop / dt / 1e12
    what = ("%d full passes over all %d rows" % (passes, w.M)) if rows == w.M else \
        ("rows 0..%d of %d" % (rows - 1, w.M))
    log("cpu oracle: %s in %.2f s with %d threads: %.4f TFLOP/s" % (what, dt, oracle.max_threads(), val))
    return {"value": val, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "%s (all %d shards, full W and V), fp64, %.1f s" % (what, w.k, dt)}


if __name__ == "__main__":
    main()
