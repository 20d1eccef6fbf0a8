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

    # Per-kernel pass: the same kernels through the per-step entry points, with
    # a HIP event pair around every launch on the stream they run on.
    stream = torch.cuda.current_stream()
    ks = args.kernel_steps or args.steps
    Y = torch.empty(w.M, Fk, dtype=tdt, device=dev)
    parts = [Z] + [torch.empty(w.M, w.H, dtype=torch.float32, device=dev) for _ in range(w.k - 1)]
    durs = {"col_gelu": [], "row_partial": [], "shard_reduce": []}
    if fused:
        durs["row_partial_accum"] = []

    def timed(kind, fn, rec):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        rec.append((kind, a, b))

    for it in range(args.warmup + ks):
        rec = []
        for i in range(w.k):
            timed("col_gelu", lambda: tpm.tp_mlp_col_gelu(X, Ws[i], bs[i], Y_i=Y), rec)
            if fused:
                kind = "row_partial" if i == 0 else "row_partial_accum"
                timed(kind, lambda: tpm.tp_mlp_row_partial(Y, Vs[i], Z_i=Z, accumulate=i > 0), rec)
            else:
                timed("row_partial", lambda: tpm.tp_mlp_row_partial(Y, Vs[i], Z_i=parts[i]), rec)
        if not fused and w.k > 1:
            timed("shard_reduce", lambda: tpm.tp_shard_reduce(parts, Z=Z), rec)
        torch.cuda.synchronize()
        if it >= args.warmup:
            for kind, a, b in rec:
                durs[kind].append(a.elapsed_time(b))
    kern = {}
    for kind, d in durs.items():
        if not d:
            continue
        avg = float(np.mean(d))
        per_step = avg * len(d) / ks
        kern[kind] = {"launches_per_step": len(d) // ks, "avg_ms": avg, "ms_per_step": per_step,
                      "flop": kernel_flops(kind, w), "bytes": kernel_bytes(kind, w, elt)}
        log("  %-18s %2d/step  avg %.4f ms  (%.4f ms/step)  %.1f TFLOP/s  %.0f GB/s" % (
            kind, len(d) // ks, avg, per_step, kernel_flops(kind, w) / avg / 1e9,
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
    roof["traffic"] = None
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


def cpu_baseline(w, inp, target_s):
    """The fp64 oracle, as it stands, on a bounded row sample of the same workload."""
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
    t = time.perf_counter()
    oracle.forward_rows(X64, W64, b64, V64, w.k, np.arange(rows))
    dt = time.perf_counter() - t
    flop = 4 * rows * w.H * w.F
    val = flop / dt / 1e12
    log("cpu oracle: %d rows in %.2f s with %d threads: %.4f TFLOP/s" % (rows, dt, oracle.max_threads(), val))
    return {"value": val, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "rows 0..%d of %d (all %d shards, full W and V), fp64, %.1f s" % (rows - 1, w.M, w.k, dt)}


if __name__ == "__main__":
    main()
