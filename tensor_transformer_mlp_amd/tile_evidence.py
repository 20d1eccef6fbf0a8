"""Measured evidence for the bf16 GEMM's tile choice.

    python -m tensor_transformer_mlp_amd.tile_evidence run OUT.json [--workloads a,b] [--reps R]
        [--launches L] [--settle-seconds S]
    python -m tensor_transformer_mlp_amd.tile_evidence summary RUN.json MFMA_DIR FETCH_DIR WRITE_DIR OUT.md \\
        "COMMANDS"

`run` (one GPU) takes each workload's bf16 shards (the benchmark's seeded
inputs) through the three GEMM steps of the forward pass -- the column step
(bias + GeLU, bf16 Y_i), the row step (fp32 partials Z_i) and the row step
with the shard sum -- once with every tile of the GEMM's table that can run
the step, all shards of a step in one launch as the library does.  Each
(step, tile) is timed with a HIP event pair around `launches` back-to-back
launches on the launching stream, `reps` times (median kept), after a settle
phase that brings the clock up.  Every tile's output is compared with the
library's own choice, bit for bit.

Run under `rocprofv3 --pmc ...` the same command gives the counters (and
the duration) of every dispatch; `summary` joins three such runs (MFMA counters, then
FETCH_SIZE, then WRITE_SIZE) with the timings:

* MFMA busy: rocprofv3's derived MfmaUtil, the MFMA pipes' busy cycles
  (SQ_VALU_MFMA_BUSY_CYCLES, summed over all SIMDs) over the kernel's active
  cycles (GRBM_GUI_ACTIVE) times the SIMD count;
* MFMA flop: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 against the algorithmic
  2 M N K n (padding of ragged tiles would show as excess);
* clock: the active cycles over the dispatch's duration in the same run;
* HBM bytes: FETCH_SIZE and WRITE_SIZE scaled by the plain-copy calibration
  kept in profiles/traffic.json (bytes per counter unit, a property of the
  chip, not of these kernels).

Dispatches are matched to (workload, step, tile) by the kernel's template
arguments and its grid size, which differ between every pair of cases.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import re
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

STEPS = ("col", "row", "sum")            # tp_mlp_step_tile's steps 0, 1, 2
STEP_EPI = {"col": 0, "row": 1, "sum": 1}  # the kernel's epilogue template argument
SIMDS = 1024                             # MI355X: 256 CUs x 4 SIMDs
PEAK_BF16 = 2516.6                       # TFLOP/s, dense


def step_shape(step: str, M: int, H: int, Fk: int):
    """(M, N, K) of one shard's GEMM in a step."""
    return (M, Fk, H) if step == "col" else (M, H, Fk)


def workgroups(tile: dict, step: str, n: int, M: int, N: int) -> int:
    tiles = -(-M // tile["bm"]) * -(-N // tile["bn"])
    return tiles if step == "sum" else tiles * n


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def run(out_json: str, workloads, reps: int, launches: int, settle: float) -> None:
    import numpy as np
    import torch

    import tensor_transformer_mlp_amd as tpm
    from tensor_transformer_mlp_amd import inputs

    tpm.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    tiles = tpm.tp_gemm_tiles()
    records = []

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    for wname in workloads:
        w = inputs.WORKLOADS[wname]
        if w.dtype != "bf16":
            raise ValueError("the tile table is the bf16 GEMM's: %s is %s" % (wname, w.dtype))
        M, H, Fk, n = w.M, w.H, w.Fk, w.k
        inp = inputs.make_inputs(w)
        X = up(inp["X"])
        Wd, bd, Vd = up(inp["W"]), up(inp["b"]), up(inp["V"])
        Ws = [Wd[:, i * Fk:(i + 1) * Fk].contiguous() for i in range(n)]
        bs = [bd[i * Fk:(i + 1) * Fk].contiguous() for i in range(n)]
        Vs = [Vd[i * Fk:(i + 1) * Fk, :].contiguous() for i in range(n)]
        del Wd, bd, Vd, inp
        Y0 = [torch.empty(M, Fk, dtype=torch.bfloat16, device=dev) for _ in range(n)]
        Y = [torch.empty(M, Fk, dtype=torch.bfloat16, device=dev) for _ in range(n)]
        P0 = [torch.empty(M, H, device=dev) for _ in range(n)]
        P = [torch.empty(M, H, device=dev) for _ in range(n)]
        S0 = torch.empty(M, H, device=dev)
        S = torch.empty(M, H, device=dev)
        tpm.tp_mlp_col_gelu_shards(X, Ws, bs, Y0)
        tpm.tp_mlp_row_partial_shards(Y0, Vs, P0)
        tpm.tp_mlp_row_partial_shards(Y0, Vs, [S0], sum_shards=True)
        torch.cuda.synchronize()
        _log("workload %s: M=%d H=%d Fk=%d, %d shards per launch" % (wname, M, H, Fk, n))

        def launcher(step, t):
            if step == "col":
                return lambda: tpm.tp_mlp_col_gelu_shards_tile(t, X, Ws, bs, Y, stream=stream)
            if step == "row":
                return lambda: tpm.tp_mlp_row_partial_shards_tile(t, Y0, Vs, P, stream=stream)
            return lambda: tpm.tp_mlp_row_partial_shards_tile(t, Y0, Vs, [S], sum_shards=True, stream=stream)

        def clear(step):
            for t in (Y if step == "col" else P if step == "row" else [S]):
                t.fill_(float("nan"))

        def same(step):
            if step == "col":
                return all(torch.equal(Y[i], Y0[i]) for i in range(n))
            if step == "row":
                return all(torch.equal(P[i], P0[i]) for i in range(n))
            return torch.equal(S, S0)

        def library(step):
            if step == "col":
                return lambda: tpm.tp_mlp_col_gelu_shards(X, Ws, bs, Y, stream=stream)
            if step == "row":
                return lambda: tpm.tp_mlp_row_partial_shards(Y0, Vs, P, stream=stream)
            return lambda: tpm.tp_mlp_row_partial_shards(Y0, Vs, [S], sum_shards=True, stream=stream)

        first = True
        for si, step in enumerate(STEPS):
            Mg, N, K = step_shape(step, M, H, Fk)
            picked = tpm.tp_mlp_step_tile(si, n, M, H, Fk)
            # every tile of the table, then (t = -1) the library's own call
            for t, shape in list(enumerate(tiles)) + [(-1, tiles[picked])]:
                f = launcher(step, t) if t >= 0 else library(step)
                clear(step)
                try:
                    f()
                except tpm.TpMlpError as e:
                    if e.code != -2 or t < 0:
                        raise
                    continue  # this tile is not compiled for the step
                torch.cuda.synchronize()
                identical = bool(same(step))
                if first and settle > 0:
                    t_end = time.perf_counter() + settle
                    while time.perf_counter() < t_end:
                        f()
                        torch.cuda.synchronize()
                    first = False
                f()
                times = []
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(launches):
                        f()
                    e1.record(stream)
                    e1.synchronize()
                    times.append(e0.elapsed_time(e1) / launches)
                ms = statistics.median(times)
                flop = 2.0 * Mg * N * K * n
                rec = {"workload": wname, "step": step, "tile": t, "picked": t == picked or t < 0, **shape,
                       "M": Mg, "N": N, "K": K, "n": n, "workgroups": workgroups(shape, step, n, Mg, N),
                       "flop": flop, "ms": ms, "tflops": flop / ms / 1e9, "bitwise_equal_to_picked": identical}
                records.append(rec)
                _log("  %-3s tile %2d %3dx%3d %dw %ds%s: %8.1f us %7.1f TFLOP/s%s" % (
                    step, t, shape["bm"], shape["bn"], shape["waves"], shape["stages"], " *" if t == picked else "  ",
                    ms * 1e3, rec["tflops"], "" if identical else "  OUTPUT DIFFERS"))
        del X, Ws, bs, Vs, Y0, Y, P0, P, S0, S
        torch.cuda.empty_cache()
    json.dump({"records": records, "reps": reps, "launches": launches}, open(out_json, "w"), indent=1)
    bad = [r for r in records if not r["bitwise_equal_to_picked"]]
    if bad:
        raise SystemExit("%d (step, tile) outputs differ from the picked tile's" % len(bad))


# --------------------------------------------------------------------------- summary

_KERNEL = re.compile(r"gemm_bf16_kernel<([^>]*)>")


def _targs(name: str):
    m = _KERNEL.search(name)
    if not m:
        return None
    out = []
    for a in m.group(1).split(","):
        a = re.sub(r"^\([^)]*\)", "", a.strip())
        out.append({"true": 1, "false": 0}.get(a, None) if a in ("true", "false") else int(a))
    return out  # EPI, LAYOUT, BM, BN, WM, WN, NBUF, KTAIL, GSUM


def _csv(d: str, pattern: str):
    paths = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not paths:
        raise FileNotFoundError("no %s under %s" % (pattern, d))
    return list(csv.DictReader(open(paths[0])))


def _dispatches(d: str, counters):
    """{dispatch id: {"name", "grid", counter: value, "ns": duration}} of the GEMM dispatches."""
    out = {}
    for r in _csv(d, "*counter_collection.csv"):
        if r["Counter_Name"] not in counters or "gemm_bf16_kernel" not in r["Kernel_Name"]:
            continue
        e = out.setdefault(r["Dispatch_Id"], {
            "name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
            "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
            "vgpr": int(r["VGPR_Count"]), "agpr": int(r["Accum_VGPR_Count"]),
            "scratch": int(r["Scratch_Size"]), "lds": int(r["LDS_Block_Size"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _match(records, disp):
    """{record index: [dispatch dicts]} by template arguments and grid size."""
    by_key = collections.defaultdict(list)
    for e in disp.values():
        a = _targs(e["name"])
        if a:
            by_key[(a[0], a[2], a[3], a[4] * a[5], a[6], a[8], e["grid"])].append(e)
    out = {}
    for i, r in enumerate(records):
        key = (STEP_EPI[r["step"]], r["bm"], r["bn"], r["waves"], r["stages"], int(r["step"] == "sum"),
               r["workgroups"] * r["waves"] * 64)
        # the library's own call shares its kernel with the picked tile's row:
        # counters only on the latter
        out[i] = by_key.get(key, []) if r["tile"] >= 0 else []
    return out


def _median(vals):
    return statistics.median(vals) if vals else None


def summary(run_json, mfma_dir, fetch_dir, write_dir, out_md, commands):
    rec = json.load(open(run_json))
    records = rec["records"]
    cal = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["copy_calibration"]
    f_scale = cal["bytes"] / cal["fetch_size"]
    w_scale = cal["bytes"] / cal["write_size"]
    mf = _match(records, _dispatches(mfma_dir, ("MfmaUtil", "SQ_VALU_MFMA_BUSY_CYCLES",
                                                "SQ_INSTS_VALU_MFMA_MOPS_BF16")))
    fe = _match(records, _dispatches(fetch_dir, ("FETCH_SIZE",)))
    wr = _match(records, _dispatches(write_dir, ("WRITE_SIZE",)))
    lines = ["# Tile choice of the bf16 GEMM: time, MFMA busy and HBM traffic per tile", "",
             "Commands (run from the repository root on one MI355X):", "", "```", commands.strip(), "```", "",
             "Each row is one forward step of a workload's shards, all shards in one launch, with one tile of "
             "the table (BM x BN outputs per workgroup, waves, LDS stages); `*` marks the tile the library "
             "picks, `library` the library's own call (the picked tile's kernel, timed through the "
             "library's entry point).  Time: median of %d "
             "event-timed groups of %d launches.  MFMA busy: rocprofv3 MfmaUtil "
             "(MFMA busy cycles over active cycles x %d SIMDs).  MFMA flop / algorithmic: "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 over 2 M N K n.  Clock: active cycles over the "
             "dispatch's duration in the counter run (each dispatch alone on the GPU).  Spill: scratch "
             "bytes per lane of the kernel (register spills).  HBM: FETCH_SIZE and WRITE_SIZE times the plain-copy "
             "calibration (%.0f and %.0f bytes per unit).  Every tile's output was bit-identical to the "
             "picked tile's." % (rec["reps"], rec["launches"], SIMDS, f_scale, w_scale), "",
             "| workload | step | tile | BM x BN, waves, stages | spill (B/lane) | workgroups "
             "| time (us) | TFLOP/s | % of peak | MFMA busy % | MFMA flop / algorithmic | clock (GHz) "
             "| HBM read (MB) | HBM write (MB) | HBM GB/s |",
             "|---|---|---:|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for i, r in enumerate(records):
        m = mf[i]
        util = _median([e["MfmaUtil"] for e in m if "MfmaUtil" in e])
        mops = _median([e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for e in m if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in e])
        clock = None
        busy = [e for e in m if "SQ_VALU_MFMA_BUSY_CYCLES" in e and e.get("MfmaUtil") and e["ns"] > 0]
        if busy:
            # active cycles = busy cycles / (SIMDs x utilisation)
            clock = _median([e["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * e["MfmaUtil"] / 100.0) / e["ns"]
                             for e in busy])
        rb = _median([e["FETCH_SIZE"] for e in fe[i] if "FETCH_SIZE" in e])
        wb = _median([e["WRITE_SIZE"] for e in wr[i] if "WRITE_SIZE" in e])
        rb = rb * f_scale if rb is not None else None
        wb = wb * w_scale if wb is not None else None
        gbs = (rb + wb) / (r["ms"] * 1e-3) / 1e9 if rb is not None and wb is not None else None
        fmt = lambda v, f: ("%" + f) % v if v is not None else "-"
        regs = "%d" % m[0]["scratch"] if m else "-"
        if r["tile"] < 0:
            label = "library"
        else:
            label = "%d%s" % (r["tile"], " *" if r["picked"] else "")
        lines.append("| %s | %s | %s | %dx%d, %d, %d | %s | %d | %.1f | %.0f | %.1f | %s | %s | %s | %s | %s "
                     "| %s |" % (
            r["workload"], r["step"], label, r["bm"], r["bn"], r["waves"],
            r["stages"], regs, r["workgroups"], r["ms"] * 1e3, r["tflops"], 100 * r["tflops"] / PEAK_BF16,
            fmt(util, ".1f"), fmt(mops * 512 / r["flop"] if mops is not None else None, ".3f"),
            fmt(clock, ".2f"), fmt(rb / 1e6 if rb is not None else None, ".1f"),
            fmt(wb / 1e6 if wb is not None else None, ".1f"), fmt(gbs, ".0f")))
    open(out_md, "w").write("\n".join(lines) + "\n")


def main(argv):
    if argv and argv[0] == "run":
        ap = argparse.ArgumentParser(prog="tile_evidence run")
        ap.add_argument("out")
        ap.add_argument("--workloads", default="gpt2_small,llama7b,gpt3_175b,long_seq")
        ap.add_argument("--reps", type=int, default=3)
        ap.add_argument("--launches", type=int, default=10)
        ap.add_argument("--settle-seconds", type=float, default=0.5)
        a = ap.parse_args(argv[1:])
        run(a.out, [w for w in a.workloads.split(",") if w], a.reps, a.launches, a.settle_seconds)
    elif argv and argv[0] == "summary" and len(argv) == 7:
        summary(*argv[1:])
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
