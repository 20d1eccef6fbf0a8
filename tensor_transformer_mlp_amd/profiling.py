"""Summaries of rocprofv3 output for the benchmark's kernels.

    python -m tensor_transformer_mlp_amd.profiling stats  TRACE_DIR  OUT.md  "COMMAND"
    python -m tensor_transformer_mlp_amd.profiling traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR \
        COPY_WRITE_DIR COPY_BYTES WORKLOAD VARIANT OUT.md "COMMANDS"

`stats` turns a `rocprofv3 --kernel-trace --stats` result into a Markdown table
(per kernel: calls, average and total duration).  `traffic` turns two
`--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of the benchmark, plus the same two
counters on a plain copy kernel of known size, into HBM bytes per launch of
each kernel kind (the copy run gives the factor between the counters' KiB and
real bytes), writes a Markdown summary, and records the figures in
profiles/traffic.json together with the SHA-256 of the kernel source they were
taken on (the benchmark reports them only while that source is unchanged).
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")

# Kernel kinds by (epilogue, operand layout, group sum) template arguments of
# the GEMMs: epilogues 0 bias+GeLU, 1 fp32 store, 2 fp32 accumulate,
# 3 bias+GeLU+GeLU', 4 multiply by aux, 5 SiLU(gate) * up, 6 bias only;
# layouts 0 NN, 1 NT, 2 TN.
_GEMM_KIND = {("0", "0"): "col_gelu", ("1", "0"): "row_partial", ("2", "0"): "row_partial_accum",
              ("3", "0"): "col_gelu_save", ("4", "1"): "grad_act", ("1", "1"): "grad_input",
              ("2", "1"): "grad_input_accum", ("1", "2"): "grad_weight", ("2", "2"): "grad_weight_accum",
              ("5", "0"): "swiglu_col", ("6", "0"): "attn_qkv"}
_GSUM_KIND = {"0": "row_sum", "1": "grad_input_sum"}


def _targ(a: str) -> str:
    """A template argument as printed by the demangler: '(tpmlp::Epilogue)1', '1', 'true'."""
    a = a.strip()
    a = re.sub(r"^\([^)]*\)", "", a)
    return {"true": "1", "false": "0"}.get(a, a)


def kernel_sources():
    """The device and host sources of libtpmlp.so (what the counters depend on)."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".h", ".cpp")) and not f.startswith("synth"))


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for path in kernel_sources():
        h.update(os.path.basename(path).encode() + b"\0")
        h.update(open(path, "rb").read())
    return h.hexdigest()


def kernel_kind(name: str):
    """Benchmark kernel kind of a device kernel name, or None."""
    if "shard_reduce_kernel" in name:
        return "shard_reduce"
    if "attention_kernel" in name:
        return "attn_core"
    if "sp_reduce_kernel" in name:
        m = re.search(r"sp_reduce_kernel<([^,>]*)", name)
        return "sp_reduce_fused" if m and _targ(m.group(1)) == "1" else "sp_reduce"
    if "colsum_" in name:
        return "colsum"
    m = re.search(r"gemm_(?:bf16|f32)_kernel<([^>]*)>", name)
    if not m:
        return None
    args = [_targ(a) for a in m.group(1).split(",")]
    if "gemm_bf16_kernel" in name and len(args) >= 9 and args[8] == "1":
        return _GSUM_KIND.get(args[1])
    return _GEMM_KIND.get((args[0], args[1]))


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    name = re.sub(r"\(.*$", "", name)
    name = name.replace("tpmlp::", "")
    return name[:90]


def _one(pattern: str) -> str:
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise FileNotFoundError(pattern)
    return files[0]


def stats_table(trace_dir: str):
    path = _one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        out.append({"name": r["Name"], "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "total_us": float(r["TotalDurationNs"]) / 1e3,
                    "pct": float(r["Percentage"]), "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3})
    return out


def write_stats(trace_dir: str, out_md: str, command: str):
    rows = stats_table(trace_dir)
    lines = ["# Kernel time: `rocprofv3 --kernel-trace --stats`", "",
             "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
             "| kernel | kind | calls | avg (us) | min (us) | max (us) | total (us) | % of GPU time |",
             "|---|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append("| `%s` | %s | %d | %.2f | %.2f | %.2f | %.1f | %.2f |" % (
            short_name(r["name"]), kernel_kind(r["name"]) or "-", r["calls"], r["avg_us"], r["min_us"],
            r["max_us"], r["total_us"], r["pct"]))
    open(out_md, "w").write("\n".join(lines) + "\n")
    return rows


def counter_per_dispatch(pmc_dir: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter."""
    path = _one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    per = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = r["Dispatch_Id"]
        per[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key, v in per.items():
        out[names[key]].append(v)
    return out


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, workload, variant,
                  out_md, commands):
    copy_bytes = int(copy_bytes)
    cf = counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE")
    cw = counter_per_dispatch(copy_write_dir, "WRITE_SIZE")
    # the copy kernel is the only dispatch with counters in those runs
    cf_vals = [v for vals in cf.values() for v in vals]
    cw_vals = [v for vals in cw.values() for v in vals]
    cf_kib = sorted(cf_vals)[len(cf_vals) // 2]
    cw_kib = sorted(cw_vals)[len(cw_vals) // 2]
    f_scale = copy_bytes / cf_kib   # bytes per counter unit
    w_scale = copy_bytes / cw_kib
    fe = counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    wr = counter_per_dispatch(write_dir, "WRITE_SIZE")
    kinds = collections.defaultdict(lambda: {"fetch": [], "write": [], "names": set()})
    for name, vals in fe.items():
        k = kernel_kind(name)
        if k:
            kinds[k]["fetch"] += vals
            kinds[k]["names"].add(short_name(name))
    for name, vals in wr.items():
        k = kernel_kind(name)
        if k:
            kinds[k]["write"] += vals
    sha = kernel_source_sha256()
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        rec = {}
    if rec.get("kernel_source_sha256") != sha:
        rec = {"kernel_source_sha256": sha, "entries": {}}
    lines = ["# HBM traffic per launch: `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`", "",
             "Commands (run from the repository root on one MI355X):", "", "```", commands.strip(), "```", "",
             "Calibration: a plain float32 copy kernel of %d bytes (read %d, write %d) reads FETCH_SIZE = %.0f "
             "and WRITE_SIZE = %.0f per dispatch, so one counter unit is %.1f bytes (fetch) and %.1f bytes "
             "(write)." % (copy_bytes, copy_bytes, copy_bytes, cf_kib, cw_kib, f_scale, w_scale), "",
             "Workload `%s`, variant `%s`; kernel source SHA-256 `%s`." % (workload, variant, sha[:16]), "",
             "| kind | device kernel | dispatches | FETCH_SIZE (median) | WRITE_SIZE (median) | "
             "HBM read (MB) | HBM write (MB) | HBM total per launch (MB) |",
             "|---|---|---:|---:|---:|---:|---:|---:|"]
    for k, d in sorted(kinds.items()):
        if not d["fetch"] or not d["write"]:
            continue
        f = sorted(d["fetch"])[len(d["fetch"]) // 2]
        wv = sorted(d["write"])[len(d["write"]) // 2]
        rb, wb = f * f_scale, wv * w_scale
        lines.append("| %s | `%s` | %d | %.0f | %.0f | %.1f | %.1f | %.1f |" % (
            k, "`, `".join(sorted(d["names"])), len(d["fetch"]), f, wv, rb / 1e6, wb / 1e6, (rb + wb) / 1e6))
        rec["entries"]["%s/%s/%s" % (workload, variant, k)] = {
            "hbm_bytes_per_launch": rb + wb, "read_bytes": rb, "write_bytes": wb,
            "fetch_size_median": f, "write_size_median": wv}
    rec["copy_calibration"] = {"bytes": copy_bytes, "fetch_size": cf_kib, "write_size": cw_kib}
    open(out_md, "w").write("\n".join(lines) + "\n")
    json.dump(rec, open(path, "w"), indent=1, sort_keys=True)


def main(argv):
    if argv and argv[0] == "stats" and len(argv) == 4:
        write_stats(argv[1], argv[2], argv[3])
    elif argv and argv[0] == "traffic" and len(argv) == 10:
        write_traffic(*argv[1:])
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
