#!/usr/bin/env python3
"""Benchmark of the tensor-parallel MLP shard forward on one MI355X.

One step = one call of tp_mlp_shard_forward: for each of the k shards the
column GEMM + bias + GeLU and the row GEMM, then the on-device shard sum, over
one batch of seeded synthetic inputs already resident in HBM.  The headline
workload is the long-sequence layer (M = 32768, H = 8192, F = 32768, k = 8),
the largest configuration; `value` is its forward throughput in the chosen
variant (fused by default: the shard sum carried through the row GEMM's
accumulator, the unsplit GEMM of the row-split identity; literal: fp32
partials and the shard-reduce kernel), and "variants" gives both.  "configs" holds the same measurement for the other
bf16 workloads (GPT-2-small, 7B and 175B shaped layers).  The backward of the
block (tp_mlp_shard_backward: per shard the training-mode column step, dA, dV,
dW + db and the partial dX, then the dX shard sum), the sequence-parallel
forward (the shard sum as a reduce-scatter over the k sequence blocks with
the residual X added), the SwiGLU block and, with --attention, the causal
tensor-parallel attention block are timed on one workload (--legs-workload,
the 7B-shaped layer by default) under "backward", "sequence_parallel",
"swiglu" and "attention".

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--variant literal|fused]
                    [--configs a,b,...] [--legs-workload NAME]
                    [--no-backward] [--no-sp] [--no-swiglu] [--attention]

Prints ONE JSON line on stdout; diagnostics go to stderr.  `value` and
ms_per_step come from K steps timed back to back between two
synchronisations; "step_ms" gives the median, minimum and 90th percentile of
K further steps timed one by one with HIP events, and "gpu_state" the socket
power and shader clock sampled from sysfs while the step repeats.  "roofline"
is the dominant kernel's (the kind with the largest time per step), timed
with HIP events on the stream it runs on.
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


def warm(step, args):
    """Untimed: the step repeated for args.settle_seconds (the GPU raises its
    clock only after some time under load: the first ~50 gpt2_small steps after
    an idle period run ~12% slower than the steady state), then args.warmup
    more steps."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle_seconds:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()


def step_distribution(step, n: int) -> dict:
    """n more steps, each between its own pair of HIP events on the stream the
    steps launch on, behind a spin kernel that keeps the GPU busy while the
    host enqueues them (so the pairs time the GPU, not the host): median,
    minimum and 90th percentile of one step (ms)."""
    import torch
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    spin = getattr(torch.cuda, "_sleep", None)
    if spin is not None:
        spin(max(3_000_000, 200_000 * n))
    for e0, e1 in ev:
        e0.record(s)
        step()
        e1.record(s)
    torch.cuda.synchronize()
    return percentiles([e0.elapsed_time(e1) for e0, e1 in ev])


def read_hwmon(dev_dir: str) -> dict | None:
    """Socket power and its cap (W) and the shader clock (MHz) from the amdgpu
    hwmon files of one device (dev_dir: its /sys/bus/pci/devices/<address> directory): plain
    file reads, no other program is run.  None if the files are not there."""
    import glob
    for d in sorted(glob.glob(os.path.join(dev_dir, "hwmon", "hwmon*"))):
        out = {}
        for fname, key, scale in (("power1_average", "socket_power_w", 1e-6), ("power1_input", "socket_power_w", 1e-6),
                                  ("power1_cap", "power_cap_w", 1e-6), ("freq1_input", "gfx_clock_mhz", 1e-6)):
            if key in out:
                continue
            try:
                out[key] = float(open(os.path.join(d, fname)).read().strip()) * scale
            except (OSError, ValueError):
                pass
        if "gfx_clock_mhz" not in out:
            clk = current_sclk_mhz(dev_dir)
            if clk is not None:
                out["gfx_clock_mhz"] = clk
        if out:
            return out
    return None


def current_sclk_mhz(dev_dir: str):
    """The shader clock level marked current ('*') in the device's pp_dpm_sclk
    table, in MHz (None if the file is missing or marks none)."""
    import re
    try:
        lines = open(os.path.join(dev_dir, "pp_dpm_sclk")).read().splitlines()
    except OSError:
        return None
    for line in lines:
        m = re.match(r"\s*\w+:\s*([0-9.]+)\s*[Mm][Hh]z\s*\*", line)
        if m:
            return float(m.group(1))
    return None


def gpu_state_during(step, seconds: float):
    """The step repeats on the GPU for `seconds` while a thread samples the
    device's socket power and shader clock from sysfs every 0.1 s; returns
    their means (None where the files are missing)."""
    import threading
    import torch
    if seconds <= 0:
        return None
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    if getattr(props, "pci_bus_id", None) is None:
        return None
    bdf = "%04x:%02x:%02x.0" % (getattr(props, "pci_domain_id", 0), props.pci_bus_id, getattr(props, "pci_device_id", 0))
    dev_dir = "/sys/bus/pci/devices/" + bdf
    if read_hwmon(dev_dir) is None:
        return None
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.wait(0.1):
            r = read_hwmon(dev_dir)
            if r:
                samples.append(r)

    th = threading.Thread(target=sampler)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    out = {"device": bdf, "samples": len(samples)}
    for key in ("socket_power_w", "power_cap_w", "gfx_clock_mhz"):
        vals = [x[key] for x in samples if key in x]
        if vals:
            out[key] = round(sum(vals) / len(vals), 1)
    return out if len(out) > 2 else None


def percentiles(ms) -> dict:
    """Median, minimum and 90th percentile (nearest rank) of a list of times."""
    t = sorted(ms)
    n = len(t)
    med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
    p90 = t[max(0, -(-9 * n // 10) - 1)]
    return {"median": round(med, 5), "min": round(t[0], 5), "p90": round(p90, 5), "n": n}


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--power-seconds", type=float, default=2.0,
                    help="after the timed steps, repeat the step this long while the device's socket power and "
                         "shader clock are sampled from sysfs; 0 disables")
    ap.add_argument("--settle-seconds", type=float, default=0.5,
                    help="before each leg's warmup steps, repeat its step for this long so that the GPU's clock "
                         "has left its idle state (untimed; 0 disables)")
    ap.add_argument("--workload", default="long_seq",
                    help="the headline workload (default: the long-sequence layer, the largest configuration)")
    ap.add_argument("--configs", default="gpt2_small,llama7b,gpt3_175b,long_seq",
                    help="comma-separated workloads whose forward is also measured and reported under "
                         "\"configs\" (empty: none)")
    ap.add_argument("--legs-workload", default="llama7b",
                    help="workload of the backward, sequence-parallel, SwiGLU and attention legs "
                         "(empty: the headline workload)")
    ap.add_argument("--variant", choices=["literal", "fused"], default="fused",
                    help="the variant `value` reports (both are timed and reported under \"variants\"): fused "
                         "carries the shard sum through the row GEMM's accumulator (the unsplit GEMM "
                         "[Y_0 .. Y_k-1] V of the row-split identity), literal materialises the k partials and "
                         "sums them with the shard-reduce kernel")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (0 disables the CPU leg)")
    ap.add_argument("--kernel-steps", type=int, default=None,
                    help="steps of the per-kernel timing pass (default: --steps)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-sp", action="store_true", help="skip the sequence-parallel leg")
    ap.add_argument("--no-swiglu", action="store_true", help="skip the SwiGLU leg")
    ap.add_argument("--attention", action="store_true",
                    help="also time the attention block (off by default: its output projection launches the "
                         "row GEMM kernel at another shape, which would mix into that kernel's profile)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain float32 copy kernel (y = x * 1) over MIB MiB, 5 times: "
                         "the known-size reference for the HBM byte counters")
    return ap.parse_args(argv)


def kernel_bytes(kind, w, elt, n):
    """Algorithmic HBM bytes of one launch of `kind` over n shards (each
    operand read once, each result written once; shared operands once)."""
    M, H, Fk, k = w.M, w.H, w.Fk, w.k
    table = {
        "col_gelu": M * H * elt + n * (H * Fk + Fk + M * Fk) * elt,
        "row_partial": n * ((M * Fk + Fk * H) * elt + M * H * 4),
        "row_sum": n * (M * Fk + Fk * H) * elt + M * H * 4,
        "shard_reduce": (k + 1) * M * H * 4,
        "col_gelu_save": M * H * elt + n * (H * Fk + Fk + 2 * M * Fk) * elt,
        "grad_act": M * H * elt + n * (Fk * H + 2 * M * Fk) * elt,
        "grad_row_weight": M * H * elt + n * (M * Fk * elt + Fk * H * 4),
        "grad_col_weight": M * H * elt + n * (M * Fk * elt + (H * Fk + Fk) * 4),
        "grad_input": n * ((M * Fk + H * Fk) * elt + M * H * 4),
        "grad_input_sum": n * (M * Fk + H * Fk) * elt + M * H * 4,
        # sequence-parallel reduce-scatter + residual: k (or 1) fp32 parts, X, fp32 blocks
        "sp_reduce": (k * 4 + elt + 4) * M * H,
        "sp_reduce_fused": (4 + elt + 4) * M * H,
        # SwiGLU column step: X once, gate and up weights, Y
        "swiglu_col": M * H * elt + n * (2 * H * Fk + M * Fk) * elt,
        # attention block (Hk = H / k per shard): projection, attention, output projection
        "attn_qkv": M * H * elt + n * (3 * H * (H // k) + 3 * (H // k) + 3 * M * (H // k)) * elt,
        "attn_core": n * 4 * M * (H // k) * elt,
        "attn_out": n * ((M * (H // k) + (H // k) * H) * elt + M * H * 4),
    }
    return table[kind]


def kernel_flops(kind, w, n):
    if kind == "shard_reduce":
        return (w.k - 1) * w.M * w.H
    if kind == "sp_reduce":
        return w.k * w.M * w.H
    if kind == "sp_reduce_fused":
        return w.M * w.H
    if kind == "swiglu_col":
        return n * 4 * w.M * w.H * w.Fk
    if kind == "attn_qkv":
        return n * 2 * w.M * w.H * 3 * (w.H // w.k)
    if kind == "attn_core":
        # causal: query t meets t + 1 keys; 2 d flop for the score, 2 d for the sum
        return n * 4 * (w.H // w.k) * w.B * (w.S * (w.S + 1) // 2)
    if kind == "attn_out":
        return n * 2 * w.M * (w.H // w.k) * w.H
    return n * 2 * w.M * w.H * w.Fk


def time_kinds(kinds, launch, nlaunch, nshards, steps, warmup, w, elt):
    """Per-kind timing: each kind's launches of one step run back to back
    between one HIP event pair on the stream they are launched on; a spin
    kernel queued first keeps the GPU busy while the host enqueues, so no host
    gap falls inside a pair.  nshards[kind]: shards per launch.
    Returns {kind: {avg_ms, ms_per_step, flop, bytes, ...}} per launch."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    durs = {kd: [] for kd in kinds}
    spin = getattr(torch.cuda, "_sleep", None)
    for it in range(warmup + steps):
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
        if it >= warmup:
            for kind, a, b in rec:
                durs[kind].append(a.elapsed_time(b) / nlaunch[kind])
    kern = {}
    for kind, d in durs.items():
        if not d:
            continue
        avg = float(np.mean(d))
        n = nshards[kind]
        kern[kind] = {"launches_per_step": nlaunch[kind], "shards_per_launch": n, "avg_ms": avg,
                      "ms_per_step": avg * nlaunch[kind], "flop": kernel_flops(kind, w, n),
                      "bytes": kernel_bytes(kind, w, elt, n)}
        log("  %-16s %2d/step x %2d shards  avg %.4f ms  (%.4f ms/step)  %.1f TFLOP/s  %.0f GB/s" % (
            kind, nlaunch[kind], n, avg, avg * nlaunch[kind], kernel_flops(kind, w, n) / avg / 1e9,
            kernel_bytes(kind, w, elt, n) / avg / 1e6))
    return kern


def roofline(kern, w, variant, dtype, kind=None):
    """Roofline entry of `kind`, by default the kind with the largest share
    of the step."""
    dom = kind or max(kern, key=lambda k_: kern[k_]["ms_per_step"])
    d = kern[dom]
    peak_f = PEAK_TFLOPS[dtype]
    t_mfma = d["flop"] / (peak_f * 1e12)
    t_hbm = d["bytes"] / (PEAK_HBM_GBS * 1e9)
    if not dom.startswith(("shard_reduce", "sp_reduce")) and t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": d["flop"] / (d["avg_ms"] * 1e-3) / 1e12, "peak": peak_f,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": d["bytes"] / (d["avg_ms"] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name, variant, dom)
    roof["kernel"] = dom
    roof["avg_ms"] = d["avg_ms"]
    return roof


def upload_workload(w, dev):
    """Seeded host inputs of workload w, the device tensors of its k shards:
    (host dict, X, [W_i], [b_i], [V_i])."""
    import numpy as np
    import torch
    from tensor_transformer_mlp_amd import inputs
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
    return inp, X, Ws, bs, Vs


def forward_leg(tpm, w, X, Ws, bs, Vs, variant, args, power_seconds, distribution=True):
    """Time tp_mlp_shard_forward on workload w: `variant` (literal: fp32 partials
    and the shard-reduce kernel; fused: the shard sum folded into the row GEMM)
    back to back, the other variant the same way (both results checked against
    each other), the step distribution and the power state, then each kernel
    kind in the step's own launch configuration.  Returns the summary dict."""
    import torch
    dev = X.device
    fused = variant == "fused"
    dt = tpm.TP_BF16 if w.dtype == "bf16" else tpm.TP_F32
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    elt = 2 if w.dtype == "bf16" else 4
    Fk = w.Fk

    def timed(fused_, Z):
        ws = torch.empty(max(tpm.tp_mlp_workspace_bytes(w.k, w.M, w.H, Fk, dt,
                                                        tpm.TP_FUSED_ACCUM if fused_ else 0), 1),
                         dtype=torch.uint8, device=dev)

        def step():
            tpm.tp_mlp_shard_forward(X, Ws, bs, Vs, Z=Z, workspace=ws, fused=fused_)

        warm(step, args)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, step, ws

    Z = torch.empty(w.M, w.H, dtype=torch.float32, device=dev)
    ms, step, ws = timed(fused, Z)
    tflops = w.flop / (ms * 1e-3) / 1e12
    log("%s %s: %d steps, %.4f ms/step, %.1f TFLOP/s (%.1f%% of %s peak)" % (
        w.name, variant, args.steps, ms, tflops, 100 * tflops / PEAK_TFLOPS[w.dtype], w.dtype))
    if not bool(torch.isfinite(Z).all()):
        raise RuntimeError("non-finite output")
    dist = None
    if distribution:
        dist = step_distribution(step, args.steps)
        log("  single steps: median %.4f ms, min %.4f, p90 %.4f" % (dist["median"], dist["min"], dist["p90"]))
    gpu_state = gpu_state_during(step, power_seconds)
    if gpu_state:
        log("  during the steps (sysfs, %d samples): %s W (cap %s W), shader clock %s MHz" % (
            gpu_state["samples"], gpu_state.get("socket_power_w"), gpu_state.get("power_cap_w"),
            gpu_state.get("gfx_clock_mhz")))
    del ws

    # The other variant of the same step, timed the same way.  Both compute
    # Z = sum_i Z_i in float32 in shard order; the fused one accumulates the
    # shards' products in one running sum, so the two agree to within the
    # float32 rounding of that sum (checked here against an element bound).
    other = "literal" if fused else "fused"
    Z2 = torch.empty_like(Z)
    oms, _, ows = timed(not fused, Z2)
    del ows
    check_variants_agree(Z, Z2, w)
    del Z2
    variants = {variant: {"value": round(tflops, 3), "ms_per_step": round(ms, 5)},
                other: {"value": round(w.flop / (oms * 1e-3) / 1e12, 3), "ms_per_step": round(oms, 5)}}
    log("  other variant (%s): %.4f ms/step, %.1f TFLOP/s" % (other, oms, w.flop / (oms * 1e-3) / 1e12))

    # Per-kernel pass: the launches of one step through the batched per-step
    # entry points, in the same launch configuration as the step (the shards
    # run in batches of up to TP_MAX_BATCH, one launch per step and batch).
    ks = args.kernel_steps or args.steps
    G = min(w.k, tpm.TP_MAX_BATCH)
    batches = [(i0, min(G, w.k - i0)) for i0 in range(0, w.k, G)]
    Yb = [torch.empty(w.M, Fk, dtype=tdt, device=dev) for _ in range(G)]
    parts = [Z] + ([] if fused else [torch.empty(w.M, w.H, dtype=torch.float32, device=dev)
                                     for _ in range(w.k - 1)])
    if fused:
        kinds = ["col_gelu", "row_sum"]
    else:
        kinds = ["col_gelu", "row_partial"] + (["shard_reduce"] if w.k > 1 else [])
    nlaunch = {"col_gelu": len(batches), "row_partial": len(batches), "row_sum": len(batches),
               "shard_reduce": 1}
    nshards = {"col_gelu": G, "row_partial": G, "row_sum": G, "shard_reduce": w.k}

    def launch(kind):
        for i0, n in batches:
            if kind == "col_gelu":
                tpm.tp_mlp_col_gelu_shards(X, Ws[i0:i0 + n], bs[i0:i0 + n], Yb[:n])
            elif kind == "row_partial":
                tpm.tp_mlp_row_partial_shards(Yb[:n], Vs[i0:i0 + n], parts[i0:i0 + n])
            elif kind == "row_sum":
                tpm.tp_mlp_row_partial_shards(Yb[:n], Vs[i0:i0 + n], [Z], sum_shards=True, accumulate=i0 > 0)
        if kind == "shard_reduce":
            tpm.tp_shard_reduce(parts, Z=Z)

    kern = time_kinds(kinds, launch, nlaunch, nshards, ks, args.warmup, w, elt)
    roof = roofline(kern, w, variant, w.dtype)
    del Yb, parts, Z
    out = {"workload": w.name, "variant": variant, "value": round(tflops, 3), "unit": "TFLOP/s",
           "ms_per_step": round(ms, 5), "pct_of_peak": round(100 * tflops / PEAK_TFLOPS[w.dtype], 2),
           "flop_per_step": w.flop, "variants": variants, "roofline": roof,
           "kernels": {k_: {"avg_ms": round(v["avg_ms"], 5), "per_step": v["launches_per_step"],
                            "shards_per_launch": v["shards_per_launch"]} for k_, v in kern.items()},
           "gpu_state": gpu_state}
    if dist is not None:
        out["step_ms"] = dist
    return out


def check_variants_agree(Z, Z2, w):
    """The literal and fused Z both hold the float32 sum over the shards of
    the shards' products and differ only in where that sum is rounded: their
    relative Frobenius difference stays at float32 rounding level (<= 1e-5).
    A sanity check of the timed outputs; parity with the oracle is the
    tests' job."""
    import torch
    den = float(torch.linalg.vector_norm(Z.double()))
    diff = float(torch.linalg.vector_norm((Z.double() - Z2.double())))
    if not bool(torch.isfinite(Z2).all()) or diff > 1e-5 * den:
        raise RuntimeError("literal and fused forward differ by %.3g (relative) on %s" % (diff / den, w.name))


def host_cpu() -> dict:
    """Model name and logical CPU count of the host, from /proc/cpuinfo."""
    model, n = None, 0
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("processor"):
                n += 1
            elif model is None and line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": n or os.cpu_count()}


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        log("bench.py measures one GPU only: the library has no multi-GPU path "
            "(the k shards run back to back on one device); run with --gpus 1")
        sys.exit(2)

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

    log("workload %s: M=%d H=%d F=%d k=%d dtype=%s variant=%s" % (w.name, w.M, w.H, w.F, w.k, w.dtype,
                                                                 args.variant))
    t = time.time()
    inp, X, Ws, bs, Vs = upload_workload(w, dev)
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.time() - t))
    head = forward_leg(tpm, w, X, Ws, bs, Vs, args.variant, args, args.power_seconds)
    del X, Ws, bs, Vs
    torch.cuda.empty_cache()

    # The other bf16 workloads' forward, the same measurement (one line holds
    # every configuration).
    configs = {w.name: {k_: head[k_] for k_ in ("value", "ms_per_step", "pct_of_peak", "variants", "roofline",
                                                 "kernels", "gpu_state")}}
    for name in [c for c in args.configs.split(",") if c and c != w.name]:
        cw = inputs.WORKLOADS[name]
        t = time.time()
        _, cX, cWs, cbs, cVs = upload_workload(cw, dev)
        log("workload %s: inputs ready in %.1f s" % (name, time.time() - t))
        r = forward_leg(tpm, cw, cX, cWs, cbs, cVs, args.variant, args, min(args.power_seconds, 1.0),
                        distribution=False)
        configs[name] = {k_: r[k_] for k_ in ("value", "ms_per_step", "pct_of_peak", "variants", "roofline",
                                               "kernels", "gpu_state")}
        configs[name]["config"] = cw.describe()
        del cX, cWs, cbs, cVs
        torch.cuda.empty_cache()

    # Training and variant legs, on one workload (default: the 7B-shaped layer).
    lw = inputs.WORKLOADS[args.legs_workload or w.name]
    bwd = sp = swiglu = attn = None
    if not (args.no_backward and args.no_sp and args.no_swiglu and not args.attention):
        _, lX, lWs, lbs, lVs = upload_workload(lw, dev)
        fused = args.variant == "fused"
        elt = 2 if lw.dtype == "bf16" else 4
        tdt = torch.bfloat16 if lw.dtype == "bf16" else torch.float32
        if not args.no_backward:
            bwd = bench_backward(tpm, lw, lX, lWs, lbs, lVs, fused, args, elt, tdt)
        if not args.no_sp and lw.M % lw.k == 0:
            sp = bench_sp(tpm, lw, lX, lWs, lbs, lVs, fused, args, elt, tdt)
        del lWs, lbs
        if not args.no_swiglu:
            swiglu = bench_swiglu(tpm, lw, lX, lVs, fused, args, elt, tdt)
        del lVs
        if args.attention and lw.dtype == "bf16":
            attn = bench_attention(tpm, lw, lX, fused, args, elt)
        del lX
        torch.cuda.empty_cache()
        for leg in (bwd, sp, swiglu, attn):
            if leg is not None:
                leg["workload"] = lw.name

    cpu = None
    if args.cpu_baseline_seconds > 0:
        cpu = cpu_baseline(w, inp, args.cpu_baseline_seconds)

    out = {
        "metric": METRIC, "value": head["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded Philox normals, random-init weights)",
        "pct_of_peak": head["pct_of_peak"], "step_ms": head["step_ms"], "gpu_state": head["gpu_state"],
        "config": dict(w.describe(), variant=args.variant, parallelism="tp%d shards on 1 GPU" % w.k),
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "variants": head["variants"],
        "cpu_baseline": cpu,
        "configs": configs,
        "backward": bwd,
        "sequence_parallel": sp,
        "swiglu": swiglu,
        "attention": attn,
    }
    print(json.dumps(out), flush=True)


def bench_backward(tpm, w, X, Ws, bs, Vs, fused, args, elt, tdt):
    """Time tp_mlp_shard_backward (recomputing Y_i and G_i from X) and its
    kernels by kind.  FLOPs counted: 5 GEMMs of 2 M H Fk per shard (the
    recompute, dA, dV, dW, dX)."""
    import numpy as np
    import torch
    from tensor_transformer_mlp_amd import inputs
    dev = X.device
    Fk, k, M, H = w.Fk, w.k, w.M, w.H
    dZ_h = inputs.draw(inputs.STREAM_DZ, (M, H), 1.0, w.dtype)
    dZ = torch.from_numpy(dZ_h.view(np.int16) if dZ_h.dtype == np.uint16 else dZ_h).to(dev)
    if dZ_h.dtype == np.uint16:
        dZ = dZ.view(torch.bfloat16)
    dX = torch.empty(M, H, dtype=torch.float32, device=dev)
    dW = [torch.empty(H, Fk, dtype=torch.float32, device=dev) for _ in range(k)]
    db = [torch.empty(Fk, dtype=torch.float32, device=dev) for _ in range(k)]
    dV = [torch.empty(Fk, H, dtype=torch.float32, device=dev) for _ in range(k)]
    dt = tpm.TP_BF16 if w.dtype == "bf16" else tpm.TP_F32
    flags = tpm.TP_FUSED_ACCUM if fused else 0
    need = tpm.tp_mlp_backward_workspace_bytes(k, M, H, Fk, dt, flags)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step():
        tpm.tp_mlp_shard_backward(X, Ws, bs, Vs, dZ, dX=dX, dW=dW, db=db, dV=dV, workspace=ws, fused=fused)

    warm(step, args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flop = 10 * M * H * w.F
    tflops = flop / (ms * 1e-3) / 1e12
    log("backward: %.4f ms/step, %.1f TFLOP/s (%.1f%% of %s peak)" % (ms, tflops, 100 * tflops / PEAK_TFLOPS[w.dtype],
                                                                    w.dtype))
    if not bool(torch.isfinite(dX).all()):
        raise RuntimeError("non-finite backward output")

    Gn = min(k, tpm.TP_MAX_BATCH)
    batches = [(i0, min(Gn, k - i0)) for i0 in range(0, k, Gn)]
    Y = [torch.empty(M, Fk, dtype=tdt, device=dev) for _ in range(Gn)]
    Gb = [torch.empty(M, Fk, dtype=tdt, device=dev) for _ in range(Gn)]
    parts = [dX] + [torch.empty(M, H, dtype=torch.float32, device=dev) for _ in range(k - 1)]
    gws = torch.empty(max(tpm.tp_mlp_grad_weight_workspace_bytes_shards(Gn, M, H, Fk, dt), 1), dtype=torch.uint8,
                      device=dev)
    kinds = ["col_gelu_save", "grad_act", "grad_row_weight", "grad_col_weight"] + \
        (["grad_input_sum"] if fused else ["grad_input"] + (["shard_reduce"] if k > 1 else []))
    nb = len(batches)
    nlaunch = {"col_gelu_save": nb, "grad_act": nb, "grad_row_weight": nb, "grad_col_weight": nb,
               "grad_input": nb, "grad_input_sum": nb, "shard_reduce": 1}
    nshards = {kd: Gn for kd in nlaunch}
    nshards["shard_reduce"] = k

    def launch(kind):
        for i0, n in batches:
            sl = slice(i0, i0 + n)
            if kind == "col_gelu_save":
                tpm.tp_mlp_col_gelu_shards(X, Ws[sl], bs[sl], Y[:n], Gb[:n])
            elif kind == "grad_act":
                tpm.tp_mlp_grad_act_shards(dZ, Vs[sl], Gb[:n], Gb[:n])
            elif kind == "grad_row_weight":
                tpm.tp_mlp_grad_row_weight_shards(Y[:n], dZ, dV[sl], workspace=gws)
            elif kind == "grad_col_weight":
                tpm.tp_mlp_grad_col_weight_shards(X, Gb[:n], dW[sl], db[sl], workspace=gws)
            elif kind == "grad_input":
                tpm.tp_mlp_grad_input_shards(Gb[:n], Ws[sl], parts[sl])
            elif kind == "grad_input_sum":
                tpm.tp_mlp_grad_input_shards(Gb[:n], Ws[sl], [dX], sum_shards=True, accumulate=i0 > 0)
        if kind == "shard_reduce":
            tpm.tp_shard_reduce(parts, Z=dX)

    kern = time_kinds(kinds, launch, nlaunch, nshards, args.kernel_steps or args.steps, args.warmup, w, elt)
    roof = roofline(kern, w, args.variant, w.dtype)
    return {"metric": "TP-shard MLP backward TFLOP/s (5 GEMMs of 2 M H F/k per shard, incl. recompute)",
            "value": round(tflops, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
            "pct_of_peak": round(100 * tflops / PEAK_TFLOPS[w.dtype], 2), "roofline": roof,
            "kernels": {k_: {"avg_ms": round(v["avg_ms"], 5), "per_step": v["launches_per_step"],
                             "shards_per_launch": v["shards_per_launch"]} for k_, v in kern.items()}}


def bench_sp(tpm, w, X, Ws, bs, Vs, fused, args, elt, tdt):
    """Time tp_mlp_shard_forward_sp (the forward whose all-reduce is a
    reduce-scatter over the k sequence blocks, with X as the residual; fp32
    blocks side by side) and its kernels by kind.  FLOPs counted: those of
    the forward (4 M H F); the roofline entry is the reduce-scatter's."""
    import torch
    dev = X.device
    Fk, k, M, H = w.Fk, w.k, w.M, w.H
    dt = tpm.TP_BF16 if w.dtype == "bf16" else tpm.TP_F32
    flags = tpm.TP_FUSED_ACCUM if fused else 0
    need = tpm.tp_mlp_sp_workspace_bytes(k, M, H, Fk, dt, flags)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    O = torch.empty(M, H, dtype=torch.float32, device=dev)

    def step():
        tpm.tp_mlp_shard_forward_sp(X, Ws, bs, Vs, O=O, workspace=ws, fused=fused)

    warm(step, args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    tflops = w.flop / (ms * 1e-3) / 1e12
    log("sequence-parallel forward: %.4f ms/step, %.1f TFLOP/s" % (ms, tflops))
    if not bool(torch.isfinite(O).all()):
        raise RuntimeError("non-finite sequence-parallel output")

    G = min(k, tpm.TP_MAX_BATCH)
    batches = [(i0, min(G, k - i0)) for i0 in range(0, k, G)]
    Yb = [torch.empty(M, Fk, dtype=tdt, device=dev) for _ in range(G)]
    parts = [torch.empty(M, H, dtype=torch.float32, device=dev) for _ in range(1 if fused else k)]
    red = "sp_reduce_fused" if fused else "sp_reduce"
    kinds = ["col_gelu", "row_sum" if fused else "row_partial", red]
    nlaunch = {"col_gelu": len(batches), "row_partial": len(batches), "row_sum": len(batches), red: 1}
    nshards = {"col_gelu": G, "row_partial": G, "row_sum": G, red: k}

    def launch(kind):
        for i0, n in batches:
            if kind == "col_gelu":
                tpm.tp_mlp_col_gelu_shards(X, Ws[i0:i0 + n], bs[i0:i0 + n], Yb[:n])
            elif kind == "row_partial":
                tpm.tp_mlp_row_partial_shards(Yb[:n], Vs[i0:i0 + n], parts[i0:i0 + n])
            elif kind == "row_sum":
                tpm.tp_mlp_row_partial_shards(Yb[:n], Vs[i0:i0 + n], parts[:1], sum_shards=True,
                                              accumulate=i0 > 0)
        if kind == red:
            tpm.tp_sp_reduce_scatter(parts, k, R=X, O=O)

    kern = time_kinds(kinds, launch, nlaunch, nshards, args.kernel_steps or args.steps, args.warmup, w, elt)
    roof = roofline(kern, w, args.variant, w.dtype, kind=red)
    return {"metric": "TP-shard MLP forward under sequence parallelism (reduce-scatter + residual) TFLOP/s",
            "value": round(tflops, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
            "pct_of_peak": round(100 * tflops / PEAK_TFLOPS[w.dtype], 2), "roofline": roof,
            "kernels": {k_: {"avg_ms": round(v["avg_ms"], 5), "per_step": v["launches_per_step"],
                             "shards_per_launch": v["shards_per_launch"]} for k_, v in kern.items()}}


def bench_swiglu(tpm, w, X, Vs, fused, args, elt, tdt):
    """Time tp_swiglu_shard_forward (the SwiGLU block: per shard one GEMM with
    the gate and up weights and the SiLU(gate) * up epilogue, the row GEMM,
    then the shard sum) on the same X and V with gate and up weights drawn for
    the workload, and its kernels by kind.  FLOPs counted: 3 GEMMs of
    2 M H F/k per shard (6 M H F); the roofline entry is the SwiGLU column
    GEMM's."""
    import numpy as np
    import torch
    from tensor_transformer_mlp_amd import inputs
    dev = X.device
    Fk, k, M, H = w.Fk, w.k, w.M, w.H

    def up(a):
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

    Wg = [up(x) for x in inputs.col_slices(inputs.draw(inputs.STREAM_W, (H, w.F), w.std, w.dtype), k)]
    Wu = [up(x) for x in inputs.col_slices(inputs.draw(inputs.STREAM_WU, (H, w.F), w.std, w.dtype), k)]
    dt = tpm.TP_BF16 if w.dtype == "bf16" else tpm.TP_F32
    flags = tpm.TP_FUSED_ACCUM if fused else 0
    ws = torch.empty(max(tpm.tp_mlp_workspace_bytes(k, M, H, Fk, dt, flags), 1), dtype=torch.uint8, device=dev)
    Z = torch.empty(M, H, dtype=torch.float32, device=dev)

    def step():
        tpm.tp_swiglu_shard_forward(X, Wg, Wu, Vs, Z=Z, workspace=ws, fused=fused)

    warm(step, args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flop = 6 * M * H * w.F
    tflops = flop / (ms * 1e-3) / 1e12
    log("swiglu forward: %.4f ms/step, %.1f TFLOP/s (%.1f%% of %s peak)" % (
        ms, tflops, 100 * tflops / PEAK_TFLOPS[w.dtype], w.dtype))
    if not bool(torch.isfinite(Z).all()):
        raise RuntimeError("non-finite SwiGLU output")

    G = min(k, tpm.TP_MAX_BATCH)
    batches = [(i0, min(G, k - i0)) for i0 in range(0, k, G)]
    Yb = [torch.empty(M, Fk, dtype=tdt, device=dev) for _ in range(G)]
    parts = [Z] + [torch.empty(M, H, dtype=torch.float32, device=dev) for _ in range(k - 1)]
    kinds = ["swiglu_col"] + (["row_sum"] if fused else ["row_partial"] + (["shard_reduce"] if k > 1 else []))
    nlaunch = {"swiglu_col": len(batches), "row_partial": len(batches), "row_sum": len(batches), "shard_reduce": 1}
    nshards = {"swiglu_col": G, "row_partial": G, "row_sum": G, "shard_reduce": k}

    def launch(kind):
        for i0, n in batches:
            if kind == "swiglu_col":
                tpm.tp_swiglu_col_shards(X, Wg[i0:i0 + n], Wu[i0:i0 + n], Yb[:n])
            elif kind == "row_partial":
                tpm.tp_mlp_row_partial_shards(Yb[:n], Vs[i0:i0 + n], parts[i0:i0 + n])
            elif kind == "row_sum":
                tpm.tp_mlp_row_partial_shards(Yb[:n], Vs[i0:i0 + n], [Z], sum_shards=True, accumulate=i0 > 0)
        if kind == "shard_reduce":
            tpm.tp_shard_reduce(parts, Z=Z)

    kern = time_kinds(kinds, launch, nlaunch, nshards, args.kernel_steps or args.steps, args.warmup, w, elt)
    roof = roofline(kern, w, args.variant, w.dtype, kind="swiglu_col")
    return {"metric": "TP-shard SwiGLU MLP forward TFLOP/s (3 GEMMs of 2 M H F/k per shard)",
            "value": round(tflops, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
            "pct_of_peak": round(100 * tflops / PEAK_TFLOPS[w.dtype], 2), "roofline": roof,
            "kernels": {k_: {"avg_ms": round(v["avg_ms"], 5), "per_step": v["launches_per_step"],
                             "shards_per_launch": v["shards_per_launch"]} for k_, v in kern.items()}}


def bench_attention(tpm, w, X, fused, args, elt):
    """Time tp_attn_shard_forward (the causal tensor-parallel attention block of
    the workload's width, heads and sequences: per shard the projection of its
    heads, their attention and the output projection, then the shard sum) on
    the same X with attention weights drawn for it, and its kernels by kind.
    FLOPs counted: the three GEMMs (8 M H^2) and the unmasked half of the
    attention (4 H B S(S+1)/2); the roofline entry is the attention kernel's."""
    import numpy as np
    import torch
    from tensor_transformer_mlp_amd import inputs
    dev = X.device
    k, M, H, nh = w.k, w.M, w.H, w.heads
    Hk, d, hk = H // k, H // nh, nh // k

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    inp = inputs.make_attention(w)
    Wqkv_h, bqkv_h = inputs.qkv_shards(inp["Wq"], inp["Wk"], inp["Wv"], inp["bq"], inp["bk"], inp["bv"], nh, k)
    Wqkv = [up(x) for x in Wqkv_h]
    bqkv = [up(x) for x in bqkv_h]
    Wo = [up(np.ascontiguousarray(inp["Wo"][i * Hk:(i + 1) * Hk])) for i in range(k)]
    del inp, Wqkv_h, bqkv_h
    flags = (tpm.TP_FUSED_ACCUM if fused else 0) | tpm.TP_CAUSAL
    ws = torch.empty(max(tpm.tp_attn_workspace_bytes(k, w.B, w.S, H, nh, tpm.TP_BF16, flags), 1),
                     dtype=torch.uint8, device=dev)
    Z = torch.empty(M, H, dtype=torch.float32, device=dev)

    def step():
        tpm.tp_attn_shard_forward(X, Wqkv, bqkv, Wo, w.B, w.S, nh, Z=Z, workspace=ws, fused=fused, causal=True)

    warm(step, args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flop = 8 * M * H * H + 4 * H * w.B * (w.S * (w.S + 1) // 2)
    tflops = flop / (ms * 1e-3) / 1e12
    log("attention forward (%d heads of %d, causal): %.4f ms/step, %.1f TFLOP/s (%.1f%% of bf16 peak)" % (
        nh, d, ms, tflops, 100 * tflops / PEAK_TFLOPS["bf16"]))
    if not bool(torch.isfinite(Z).all()):
        raise RuntimeError("non-finite attention output")

    # The other variant of the same step, timed the same way.
    oflags = (0 if fused else tpm.TP_FUSED_ACCUM) | tpm.TP_CAUSAL
    ows = torch.empty(max(tpm.tp_attn_workspace_bytes(k, w.B, w.S, H, nh, tpm.TP_BF16, oflags), 1),
                      dtype=torch.uint8, device=dev)
    Z2 = torch.empty_like(Z)

    def ostep():
        tpm.tp_attn_shard_forward(X, Wqkv, bqkv, Wo, w.B, w.S, nh, Z=Z2, workspace=ows, fused=not fused,
                                  causal=True)

    warm(ostep, args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ostep()
    torch.cuda.synchronize()
    oms = (time.perf_counter() - t0) * 1e3 / args.steps
    check_variants_agree(Z, Z2, w)
    variants = {args.variant: {"value": round(tflops, 3), "ms_per_step": round(ms, 5)},
                ("literal" if fused else "fused"): {"value": round(flop / (oms * 1e-3) / 1e12, 3),
                                                    "ms_per_step": round(oms, 5)}}
    log("  other variant (%s): %.4f ms/step, %.1f TFLOP/s" % ("literal" if fused else "fused", oms,
                                                            flop / (oms * 1e-3) / 1e12))
    del ows, Z2

    G = min(k, tpm.TP_MAX_BATCH)
    batches = [(i0, min(G, k - i0)) for i0 in range(0, k, G)]
    QKV = [torch.empty(M, 3 * Hk, dtype=torch.bfloat16, device=dev) for _ in range(G)]
    A = [torch.empty(M, Hk, dtype=torch.bfloat16, device=dev) for _ in range(G)]
    parts = [Z] + [torch.empty(M, H, dtype=torch.float32, device=dev) for _ in range(k - 1)]
    kinds = ["attn_qkv", "attn_core", "attn_out"] + (["shard_reduce"] if k > 1 and not fused else [])
    nlaunch = {"attn_qkv": len(batches), "attn_core": len(batches), "attn_out": len(batches), "shard_reduce": 1}
    nshards = {"attn_qkv": G, "attn_core": G, "attn_out": G, "shard_reduce": k}

    def launch(kind):
        for i0, n in batches:
            if kind == "attn_qkv":
                tpm.tp_attn_qkv_shards(X, Wqkv[i0:i0 + n], bqkv[i0:i0 + n], QKV[:n])
            elif kind == "attn_core":
                tpm.tp_attn_core_shards(QKV[:n], A[:n], w.B, w.S, hk, d, causal=True)
            elif kind == "attn_out":
                if fused:
                    tpm.tp_mlp_row_partial_shards(A[:n], Wo[i0:i0 + n], [Z], sum_shards=True, accumulate=i0 > 0)
                else:
                    tpm.tp_mlp_row_partial_shards(A[:n], Wo[i0:i0 + n], parts[i0:i0 + n])
        if kind == "shard_reduce":
            tpm.tp_shard_reduce(parts, Z=Z)

    kern = time_kinds(kinds, launch, nlaunch, nshards, args.kernel_steps or args.steps, args.warmup, w, elt)
    roof = roofline(kern, w, args.variant, "bf16", kind="attn_core")
    return {"metric": "TP-shard attention block forward TFLOP/s (causal; 3 projections + attention)",
            "value": round(tflops, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
            "pct_of_peak": round(100 * tflops / PEAK_TFLOPS["bf16"], 2), "heads": nh, "head_dim": d,
            "variants": variants, "roofline": roof,
            "kernels": {k_: {"avg_ms": round(v["avg_ms"], 5), "per_step": v["launches_per_step"],
                             "shards_per_launch": v["shards_per_launch"]} for k_, v in kern.items()}}


def measured_traffic(workload, variant, kind):
    """HBM bytes per launch of `kind` from the committed counter summary
    (profiles/traffic.json), or None if that summary does not cover this
    kernel or was taken on a different kernel source."""
    from tensor_transformer_mlp_amd.profiling import kernel_source_sha256
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
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

    W64, b64, V64 = oracle.widen(inp["W"]), oracle.widen(inp["b"]), oracle.widen(inp["V"])
    probe = min(w.M, 32)
    t = time.perf_counter()
    oracle.forward_rows(oracle.widen(inp["X"][:probe]), W64, b64, V64, w.k)
    tp = time.perf_counter() - t
    rows = int(min(w.M, max(probe, probe * target_s / max(tp, 1e-6))))
    X64 = oracle.widen(inp["X"][:rows])
    passes, dt = 0, 0.0
    while passes == 0 or (rows == w.M and dt < target_s and passes < 100):
        t = time.perf_counter()
        oracle.forward_rows(X64, W64, b64, V64, w.k)
        dt += time.perf_counter() - t
        passes += 1
    flop = 4 * rows * w.H * w.F * passes
    val = flop / dt / 1e12
    what = ("%d full passes over all %d rows" % (passes, w.M)) if rows == w.M else \
        ("rows 0..%d of %d" % (rows - 1, w.M))
    log("cpu oracle: %s in %.2f s with %d threads: %.4f TFLOP/s" % (what, dt, oracle.max_threads(), val))
    return dict({"value": val, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
                 "sample": "%s of the %s workload (all %d shards, full W and V), fp64, %.1f s" % (
                     what, w.name, w.k, dt)}, **host_cpu())


if __name__ == "__main__":
    main()
