"""The benchmark's output line on the GPU: bench.py's main, run in this
process (no child process) on the default workload with short legs, prints
one JSON line with every field of its contract: metric and value, the step
timing, the roofline object of the dominant kernel and the CPU-oracle
baseline."""
import json
import os
import sys

import pytest

from _helpers import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_output_line(capsys):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sys.path.insert(0, ROOT)
    import bench
    say("bench.py contract (gpt2_small, 3 steps)")
    bench.main(["--steps", "3", "--warmup", "1", "--settle-seconds", "0", "--power-seconds", "0.3",
                "--cpu-baseline-seconds", "0.5", "--no-backward", "--no-sp", "--no-swiglu"])
    out = [l for l in capsys.readouterr().out.splitlines() if l.strip()]
    assert len(out) == 1, out
    d = json.loads(out[0])
    assert d["metric"].startswith("TP-shard MLP forward TFLOP/s")
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["n_gpus"] == 1
    assert d["steps"] == 3 and d["warmup"] == 1 and d["vs_baseline"] is None and d["dtype"] == "bf16"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - 4 * 8192 * 768 * 3072 / (d["ms_per_step"] * 1e-3) / 1e12) <= 1e-3 * d["value"] + 1e-3
    assert d["config"]["workload"] == "gpt2_small" and d["config"]["variant"] == "literal"
    assert set(d["variants"]) == {"literal", "fused"}
    sm = d["step_ms"]
    assert sm["n"] == 3 and 0 < sm["min"] <= sm["median"] <= sm["p90"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["peak"] == (8000.0 if r["bound"] == "hbm" else 2516.6)
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9 and r["achieved"] > 0
    assert "traffic" in r and (r["traffic"] is None or r["traffic"] > 0)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["unit"] == "TFLOP/s" and c["sample"]
    assert set(d["kernels"]) == {"col_gelu", "row_partial", "shard_reduce"}
