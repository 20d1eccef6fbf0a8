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
    say("bench.py contract (default workload long_seq, 2 steps; gpt2_small config and backward leg)")
    bench.main(["--steps", "2", "--warmup", "1", "--settle-seconds", "0", "--power-seconds", "0.3",
                "--cpu-baseline-seconds", "0.5", "--configs", "gpt2_small", "--legs-workload", "gpt2_small",
                "--no-sp", "--no-swiglu"])
    out = [l for l in capsys.readouterr().out.splitlines() if l.strip()]
    assert len(out) == 1, out
    d = json.loads(out[0])
    assert d["metric"].startswith("TP-shard MLP forward TFLOP/s")
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["n_gpus"] == 1
    assert d["steps"] == 2 and d["warmup"] == 1 and d["vs_baseline"] is None and d["dtype"] == "bf16"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    M, H, F = 32768, 8192, 32768
    assert abs(d["value"] - 4 * M * H * F / (d["ms_per_step"] * 1e-3) / 1e12) <= 1e-3 * d["value"] + 1e-3
    assert d["config"]["workload"] == "long_seq" and d["config"]["variant"] == "fused"
    assert (d["config"]["M"], d["config"]["H"], d["config"]["F"], d["config"]["k"]) == (M, H, F, 8)
    assert set(d["variants"]) == {"literal", "fused"}
    sm = d["step_ms"]
    assert sm["n"] == 2 and 0 < sm["min"] <= sm["median"] <= sm["p90"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["peak"] == (8000.0 if r["bound"] == "hbm" else 2516.6)
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9 and r["achieved"] > 0
    assert "traffic" in r and (r["traffic"] is None or r["traffic"] > 0)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["unit"] == "TFLOP/s" and c["sample"]
    assert c["logical_cpus"] >= 1 and "cpu_model" in c
    assert set(d["kernels"]) == {"col_gelu", "row_sum"}
    assert set(d["configs"]) == {"long_seq", "gpt2_small"}
    for name, cf in d["configs"].items():
        assert cf["value"] > 0 and set(cf["variants"]) == {"literal", "fused"}, name
        assert cf["roofline"]["frac"] > 0 and cf["kernels"], name
    assert d["configs"]["long_seq"]["value"] == d["value"]
    assert d["configs"]["gpt2_small"]["config"]["M"] == 8192
    assert d["backward"]["workload"] == "gpt2_small" and d["backward"]["value"] > 0
    assert d["sequence_parallel"] is None and d["swiglu"] is None
