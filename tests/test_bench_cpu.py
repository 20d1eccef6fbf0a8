"""Host logic of bench.py (no GPU): the one-GPU refusal, the per-step
percentiles, the algorithmic bytes and flops of each kernel kind against
their closed forms at the gpt2_small shapes, the roofline classification (left or right of the bf16
ridge, 2516.6 TFLOP/s over 8 TB/s = 315 flop/byte), and the guard that drops
the measured HBM traffic once the kernel source differs from the one the
counters were taken on."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as b
    return b


@pytest.fixture(scope="module")
def gpt2():
    from tensor_transformer_mlp_amd import inputs
    return inputs.WORKLOADS["gpt2_small"]


def test_more_than_one_gpu_is_refused(bench, capsys):
    """Run in this process: the refusal comes before anything touches the GPU."""
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code == 2
    out = capsys.readouterr()
    assert "one GPU" in out.err and out.out == ""


def test_kernel_bytes_and_flops_closed_forms(bench, gpt2):
    M, H, Fk, k = 8192, 768, 768, 4
    assert (gpt2.M, gpt2.H, gpt2.Fk, gpt2.k) == (M, H, Fk, k)
    # row step of all 4 shards: Y_i and V_i read once each, fp32 Z_i written once each
    assert bench.kernel_bytes("row_partial", gpt2, 2, k) == k * ((M * Fk + Fk * H) * 2 + M * H * 4) == 155_713_536
    # column step: X once (shared), W_i, b_i, Y_i per shard
    assert bench.kernel_bytes("col_gelu", gpt2, 2, k) == M * H * 2 + k * (H * Fk + Fk + M * Fk) * 2
    # reduce: k partials read, Z written
    assert bench.kernel_bytes("shard_reduce", gpt2, 2, k) == (k + 1) * M * H * 4
    # the two GEMM steps hold all of the block's 4 M H F flop
    total = bench.kernel_flops("col_gelu", gpt2, k) + bench.kernel_flops("row_partial", gpt2, k)
    assert total == 4 * M * H * gpt2.F == gpt2.flop
    assert bench.kernel_flops("shard_reduce", gpt2, k) == (k - 1) * M * H
    assert bench.kernel_flops("swiglu_col", gpt2, k) == 2 * bench.kernel_flops("col_gelu", gpt2, k)


def _kern(bench, w, kind, avg_ms):
    return {kind: {"ms_per_step": avg_ms, "avg_ms": avg_ms, "flop": bench.kernel_flops(kind, w, w.k),
                   "bytes": bench.kernel_bytes(kind, w, 2, w.k)}}


def test_roofline_sides_of_the_ridge(bench, gpt2, monkeypatch):
    monkeypatch.setattr(bench, "measured_traffic", lambda *a: None)
    # row step: 38.7 GFLOP over 155.7 MB = 248 flop/byte < 315: priced against HBM
    r = bench.roofline(_kern(bench, gpt2, "row_partial", 0.05), gpt2, "literal", "bf16")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(155_713_536 / 0.05e-3 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    # column step: 38.7 GFLOP over 67.6 MB, right of the ridge: priced against the MFMA peak
    r = bench.roofline(_kern(bench, gpt2, "col_gelu", 0.05), gpt2, "literal", "bf16")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
    assert r["achieved"] == pytest.approx(bench.kernel_flops("col_gelu", gpt2, 4) / 0.05e-3 / 1e12)
    # the dominant kind is the one with the largest time per step
    kern = {**_kern(bench, gpt2, "col_gelu", 0.04), **_kern(bench, gpt2, "row_partial", 0.05),
            **_kern(bench, gpt2, "shard_reduce", 0.02)}
    assert bench.roofline(kern, gpt2, "literal", "bf16")["kernel"] == "row_partial"
    assert bench.roofline(kern, gpt2, "literal", "bf16", kind="shard_reduce")["bound"] == "hbm"


def test_traffic_is_dropped_when_the_kernel_source_changed(bench, monkeypatch):
    import tensor_transformer_mlp_amd.profiling as prof
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path))
    key = next(iter(rec["entries"]))
    workload, variant, kind = key.split("/")
    monkeypatch.setattr(prof, "kernel_source_sha256", lambda: rec["kernel_source_sha256"])
    assert bench.measured_traffic(workload, variant, kind) == rec["entries"][key]["hbm_bytes_per_launch"]
    assert bench.measured_traffic(workload, variant, "no_such_kind") is None
    monkeypatch.setattr(prof, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.measured_traffic(workload, variant, kind) is None


def test_step_percentiles(bench):
    # median of an even count is the mean of the middle two; p90 is the
    # nearest-rank 90th percentile (the ceil(0.9 n)-th smallest)
    assert bench.percentiles([5.0, 1.0, 2.0, 3.0, 4.0]) == {"median": 3.0, "min": 1.0, "p90": 5.0, "n": 5}
    assert bench.percentiles([float(i) for i in range(10, 0, -1)]) == {"median": 5.5, "min": 1.0, "p90": 9.0,
                                                                          "n": 10}
    t = [0.1] * 95 + [0.5] * 5
    assert bench.percentiles(t)["p90"] == 0.1 and bench.percentiles(t)["median"] == 0.1
    assert bench.percentiles([0.25]) == {"median": 0.25, "min": 0.25, "p90": 0.25, "n": 1}


def test_hwmon_read(bench, tmp_path):
    d = tmp_path / "hwmon" / "hwmon3"
    d.mkdir(parents=True)
    (d / "power1_average").write_text("1258000000\n")
    (d / "freq1_input").write_text("1986000000\n")
    assert bench.read_hwmon(str(tmp_path)) == {"socket_power_w": 1258.0, "gfx_clock_mhz": 1986.0}
    (d / "power1_cap").write_text("1400000000\n")
    assert bench.read_hwmon(str(tmp_path))["power_cap_w"] == 1400.0
    (d / "power1_cap").unlink()
    (d / "power1_average").unlink()
    (d / "power1_input").write_text("700000000\n")
    assert bench.read_hwmon(str(tmp_path)) == {"socket_power_w": 700.0, "gfx_clock_mhz": 1986.0}
    assert bench.read_hwmon(str(tmp_path / "missing")) is None
    # no freq1_input: the current level of pp_dpm_sclk
    (d / "freq1_input").unlink()
    (tmp_path / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1933Mhz *\n2: 2400Mhz\n")
    assert bench.read_hwmon(str(tmp_path)) == {"socket_power_w": 700.0, "gfx_clock_mhz": 1933.0}
    (tmp_path / "pp_dpm_sclk").write_text("S: 1986Mhz *\n")
    assert bench.current_sclk_mhz(str(tmp_path)) == 1986.0
    (tmp_path / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.current_sclk_mhz(str(tmp_path)) is None
