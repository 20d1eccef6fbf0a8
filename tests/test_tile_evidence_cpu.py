"""Host logic of tensor_transformer_mlp_amd.tile_evidence: dispatches of
rocprofv3 counter runs are matched to (workload, step, tile) by the kernel's
template arguments and grid size, and the table's derived figures (MFMA
busy, flop ratio, clock, HBM bytes) follow from the counters as documented."""
import csv
import json
import os

from tensor_transformer_mlp_amd import tile_evidence as te

HEAD = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
        "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
        "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _kernel(epi, bm, bn, wm, wn, nbuf, gsum):
    return ("void tpmlp::gemm_bf16_kernel<(tpmlp::Epilogue)%d, 0, %d, %d, %d, %d, %d, false, %s>"
            "(tpmlp::GemmParams)" % (epi, bm, bn, wm, wn, nbuf, "true" if gsum else "false"))


def _write(d, rows):
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEAD)
        for i, (did, name, grid, ctr, val, ns) in enumerate(rows):
            w.writerow([i, did, "Agent 1", 1, 1, 1, grid, 7, name, 512, 73728, 0, 64, 0, 48, ctr, val,
                        1000, 1000 + ns])


def test_summary_matches_and_derives(tmp_path):
    # gpt2_small-like shards: M=8192, N=K=768, n=4; tile A = 128x256 (8 waves, 3 stages), tile B =
    # 256x256 (8 waves, 4 stages); the row step and the shard sum share the epilogue argument
    tA = {"bm": 128, "bn": 256, "waves": 8, "stages": 3}
    tB = {"bm": 256, "bn": 256, "waves": 8, "stages": 4}
    recs = []
    for step, t, shape in (("col", 6, tA), ("col", 0, tB), ("row", 6, tA), ("sum", 6, tA)):
        wg = te.workgroups(shape, step, 4, 8192, 768)
        flop = 2.0 * 8192 * 768 * 768 * 4
        recs.append({"workload": "w", "step": step, "tile": t, "picked": t == 6, **shape, "M": 8192, "N": 768,
                     "K": 768, "n": 4, "workgroups": wg, "flop": flop, "ms": 0.05, "tflops": flop / 0.05 / 1e9,
                     "bitwise_equal_to_picked": True})
    assert [r["workgroups"] for r in recs] == [768, 384, 768, 192]
    run = tmp_path / "run.json"
    json.dump({"records": recs, "reps": 3, "launches": 10}, open(run, "w"))
    kA_col, kB_col = _kernel(0, 128, 256, 2, 4, 3, False), _kernel(0, 256, 256, 2, 4, 4, False)
    kA_row, kA_sum = _kernel(1, 128, 256, 2, 4, 3, False), _kernel(1, 128, 256, 2, 4, 3, True)
    flop = recs[0]["flop"]
    ns = 50000
    # MfmaUtil 40 %: busy cycles = 0.40 * 1024 SIMDs * active; active = 2.0 GHz * 50 us = 100000 cycles
    busy = 0.40 * 1024 * 100000
    mf, did = [], 0
    for k, grid in ((kA_col, 768 * 512), (kB_col, 384 * 512), (kA_row, 768 * 512), (kA_sum, 192 * 512)):
        for rep in range(2):
            did += 1
            mf += [(did, k, grid, "MfmaUtil", 40.0, ns), (did, k, grid, "SQ_VALU_MFMA_BUSY_CYCLES", busy, ns),
                   (did, k, grid, "SQ_INSTS_VALU_MFMA_MOPS_BF16", flop / 512, ns)]
    mf.append((did + 1, "void other_kernel<1>", 4096, "MfmaUtil", 99.0, ns))
    _write(str(tmp_path / "mfma"), mf)
    _write(str(tmp_path / "fetch"), [(1, kA_col, 768 * 512, "FETCH_SIZE", 1000.0, ns),
                                     (2, kB_col, 384 * 512, "FETCH_SIZE", 3000.0, ns)])
    _write(str(tmp_path / "write"), [(1, kA_col, 768 * 512, "WRITE_SIZE", 500.0, ns)])
    out = tmp_path / "t.md"
    te.summary(str(run), str(tmp_path / "mfma"), str(tmp_path / "fetch"), str(tmp_path / "write"), str(out),
               "cmd")
    rows = [l for l in open(out).read().splitlines() if l.startswith("| w |")]
    assert len(rows) == 4
    cells = [[c.strip() for c in r.strip("|").split("|")] for r in rows]
    cal = json.load(open(os.path.join(te.ROOT, "profiles", "traffic.json")))["copy_calibration"]
    fs, ws = cal["bytes"] / cal["fetch_size"], cal["bytes"] / cal["write_size"]
    c0 = cells[0]
    assert c0[2] == "6 *" and c0[5] == "768"
    assert c0[9] == "40.0" and c0[10] == "1.000" and c0[11] == "2.00"
    assert c0[12] == "%.1f" % (1000 * fs / 1e6) and c0[13] == "%.1f" % (500 * ws / 1e6)
    assert c0[14] == "%.0f" % ((1000 * fs + 500 * ws) / 0.05e-3 / 1e9)
    assert cells[1][2] == "0" and cells[1][12] == "%.1f" % (3000 * fs / 1e6) and cells[1][13] == "-"
    # the row step and the shard sum are told apart by the group-sum argument and the grid
    assert cells[2][9] == "40.0" and cells[3][9] == "40.0" and cells[2][12] == "-"


def test_template_arguments_parse():
    name = _kernel(3, 128, 256, 2, 4, 3, True)
    assert te._targs(name) == [3, 0, 128, 256, 2, 4, 3, 0, 1]
    assert te._targs("void at::native::foo<int>(int)") is None
