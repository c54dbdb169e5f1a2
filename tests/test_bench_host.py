"""Host logic of bench.py, no GPU: the rocprofv3 counter summaries it writes and reads
back (HBM traffic, MFMA utilisation), their source-hash check, and the one-GPU rule."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

TRACE_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
              "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
              "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_COLS)
        w.writeheader()
        for r in rows:
            full = {c: 0 for c in TRACE_COLS}
            full.update(r)
            w.writerow(full)


def row(dispatch, kernel, grid, counter, value, t0=0, t1=1000):
    return {"Dispatch_Id": dispatch, "Kernel_Name": kernel, "Grid_Size": grid,
            "Counter_Name": counter, "Counter_Value": value, "Start_Timestamp": t0,
            "End_Timestamp": t1}


def test_traffic_summary_scaled_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "t.json"))
    copy_kib = bench.COPY_BYTES / 1024
    k = "void moe::ffn_skinny_kernel<1, 16, 0>(args)"
    # FETCH_SIZE counts half the copy's bytes (scale 2); WRITE_SIZE all of them (scale 1)
    fetch = [row(1, "__amd_rocclr_copyBuffer", 131072, "FETCH_SIZE", copy_kib / 2),
             row(2, k, 4096, "FETCH_SIZE", 1000.0), row(3, k, 4096, "FETCH_SIZE", 3000.0)]
    wr = [row(1, "__amd_rocclr_copyBuffer", 131072, "WRITE_SIZE", copy_kib),
          row(2, k, 4096, "WRITE_SIZE", 10.0), row(3, k, 4096, "WRITE_SIZE", 30.0)]
    write_csv(tmp_path / "f.csv", fetch)
    write_csv(tmp_path / "w.csv", wr)
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    t = json.load(open(tmp_path / "t.json"))
    assert t["scale"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert t["scale"]["WRITE_SIZE"] == pytest.approx(1.0)
    g = t["kernels"][k]["4096"]
    assert g["launches"] == 2
    assert g["read_bytes"] == pytest.approx(2000.0 * 1024 * 2)   # mean 2000 KiB x 2
    assert g["write_bytes"] == pytest.approx(20.0 * 1024)
    want = 2000.0 * 1024 * 2 + 20.0 * 1024
    assert bench.traffic_for("ffn_skinny_kernel<1, 16, 0>", want * 1.3) == pytest.approx(want)


def test_summaries_are_ignored_once_the_kernels_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "t.json"))
    monkeypatch.setattr(bench, "MFMA_JSON", str(tmp_path / "m.json"))
    k = "void moe::ffn_lds_kernel<0>(args)"
    stale = {"source_sha256": "0" * 64,
             "kernels": {k: {"2756608": {"read_bytes": 1.0, "write_bytes": 1.0, "launches": 1,
                                          "mfma_busy_frac": 0.5}}}}
    for name in ("t.json", "m.json"):
        with open(tmp_path / name, "w") as f:
            json.dump(stale, f)
    assert bench.traffic_for("ffn_lds_kernel<0>", 2.0) is None
    assert bench.mfma_for("ffn_lds_kernel<0>", 2756608) is None
    # the same data under the current sources' hash is used
    stale["source_sha256"] = bench.kernel_source_hash()
    for name in ("t.json", "m.json"):
        with open(tmp_path / name, "w") as f:
            json.dump(stale, f)
    assert bench.traffic_for("ffn_lds_kernel<0>", 2.0) == pytest.approx(2.0)
    assert bench.mfma_for("ffn_lds_kernel<0>", 2756608)["mfma_busy_frac"] == 0.5


def test_traffic_lookup_takes_the_grid_nearest_the_algorithmic_bytes(tmp_path, monkeypatch):
    """One kernel, two launch grids (two workloads): the entry nearest the launch's
    algorithmic bytes is taken, and none when no entry is within a factor of 2."""
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "t.json"))
    k = "void moe::ffn_lds_kernel<0>(args)"
    t = {"source_sha256": bench.kernel_source_hash(),
         "kernels": {k: {"1": {"read_bytes": 1.0, "write_bytes": 1.0},
                         "2": {"read_bytes": 500.0, "write_bytes": 500.0}}}}
    with open(tmp_path / "t.json", "w") as f:
        json.dump(t, f)
    assert bench.traffic_for("ffn_lds_kernel<0>", 900.0) == pytest.approx(1000.0)
    assert bench.traffic_for("ffn_lds_kernel<0>", 1.5) == pytest.approx(2.0)
    assert bench.traffic_for("ffn_lds_kernel<0>", 40.0) is None
    assert bench.traffic_for("ffn_skinny_kernel", 1000.0) is None


def test_mfma_summary_from_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "MFMA_JSON", str(tmp_path / "m.json"))
    k = "void moe::ffn_lds_kernel<0>(args)"
    # 2 ms; 3.2e6 active cycles per XCD (summed over 8) -> 1.6 GHz; half of the SIMD
    # cycles busy; MOPS x 512 = flops
    t0, t1 = 1_000_000, 3_000_000          # ns
    active = 3.2e6 * bench.XCDS
    busy = 0.5 * 3.2e6 * bench.SIMDS
    mops = 1e9
    rows = [row(7, k, 2756608, "GRBM_GUI_ACTIVE", active, t0, t1),
            row(7, k, 2756608, "SQ_VALU_MFMA_BUSY_CYCLES", busy, t0, t1),
            row(7, k, 2756608, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops, t0, t1),
            # a kernel without MFMA work is left out
            row(8, "void moe::combine_kernel<8>(args)", 99, "GRBM_GUI_ACTIVE", 5.0, t0, t1),
            row(8, "void moe::combine_kernel<8>(args)", 99, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0, t0, t1)]
    write_csv(tmp_path / "c.csv", rows)
    bench.write_mfma(str(tmp_path / "c.csv"))
    g = bench.mfma_for("ffn_lds_kernel<0>", 2756608)
    assert g["ms"] == pytest.approx(2.0)
    assert g["clock_ghz"] == pytest.approx(1.6)
    assert g["mfma_busy_frac"] == pytest.approx(0.5)
    assert g["mfma_flops"] == pytest.approx(mops * 512)
    assert g["mfma_tflops"] == pytest.approx(mops * 512 / 2e-3 / 1e12)
    assert bench.mfma_for("combine_kernel<8>", 99) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
