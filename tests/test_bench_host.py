"""Host-side pieces of bench.py (no GPU): kernel-name parsing for profiler
output, the source hash that guards counter figures, and the one-GPU rule."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_names_from_profiler_output():
    cases = {
        "void w4a16::gemm_tile_kernel<8, 2, 2>(_Float16 const*, unsigned int const*)":
            "gemm_tile_kernel<8,2,2>",
        "_ZN5w4a1616gemm_tile_kernelILi8ELi2ELi2EEEvPKDF16_PKjS2_PDF16_iiiyiPjPf":
            "gemm_tile_kernel<8,2,2>",
        "_ZN5w4a1611gemm_kernelILi1ELi4ELi4ELi2EEEvPKDF16_": "gemm_kernel<1,4,4,2>",
        "_ZN5w4a1613repack_kernelEPKjPjii": "repack_kernel",
        # the fused-epilogue switch (a bool template argument) is dropped
        "_ZN5w4a1615gemm_lds_kernelILi4ELi2ELi2ELi4ELi3ELb1EEEvPKDF16_PKjS2_PDF16_iiimiPjPf"
        "NS_8EpilogueE": "gemm_lds_kernel<4,2,2,4,3>",
        "void w4a16::gemm_lds_kernel<4, 1, 1, 8, 3, false>(_Float16 const*)":
            "gemm_lds_kernel<4,1,1,8,3>",
        # and so is the weight format after it
        "_ZN5w4a1615gemm_lds_kernelILi4ELi1ELi1ELi8ELi3ELb0ELi2EEEvPKDF16_PKjS2_PDF16_"
        "iiimiPjPfNS_8EpilogueEPKh": "gemm_lds_kernel<4,1,1,8,3>",
        "void w4a16::gemm_kernel<1, 1, 8, 2, false, 3>(_Float16 const*)": "gemm_kernel<1,1,8,2>",
        "_ZN5w4a1614gemm_sk_kernelILi2ELi4ELi3ELi8ELb0ELi0EEEvPKDF16_PKjS2_PDF16_iiimiiPjPf":
            "gemm_sk_kernel<2,4,3,8>",
    }
    for raw, short in cases.items():
        assert bench._short_kernel_name(raw) == short


def test_source_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16


def test_traffic_is_null_for_other_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_source_hash": "0" * 16,
                             "kernels": {"k<1>": {"hbm_bytes_per_dispatch": 5.0}}}))
    assert bench.measured_traffic("k<1>", str(f)) is None
    f.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(),
                             "kernels": {"k<1>": {"hbm_bytes_per_dispatch": 5.0}}}))
    assert bench.measured_traffic("k<1>", str(f)) == 5.0
    assert bench.measured_traffic("k<2>", str(f)) is None
    assert bench.measured_traffic("k<1>", str(tmp_path / "absent.json")) is None


def test_headline_workload_is_the_large_layer_sweep(monkeypatch):
    """The default line times the batch sweep M = 1..128 on the 18432 x 73728
    layer, the configuration the metric is quoted on."""
    wl = bench.WORKLOADS["sweep"]
    assert wl["layers"] == [("large", 18432, 73728)]
    assert wl["batches"] == [1, 2, 4, 8, 16, 32, 64, 128]
    # two copies of 680 MB of packed weights: well past the 256 MB cache
    assert wl["copies"] * 18432 * 73728 // 2 > 2 * 256 * 10**6
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    assert bench.parse().workload == "sweep"


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                          timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def _fake_pmc_db(path, rows):
    import sqlite3
    path.parent.mkdir(parents=True, exist_ok=True)
    con = sqlite3.connect(str(path))
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, "
                "counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_pmc_kernels_summary(tmp_path):
    k = "_ZN5w4a1615gemm_lds_kernelILi8ELi2ELi1ELi8ELi3ELb0ELi0EEEvPKDF16_"
    # two dispatches of one GEMM kernel and one of another kernel (ignored)
    rows = []
    for d, busy, gui in ((1, 1024 * 500.0, 8 * 1000.0), (2, 1024 * 700.0, 8 * 1000.0)):
        rows += [(d, k, "SQ_VALU_MFMA_BUSY_CYCLES", busy), (d, k, "GRBM_GUI_ACTIVE", gui),
                 (d, k, "SQ_INSTS_VALU_MFMA_MOPS_F16", 32.0)]
    rows.append((3, "elementwise_kernel", "GRBM_GUI_ACTIVE", 5.0))
    _fake_pmc_db(tmp_path / "run_a" / "x" / "run_results.db", rows)
    out = tmp_path / "out.json"
    bench.pmc_kernels(str(out), [str(tmp_path / "run_a")])
    summ = json.loads(out.read_text())
    e = summ["runs"]["run_a"]["kernels"]["gemm_lds_kernel<8,2,1,8,3>"]
    assert list(summ["runs"]["run_a"]["kernels"]) == ["gemm_lds_kernel<8,2,1,8,3>"]
    assert e["GRBM_GUI_ACTIVE"]["dispatches"] == 2
    assert e["SQ_VALU_MFMA_BUSY_CYCLES"]["sum_per_dispatch"] == 1024 * 600.0
    # busy cycles over (one XCD's active cycles x 1024 SIMDs): 600 / 1000
    assert abs(e["mfma_util_percent"] - 60.0) < 1e-9
    assert summ["kernel_source_hash"] == bench.kernel_source_hash()
