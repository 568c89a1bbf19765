"""Host-side summaries of rocprofv3 counter output (no GPU, no profiler)."""
import csv
import os
import sys
from types import SimpleNamespace

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from expert_ffn_layer_gemm_amd import profiling  # noqa: E402

KERNEL = "void moe::k_tiled3<false, true, 2, 4, 256, 2, 2, 128, false>(moe::GemmArgs)"


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_stall_summary_fractions(tmp_path, monkeypatch):
    monkeypatch.setattr(profiling, "OUT_DIR", str(tmp_path))
    vals = {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 250.0, "SQ_WAIT_INST_ANY": 400.0,
            "SQ_WAIT_INST_LDS": 10.0, "SQ_ACTIVE_INST_ANY": 350.0, "SQ_ACTIVE_INST_VALU": 100.0,
            "SQ_ACTIVE_INST_LDS": 30.0, "SQ_LDS_BANK_CONFLICT": 0.0}
    rows = []
    for d in (1, 2):                                   # two dispatches, counters split over two rows each
        for k, v in vals.items():
            rows += [{"Dispatch_Id": d, "Kernel_Name": KERNEL, "Counter_Name": k, "Counter_Value": v / 2}] * 2
    rows.append({"Dispatch_Id": 3, "Kernel_Name": "other", "Counter_Name": "SQ_WAVE_CYCLES",
                 "Counter_Value": 1e9})                # another kernel: ignored
    path = tmp_path / "c.csv"
    _write_counters(path, rows)
    profiling.stall_summary(SimpleNamespace(counters=str(path), rocprof_kernel="k_tiled3<false, true,",
                                            workload="w", bench_kernel="k", cmd="cmd"))
    text = (tmp_path / "k_w_stalls.txt").read_text()
    assert "dispatches: 2; SQ_WAVE_CYCLES 1000 per dispatch" in text
    assert "SQ_WAIT_ANY | 250 | 0.250 |" in text
    assert "SQ_WAIT_INST_ANY | 400 | 0.400 |" in text
    assert "# command: cmd" in text


def test_busy_summary_clock_and_rate(tmp_path, monkeypatch):
    """1 ms kernel, 2e6 GPU-active cycles per XCD -> 2.0 GHz; half the SIMD
    cycles MFMA-busy; 1e8 MFMAs of 16384 FLOP in 1 ms -> 1638.4 TFLOP/s."""
    monkeypatch.setattr(profiling, "OUT_DIR", str(tmp_path))
    gui = 2e6
    vals = {"GRBM_GUI_ACTIVE": 8 * gui, "SQ_BUSY_CYCLES": 1.0,
            "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * gui, "SQ_INSTS_MFMA": 1e8}
    rows = [{"Dispatch_Id": d, "Kernel_Name": KERNEL, "Counter_Name": k, "Counter_Value": v}
            for d in (1, 2) for k, v in vals.items()]
    cpath = tmp_path / "c.csv"
    _write_counters(cpath, rows)
    tpath = tmp_path / "t.csv"
    with open(tpath, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerow({"Kernel_Name": KERNEL, "Start_Timestamp": 0, "End_Timestamp": 1_000_000})
        w.writerow({"Kernel_Name": KERNEL, "Start_Timestamp": 5_000_000, "End_Timestamp": 6_000_000})
    profiling.busy_summary(SimpleNamespace(counters=str(cpath), trace=str(tpath), rocprof_kernel="k_tiled3<false",
                                           workload="w", bench_kernel="k", cmd="cmd", mfma_flop=16384.0,
                                           peak_tflops=2500.0))
    text = (tmp_path / "k_w_mfma_busy.txt").read_text()
    assert "average duration 1000.0 us" in text
    assert "clock 2.000 GHz" in text
    assert "matrix cores busy 50.0 %" in text
    assert "1638.4 TFLOP/s, 65.5 %" in text
