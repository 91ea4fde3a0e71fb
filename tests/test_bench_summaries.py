"""Host logic of bench.py that turns rocprofv3 output into the committed summaries:
the per-kernel counter ratios, the timed-region average of a kernel trace, and the
guard that drops the HBM traffic record once the GEMM source has changed.  Synthetic
CSVs with known values; no GPU."""
import csv
import json

import pytest

import bench

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
        "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
        "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _counter_csv(path, kernels):
    """kernels: {name: [ {counter: value}, ... one dict per dispatch ]}; each value is
    split over two rows (two instances), as rocprofv3 reports per-instance values."""
    rows, did = [], 0
    for name, disps in kernels.items():
        for d in disps:
            did += 1
            for c, v in d.items():
                for half in (0.25 * v, 0.75 * v):
                    rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": c,
                                 "Counter_Value": half})
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS, restval="0")
        w.writeheader()
        w.writerows(rows)


def _stats_csv(path, durations_ns):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage",
                                          "MinNs", "MaxNs"], restval="0")
        w.writeheader()
        for n, ns in durations_ns.items():
            w.writerow({"Name": n, "Calls": 8, "AverageNs": ns})


def test_kernel_util_ratios(tmp_path):
    # MFMA busy summed over 1024 SIMDs, SQ busy over 32 shader engines, GRBM over 8 XCDs:
    # 1024 * 500 / (32 * 1000) per SIMD / per SE -> 50%; GPU busy 8 * 2000 -> 25%.
    # The early dispatches (clocks ramping) carry other values and must be ignored:
    # only the last quarter (2 of 8) counts.
    good = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 500.0, "SQ_BUSY_CYCLES": 32 * 1000.0,
            "GRBM_GUI_ACTIVE": 8 * 2000.0, "SQ_WAIT_ANY": 30.0, "SQ_WAVE_CYCLES": 120.0}
    early = dict(good, SQ_VALU_MFMA_BUSY_CYCLES=1.0)
    lds = {"SQ_LDS_IDX_ACTIVE": 300.0, "SQ_LDS_BANK_CONFLICT": 60.0, "SQ_BUSY_CYCLES": 100.0,
           "SQ_WAVE_CYCLES": 1.0, "GRBM_GUI_ACTIVE": 1.0}
    util, ldsf, stats = tmp_path / "u.csv", tmp_path / "l.csv", tmp_path / "s.csv"
    _counter_csv(util, {"k_a(int)": [early] * 6 + [good] * 2, "copy_kernel": [dict(good, SQ_VALU_MFMA_BUSY_CYCLES=0.0)] * 4})
    _counter_csv(ldsf, {"k_a(int)": [lds] * 8})
    _stats_csv(stats, {"k_a(int)": 12345.0})
    text = bench.summarize_kernel_util(str(util), str(stats), ["cmd"], "t", lds_csv=str(ldsf))
    row = [l for l in text.splitlines() if l.startswith("| `k_a`")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1:] == ["8", "12.35", "50.0%", "25.0%", "25.0%", "3.00", "0.20"]
    assert "copy_kernel" not in text                      # no MFMA work: not a GEMM row


def test_timed_region_average(tmp_path):
    trace = tmp_path / "t.csv"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # 5 warmup launches of 200 ns, then 3 timed launches of 100 ns, written out of order
        rows = [(i * 1000, 200) for i in range(5)] + [(10000 + i * 1000, 100) for i in range(3)]
        for s, d in reversed(rows):
            w.writerow({"Kernel_Name": bench.GEMM_KERNEL_PREFIX + "(...)", "Start_Timestamp": s,
                        "End_Timestamp": s + d})
        w.writerow({"Kernel_Name": "other", "Start_Timestamp": 99999, "End_Timestamp": 199999})
    assert bench.timed_region_avg_ns(str(trace), 3) == pytest.approx(100.0)
    assert bench.timed_region_avg_ns(str(trace), 4) == pytest.approx(125.0)


def test_traffic_record_needs_the_current_kernel_source(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.measured_traffic() is None                # no record
    rec.write_text(json.dumps({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 7}))
    assert bench.measured_traffic() is None                # taken on another source
    rec.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 7}))
    assert bench.measured_traffic() == 7
