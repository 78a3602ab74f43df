"""The per-launch clock of launch_trace.py from a counter run (CPU only, synthetic CSV)."""
import csv

from tiled_gemm_output_amd import launch_trace


def write_counters(path, launches):
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (t0, t1, cycles) in enumerate(launches):
            row = {c: 0 for c in cols}
            row.update(Dispatch_Id=i + 1, Kernel_Name="macro_tile_kernel", Counter_Name="GRBM_GUI_ACTIVE",
                       Counter_Value=cycles, Start_Timestamp=t0, End_Timestamp=t1)
            w.writerow(row)
        # another kernel's dispatch is ignored
        row = {c: 0 for c in cols}
        row.update(Dispatch_Id=99, Kernel_Name="other_kernel", Counter_Name="GRBM_GUI_ACTIVE", Counter_Value=1,
                   Start_Timestamp=5, End_Timestamp=6)
        w.writerow(row)


def test_clock_is_cycles_per_xcd_over_duration(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    # out of order on purpose: dispatches are sorted by start time
    launches = [(2_000_000, 2_800_000, 8 * 1_360_000), (1_000, 801_000, 8 * 1_600_000)]
    write_counters(d / "trace_counter_collection.csv", launches)
    t = launch_trace.from_rocprof(str(d))
    per = t["launches"]
    assert [p["launch"] for p in per] == [1, 2]
    assert abs(per[0]["us"] - 800.0) < 1e-9 and abs(per[0]["mhz"] - 2000.0) < 1e-9  # 1.6 M cycles in 800 us
    assert abs(per[1]["us"] - 800.0) < 1e-9 and abs(per[1]["mhz"] - 1700.0) < 1e-9
    assert abs(per[1]["start_ms"] - 1.999) < 1e-9
    text = launch_trace.table(t, 2.0 * 8192 ** 3)
    assert "| 1-1 | 800.0 | 800.0 |" in text and "| 2-2 |" in text
