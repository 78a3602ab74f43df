"""The model-vs-counter report on synthetic rocprofv3 CSV files (host only)."""
import os

from tiled_gemm_output_amd import inputs, report

HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size","Kernel_Id",'
          '"Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count","Accum_VGPR_Count",'
          '"SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')


def write_csv(d, name, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, name + "_counter_collection.csv"), "w") as f:
        f.write(HEADER + "\n")
        for i, (kern, counter, value) in enumerate(rows):
            f.write('%d,%d,"Agent 1",1,1,1,64,1,"%s",256,0,0,0,0,0,"%s",%f,0,1\n' % (i + 1, i + 1, kern, counter, value))


def test_counters_and_scales(tmp_path):
    d1, d2 = str(tmp_path / "fetch"), str(tmp_path / "write")
    # two cold dispatches are skipped, then the mean of the rest per kernel
    write_csv(d1, "g", [("macro_tile_kernel", "FETCH_SIZE", v) for v in (999, 999, 100, 300)] +
              [("splitk_reduce_kernel", "FETCH_SIZE", v) for v in (50, 50, 10, 10)])
    write_csv(d2, "g", [("void tg::macro_tile_kernel<...>", "WRITE_SIZE", 64.0)] * 4)
    c = report.read_counters([d1, d2])
    assert c["macro_tile_kernel"]["FETCH_SIZE"] == 200 and c["macro_tile_kernel"]["WRITE_SIZE"] == 64
    assert c["splitk_reduce_kernel"]["FETCH_SIZE"] == 10
    cf, cw = str(tmp_path / "cf"), str(tmp_path / "cw")
    # the copy probe: 1 GiB; FETCH_SIZE reads half of it, WRITE_SIZE all of it (plus a small fill dispatch)
    write_csv(cf, "c", [("copy", "FETCH_SIZE", 4.0)] + [("copy", "FETCH_SIZE", 524288.0)] * 5)
    write_csv(cw, "c", [("copy", "WRITE_SIZE", 1048576.0)] * 5)
    fs, ws = report.copy_scale(cf, cw)
    assert fs == 2.0 and ws == 1.0
    w = inputs.WORKLOADS["skinny128x8192x8192_bf16"]
    r = report.report(w, report.plan_for(w), c, (fs, ws))
    read = r["measured"]["HBM read bytes (FETCH_SIZE, scaled)"][0]
    assert read == (200 + 10) * 1024 * 2.0
    assert r["model"]["split-K workspace bytes (written + read)"][0] == 2 * 4 * 4 * 128 * 8192
    text = report.render(r, markdown=True)
    assert text.startswith("### skinny128x8192x8192_bf16: tile 128x128x64") and "| flops (2MNK) |" in text


def test_matrix_pipe_busy(tmp_path):
    """Busy cycles are summed over 1024 SIMDs and GRBM_GUI_ACTIVE over 8 XCDs."""
    d = str(tmp_path / "mfma")
    rows = []
    for _ in range(4):
        rows += [("macro_tile_kernel", "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 750.0),
                 ("macro_tile_kernel", "GRBM_GUI_ACTIVE", 8 * 1000.0),
                 ("macro_tile_kernel", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1.0)]
    write_csv(d, "g", rows)
    c = report.read_counters([d], skip=0)
    w = inputs.WORKLOADS["square4096_bf16"]
    r = report.report(w, report.plan_for(w), c, None)
    key = "macro_tile_kernel: matrix pipe busy (MFMA busy cycles per SIMD / active cycles)"
    assert abs(r["measured"][key][0] - 0.75) < 1e-12 and r["measured"][key][1] == "75.0%"
