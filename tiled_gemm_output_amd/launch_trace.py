"""Per-launch time and gfx clock over the first launches of a process.

Two ways to see how the card's clock settles under a sustained product:

* run mode (no profiler): a fresh process launches the workload N times back to
  back with no warm-up, HIP events around each launch on the launch stream.

      python3 tiled_gemm_output_amd/launch_trace.py --launches 300 --json out.json

* counter mode: the same launches under ``rocprofv3 --pmc GRBM_GUI_ACTIVE``; the
  counter is the busy cycles of the graphics block summed over the 8 XCDs, so
  cycles / 8 / dispatch duration is the clock each dispatch actually ran at (the
  driver's metrics table, which amd-smi reads, is refreshed far less often than a
  launch lasts).

      rocprofv3 --pmc GRBM_GUI_ACTIVE -T -d D -o trace -f csv -- \\
          python3 tiled_gemm_output_amd/launch_trace.py --launches 300
      python3 tiled_gemm_output_amd/launch_trace.py --from-rocprof D

Both print a table of launch ranges (mean time per launch, TFLOP/s, clock).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

if __package__ in (None, ""):  # run as a script (as under rocprofv3): import the package by path
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    __package__ = "tiled_gemm_output_amd"
    import tiled_gemm_output_amd  # noqa: F401  (the parent package of the relative imports below)

XCDS = 8  # GRBM_GUI_ACTIVE is summed over the MI355X's 8 XCDs
RANGES = [(1, 1), (2, 5), (6, 25), (26, 50), (51, 100), (101, 150), (151, 200), (201, 250), (251, 300),
          (301, 400), (401, 600), (601, 1000)]


def run(workload: str, launches: int) -> dict:
    import numpy as np
    import torch

    from . import inputs, tgemm

    if not torch.cuda.is_available():
        raise SystemExit("launch_trace: no GPU visible")
    w = inputs.WORKLOADS[workload]
    dtype = tgemm.DTYPES[w.dtype]
    a, b = inputs.make(w)
    torch.cuda.set_device(0)
    da = torch.from_numpy(a.view(np.int16 if a.dtype == np.uint16 else np.int32)).cuda()
    db = torch.from_numpy(b.view(np.int16 if b.dtype == np.uint16 else np.int32)).cuda()
    ob = tgemm.OUT_BYTES[dtype]
    dc = torch.empty((w.M, w.N), dtype=torch.int16 if ob == 2 else torch.int32, device="cuda")
    h = tgemm.gemm_create()
    if w.tile:
        tgemm.check(tgemm.gemm_set_tile(h, *w.tile), "gemm_set_tile")
    plan = tgemm.gemm_plan(h, w.M, w.N, w.K, da.data_ptr(), w.K, db.data_ptr(), w.N, dc.data_ptr(), w.N, dtype)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    e0 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(launches):
        ev[i][0].record(stream)
        tgemm.check(tgemm.gemm_run(h, w.M, w.N, w.K, da.data_ptr(), w.K, db.data_ptr(), w.N, dc.data_ptr(), w.N,
                                   dtype, sp), "gemm_run")
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    tgemm.gemm_destroy(h)
    start_ms = [e0.elapsed_time(s) for s, _ in ev]
    dur_us = [1e3 * s.elapsed_time(e) for s, e in ev]
    per = [{"launch": i + 1, "start_ms": start_ms[i], "us": dur_us[i], "mhz": None} for i in range(launches)]
    return {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "flops": 2.0 * w.M * w.N * w.K,
            "kernel": plan["kernel_name"], "tile": [plan["tile_m"], plan["tile_n"], plan["tile_k"]],
            "source": "HIP events around each launch on the launch stream (no profiler)", "launches": per}


def from_rocprof(d: str) -> dict:
    """Per-dispatch duration and clock (GRBM_GUI_ACTIVE / 8 / duration) from a counter run."""
    rows = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != "GRBM_GUI_ACTIVE" or "tile_kernel" not in r["Kernel_Name"]:
                    continue
                rows[(path, int(r["Dispatch_Id"]))] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                                                       float(r["Counter_Value"]))
    if not rows:
        raise SystemExit("launch_trace: no GRBM_GUI_ACTIVE dispatches under %s" % d)
    per = []
    t_first = min(v[0] for v in rows.values())
    for i, key in enumerate(sorted(rows, key=lambda k: rows[k][0])):
        t0, t1, cyc = rows[key]
        dur_ns = max(t1 - t0, 1)
        per.append({"launch": i + 1, "start_ms": 1e-6 * (t0 - t_first), "us": 1e-3 * dur_ns,
                    "mhz": 1e3 * cyc / XCDS / dur_ns})
    return {"source": "rocprofv3 --pmc GRBM_GUI_ACTIVE (per dispatch; clock = cycles / %d XCDs / duration)" % XCDS,
            "launches": per}


def table(t: dict, flops: float | None) -> str:
    import statistics

    per = t["launches"]
    lines = ["| launches | mean us per launch | min us | TFLOP/s (mean) | gfx MHz, median |", "|---|---|---|---|---|"]
    for lo, hi in RANGES:
        sel = [p for p in per if lo <= p["launch"] <= hi]
        if not sel:
            continue

        def med(key):
            v = [p[key] for p in sel if p.get(key) is not None]
            return "%.0f" % statistics.median(v) if v else "-"

        mean = sum(p["us"] for p in sel) / len(sel)
        lines.append("| %d-%d | %.1f | %.1f | %s | %s |" % (
            lo, sel[-1]["launch"], mean, min(p["us"] for p in sel),
            "%.0f" % (flops / (mean * 1e-6) / 1e12) if flops else "-", med("mhz")))
    return "\n".join(lines)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="square8192_bf16")
    ap.add_argument("--launches", type=int, default=300)
    ap.add_argument("--json", default=None, help="write the per-launch record here")
    ap.add_argument("--from-rocprof", default=None, help="render a GRBM_GUI_ACTIVE counter run instead")
    ap.add_argument("--flops", type=float, default=None, help="flops per launch for --from-rocprof (default 2*8192^3)")
    args = ap.parse_args(argv)
    if args.from_rocprof:
        t = from_rocprof(args.from_rocprof)
        flops = args.flops or 2.0 * 8192 ** 3
    else:
        t = run(args.workload, args.launches)
        flops = t["flops"]
        print("launch_trace: %s, %s, %d launches" % (t["workload"], t["kernel"], len(t["launches"])), flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(t, f)
    print(t["source"])
    print(table(t, flops), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
