"""Model-vs-counter report: what a planned call requests, next to what the GPU's
counters saw.

The model is the library's gemm_model (the no-reuse traffic count of "Reading a
matrix multiply through its tiles", section "Count the repeated reads", over
actual ranges at partial tiles, plus the work the kernel executes). The measured
side comes from rocprofv3 counter runs of ``bench.py`` on the same workload, one
counter group per run:

    rocprofv3 --pmc FETCH_SIZE -T -d D1 -o gemm -f csv -- python3 bench.py --workload W --no-cpu-baseline
    rocprofv3 --pmc WRITE_SIZE -T -d D2 -o gemm -f csv -- python3 bench.py --workload W --no-cpu-baseline
    rocprofv3 --pmc TCP_TCC_READ_REQ_sum -T -d D3 ...
    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE \\
        SQ_VALU_MFMA_BUSY_CYCLES -T -d D4 ...
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE ... -- python3 bench.py --copy-probe   (calibration)

    python -m tiled_gemm_output_amd.report --workload W --counters D1 D2 D3 D4 \\
        --copy-fetch C1 --copy-write C2

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled to bytes by what they read
for the 1 GiB device copy of ``bench.py --copy-probe``. Without counter
directories only the model is printed (no GPU needed for the automatic tile).
"""
from __future__ import annotations

import argparse
import collections
import csv
import ctypes
import glob
import json
import os
import sys

from . import inputs, tgemm

KERNELS = ("macro_tile_kernel", "small_tile_kernel", "i32_tile_kernel", "splitk_reduce_kernel", "zero_fill_kernel",
           "repack_rows_kernel")
MFMA_MOP_FLOPS = 512  # flops per unit of SQ_INSTS_VALU_MFMA_MOPS_* (checked against the model in the report)
SIMDS, XCDS = 1024, 8  # MI355X: 256 CUs x 4 SIMDs, 8 XCDs


def read_counters(dirs, skip: int = 2) -> dict:
    """{kernel name: {counter: mean value per dispatch}} over every
    *_counter_collection.csv under the given rocprofv3 output directories (the
    first `skip` dispatches of each kernel, cold caches, are left out when more
    remain)."""
    per = collections.defaultdict(lambda: collections.defaultdict(dict))  # kernel -> dispatch -> counter -> value
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    name = next((k for k in KERNELS if k in r["Kernel_Name"]), None)
                    if name is None:
                        continue
                    key = (path, int(r["Dispatch_Id"]))
                    per[name][key][r["Counter_Name"]] = float(r["Counter_Value"])
    out = {}
    for name, disp in per.items():
        sums, counts = collections.defaultdict(float), collections.defaultdict(int)
        by_file = collections.defaultdict(list)
        for key in disp:
            by_file[key[0]].append(key)
        for keys in by_file.values():
            keys.sort(key=lambda k: k[1])
            use = keys[skip:] if len(keys) > skip else keys
            for k in use:
                for c, v in disp[k].items():
                    sums[c] += v
                    counts[c] += 1
        out[name] = {c: sums[c] / counts[c] for c in sums}
    return out


def copy_scale(fetch_dir, write_dir, copy_bytes: int = 1 << 30):
    """(fetch scale, write scale): bytes per counted KiB, from the copy probe's dispatches."""
    def mean_of(d, counter):
        vals = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                vals += [float(r["Counter_Value"]) for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        if not vals:
            raise ValueError("no %s values under %s" % (counter, d))
        big = [v for v in vals if v > 0.25 * max(vals)]  # the copy dispatches, not the fill
        return sum(big) / len(big)

    return copy_bytes / (mean_of(fetch_dir, "FETCH_SIZE") * 1024.0), copy_bytes / (mean_of(write_dir, "WRITE_SIZE") * 1024.0)


def _host_plan(w, tile, auto: dict, split_k: int) -> dict:
    """The plan fields the model needs, for a forced tile without a device (the
    library's plan needs a handle for that): kernel by tile and dtype, the given
    split count; LDS size unknown (0)."""
    p = dict(auto)
    p["tile_m"], p["tile_n"], p["tile_k"] = tile
    if w.dtype == "i32":
        p["kernel"] = 2
    else:
        p["kernel"] = 3 if tuple(tile) == (16, 16, 32) else 4
    p["grid"] = -(-w.M // tile[0]) * -(-w.N // tile[1])
    p["split_k"] = max(split_k, 1) if p["kernel"] == 4 else 1
    p["lds_bytes"] = 0
    p["kernel_name"] = tgemm.KERNEL_NAMES[p["kernel"]] + " (plan built on the host)"
    return p


def plan_for(w, tile=None, op="nn", split_k=0):
    """gemm_plan_op for a workload (dense, aligned pointers). A forced tile or split
    needs a handle, hence a GPU; without one the plan is built on the host."""
    op_a = tgemm.OP_T if op[0] == "t" else tgemm.OP_N
    op_b = tgemm.OP_T if op[1] == "t" else tgemm.OP_N
    lda = w.M if op_a == tgemm.OP_T else w.K
    ldb = w.K if op_b == tgemm.OP_T else w.N
    dtype = tgemm.DTYPES[w.dtype]
    h = None
    if tile or split_k:
        try:
            h = tgemm.gemm_create()
        except tgemm.GemmError as e:
            if e.status != tgemm.ERR_NO_DEVICE:
                raise
            auto = plan_for(w, None, op, 0)
            if tile is None:
                tile = (auto["tile_m"], auto["tile_n"], auto["tile_k"])
            return _host_plan(w, tile, auto, split_k)
        if tile:
            tgemm.check(tgemm.gemm_set_tile(h, *tile), "gemm_set_tile")
        tgemm.check(tgemm.gemm_set_split_k(h, split_k), "gemm_set_split_k")
    try:
        return tgemm.gemm_plan_op(h, op_a, op_b, w.M, w.N, w.K, ctypes.c_void_p(1 << 20), max(lda, 1),
                                  ctypes.c_void_p(1 << 21), max(ldb, 1), ctypes.c_void_p(1 << 22), max(w.N, 1), dtype)
    finally:
        if h is not None:
            tgemm.gemm_destroy(h)


def report(w, plan, counters=None, scales=None) -> dict:
    """Model and (if given) measured figures of one workload, as a dict of rows."""
    dtype = tgemm.DTYPES[w.dtype]
    m = tgemm.gemm_model(plan, w.M, w.N, w.K, dtype)
    requested = m["bytes_a"] + m["bytes_b"]
    rows = collections.OrderedDict()
    rows["flops (2MNK)"] = (m["flops"], None)
    rows["executed flops (partial M, N tiles padded)"] = (m["executed_flops"], None)
    rows["requested A bytes (no reuse)"] = (m["bytes_a"], None)
    rows["requested B bytes (no reuse)"] = (m["bytes_b"], None)
    rows["C bytes written"] = (m["bytes_c"], None)
    rows["split-K workspace bytes (written + read)"] = (m["bytes_workspace"], None)
    rows["compulsory bytes (A, B once; C once)"] = (m["compulsory_bytes"], None)
    rows["working set per tile (bytes)"] = (m["footprint_bytes"], None)
    meas = collections.OrderedDict()
    if counters:
        tot = collections.defaultdict(float)
        for kern, cs in counters.items():
            for c, v in cs.items():
                tot[c] += v
        fs, ws = scales if scales else (None, None)
        if "FETCH_SIZE" in tot and fs:
            meas["HBM read bytes (FETCH_SIZE, scaled)"] = (tot["FETCH_SIZE"] * 1024 * fs,
                                                           "%.3fx compulsory A+B, %.4fx requested A+B" % (
                                                               tot["FETCH_SIZE"] * 1024 * fs /
                                                               max(m["compulsory_bytes"] - m["bytes_c"], 1),
                                                               tot["FETCH_SIZE"] * 1024 * fs / max(requested, 1)))
        if "WRITE_SIZE" in tot and ws:
            meas["HBM write bytes (WRITE_SIZE, scaled)"] = (tot["WRITE_SIZE"] * 1024 * ws, "%.3fx C bytes" % (
                tot["WRITE_SIZE"] * 1024 * ws / max(m["bytes_c"], 1)))
        if "TCP_TCC_READ_REQ_sum" in tot:
            req = tot["TCP_TCC_READ_REQ_sum"]
            meas["L2 read requests (TCP_TCC_READ_REQ_sum)"] = (req, "x 64 B = %.4fx, x 128 B = %.4fx requested A+B" % (
                req * 64 / max(requested, 1), req * 128 / max(requested, 1)))
        mops = tot.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + tot.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        if mops:
            meas["MFMA flops (MFMA_MOPS x %d)" % MFMA_MOP_FLOPS] = (mops * MFMA_MOP_FLOPS, "%.4fx executed flops" % (
                mops * MFMA_MOP_FLOPS / max(m["executed_flops"], 1)))
        for kern, cs in counters.items():
            if cs.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in cs:
                # busy cycles are summed over the 1024 SIMDs, GRBM_GUI_ACTIVE over the 8 XCDs
                busy = (cs["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS) / (cs["GRBM_GUI_ACTIVE"] / XCDS)
                meas["%s: matrix pipe busy (MFMA busy cycles per SIMD / active cycles)" % kern] = (busy, "%.1f%%" % (
                    100 * busy))
        for kern, cs in counters.items():
            for c, v in sorted(cs.items()):
                meas["raw %s %s (per dispatch)" % (kern, c)] = (v, None)
    return {"workload": w.name, "plan": plan, "model": rows, "measured": meas}


def render(r, markdown: bool = False) -> str:
    p = r["plan"]
    head = "%s: tile %dx%dx%d, kernel %s, split_k %d, grid %d" % (
        r["workload"], p["tile_m"], p["tile_n"], p["tile_k"], p["kernel_name"], p["split_k"], p["grid"])
    lines = []
    if markdown:
        lines += ["### " + head, "", "| quantity | value | note |", "|---|---|---|"]
        for k, (v, note) in list(r["model"].items()) + list(r["measured"].items()):
            lines.append("| %s | %.6g | %s |" % (k, v, note or ""))
    else:
        lines.append(head)
        for k, (v, note) in list(r["model"].items()) + list(r["measured"].items()):
            lines.append("  %-52s %16.6g  %s" % (k, v, note or ""))
    return "\n".join(lines)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="square8192_bf16", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--tile", default=None, help="forced tile tm,tn,tk (needs a GPU for the plan)")
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--op", default="nn", choices=["nn", "nt", "tn", "tt"])
    ap.add_argument("--counters", nargs="*", default=[], help="rocprofv3 -d directories of counter runs")
    ap.add_argument("--copy-fetch", default=None, help="rocprofv3 -d directory of FETCH_SIZE on bench.py --copy-probe")
    ap.add_argument("--copy-write", default=None, help="rocprofv3 -d directory of WRITE_SIZE on bench.py --copy-probe")
    ap.add_argument("--markdown", action="store_true")
    ap.add_argument("--json", action="store_true")
    args = ap.parse_args(argv)
    w = inputs.WORKLOADS[args.workload]
    tile = tuple(int(x) for x in args.tile.split(",")) if args.tile else None
    plan = plan_for(w, tile, args.op, args.split_k)
    counters = read_counters(args.counters) if args.counters else None
    scales = copy_scale(args.copy_fetch, args.copy_write) if args.copy_fetch and args.copy_write else None
    r = report(w, plan, counters, scales)
    if args.json:
        print(json.dumps({"workload": r["workload"], "plan": r["plan"],
                          "model": {k: v for k, (v, _) in r["model"].items()},
                          "measured": {k: v for k, (v, _) in r["measured"].items()}}))
    else:
        print(render(r, args.markdown))
    return 0


if __name__ == "__main__":
    sys.exit(main())
