#!/usr/bin/env python3
"""Benchmark of the output-stationary tiled GEMM C = A @ B on one MI355X.

A step is one gemm_run (one kernel launch) over resident device inputs; the
default workload is the square bf16 product M = N = K = 8192 (bf16 inputs, fp32
accumulation, bf16 output). Prints ONE JSON line on stdout:

  value        TFLOP/s = 2*M*N*K / (time per step)
  roofline     the dominant kernel against its roof: MFMA peak (dense bf16
               2516.6 TFLOP/s = 256 CUs x 4096 flop/clk x 2.4 GHz) for
               compute-bound shapes, HBM (8000 GB/s, compulsory bytes) otherwise;
               `achieved` uses the kernel's average launch time from HIP events
               on the launch stream; `traffic` = HBM bytes per launch from the
               committed rocprofv3 counter file of this kernel source, else null
  cpu_baseline the oracle (plain CPU triple loop, binary64 sums) timed on a
               bounded sample of rows of the same product on the host cores
  check        the sampled rows of the GPU result against those oracle rows
  sclk         the gfx clock and socket power under the same load (the driver's metrics
               table, read in process through amdsmi while the launches continue after
               the timed region) and the MFMA peak and fraction at that clock

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of MFMA peak at 1 GPU (bf16 8192³; ragged shapes)"
PEAK_MFMA_16BIT_TFLOPS = 2516.6  # dense fp16/bf16: 256 CUs x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBPS = 8000.0
RIDGE = PEAK_MFMA_16BIT_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)  # flop per byte


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "tiled_gemm_output_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, sha: str):
    """HBM bytes per launch from profiles/counters_<workload>.json if it was taken
    on this kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != sha:
        return None
    return d.get("hbm_bytes_per_launch")


def smi_reader():
    """A function returning (gfx clock in MHz averaged over the XCDs, the reported maximum
    clock, socket power in W) for the GPU torch uses as device 0, read in this process from
    the driver's metrics table through the amdsmi library (no child process); None when the
    library or the table is not usable here."""
    try:
        import amdsmi
        import torch

        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        props = torch.cuda.get_device_properties(0)
        want = tuple(getattr(props, k, None) for k in ("pci_domain_id", "pci_bus_id", "pci_device_id"))
        handle = None
        for h in handles:
            dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")
            if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                handle = h
        if handle is None and len(handles) == 1:
            handle = handles[0]
        if handle is None:
            return None
        try:
            top = float(amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)["max_clk"])
        except Exception:
            top = None
    except Exception:
        return None

    def num(x):
        return float(x) if isinstance(x, (int, float)) and not isinstance(x, bool) else None

    def read():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        except Exception:
            return None, None, None
        clks = m.get("current_gfxclks")
        cur = [num(v) for v in clks] if isinstance(clks, (list, tuple)) else []
        cur = [v for v in cur if v is not None and 0 < v < 10000]  # unused XCD slots read as N/A or 0xFFFF
        if not cur:
            return None, None, None
        watts = num(m.get("current_socket_power"))
        if watts is None or watts >= 65535:
            watts = num(m.get("average_socket_power"))
        return sum(cur) / len(cur), top, watts

    return read


# The driver's metrics table (what amd-smi shows) is refreshed far less often than a launch
# lasts (it changed once in the first 820 ms of load): readings in the first second of the
# window may still show the clock from before the load, and are left out.
CLOCK_SETTLE_S = 1.0


def sample_clock_under_load(step, seconds: float):
    """Keep launching ``step`` for CLOCK_SETTLE_S + ``seconds`` while a second thread reads
    the gfx clock and socket power (smi_reader) back to back; returns the clock samples
    (MHz), the power samples (W), both read after the first CLOCK_SETTLE_S seconds and while
    the launches were running, and the reported maximum clock."""
    import threading

    import torch

    samples, top = [], [None]
    stop = threading.Event()
    read = smi_reader()
    if read is None:
        return [], [], None

    def sampler():
        while not stop.is_set():
            t0 = time.perf_counter()
            mhz, mx, watts = read()
            if mhz is None:
                return
            samples.append((t0, time.perf_counter(), mhz, watts))
            top[0] = mx
            time.sleep(0.005)

    th = threading.Thread(target=sampler, daemon=True)
    t_keep = time.perf_counter() + CLOCK_SETTLE_S
    t_end = t_keep + seconds
    for _ in range(20):
        step()
    th.start()
    while time.perf_counter() < t_end or (th.is_alive() and not any(x[0] >= t_keep for x in samples)
                                          and time.perf_counter() < t_end + 10):
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    load_end = time.perf_counter()
    stop.set()
    th.join(timeout=20)
    # only readings taken after the settle time and completed while the launches were still running
    kept = [(mhz, watts) for t0, t, mhz, watts in samples if t0 >= t_keep and t <= load_end]
    return [m for m, _ in kept], [w for _, w in kept if w is not None], top[0]


def cpu_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, min(n, 16))


def cpu_model() -> str | None:
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(o, a, b, w, target_s: float):
    """Time the oracle on a bounded set of full rows; return (baseline dict, rows, oracle rows)."""
    import numpy as np

    threads = cpu_threads()
    in_kind, out_kind = w.in_kind, w.out_kind
    rng = np.random.default_rng(w.index)
    # calibrate with one row per thread
    probe = np.sort(rng.choice(w.M, size=min(threads, w.M), replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    o.gemm_rows(a, b, probe, in_kind, out_kind, threads=threads)
    t_probe = time.perf_counter() - t0
    per_round = max(t_probe, 1e-4)  # one row per thread
    rounds = max(1, int(target_s / per_round))
    n = int(min(w.M, rounds * len(probe)))
    rows = np.sort(rng.choice(w.M, size=n, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    ref = o.gemm_rows(a, b, rows, in_kind, out_kind, threads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * n * w.N * w.K
    base = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": "%d of the %d output rows (%d x %d x %d x 2 = %.3g flop, binary64 sums) in %.1f s; "
                  "full product extrapolates to %.0f s" % (n, w.M, n, w.N, w.K, flops, dt,
                                                            2.0 * w.M * w.N * w.K / (flops / dt)),
    }
    return base, rows, ref


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The card's clock settles only after ~100 launches of sustained load (8192^3 runs
    # ~915 us per launch at first, ~795 us from then on); the default warmup covers that.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="square8192_bf16")
    ap.add_argument("--shape", default=None,
                    help="M,N,K replacing the workload's dimensions (same formats, value law and seeds)")
    ap.add_argument("--tile", default=None, help="force a tile, e.g. 256,256,64")
    ap.add_argument("--split-k", type=int, default=0, help="force the K-slice count (0: the library's choice)")
    ap.add_argument("--op", default="nn", choices=["nn", "nt", "tn", "tt"],
                    help="operand forms: t = that operand is stored transposed (A as K x M, B as N x K)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed steps in one HIP graph and replay it once (for products so small "
                         "that the host's launch loop, not the GPU, would set the step rate); the time per launch "
                         "is then the time per step")
    # the one-row-per-thread calibration overestimates the per-row cost about twofold:
    # a 22 s target gives about 10-12 s of oracle work
    ap.add_argument("--cpu-seconds", type=float, default=22.0)
    ap.add_argument("--clock-window", type=float, default=2.0,
                    help="seconds of clock readings kept while the launches continue after the timed "
                         "region, after a first second whose readings are left out (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain device copy of 1 GiB (5 times): the known-size kernel whose "
                         "FETCH_SIZE / WRITE_SIZE readings scale the GEMM's counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py: one GPU only; --gpus %d is not supported. Across GPUs the product would be split "
            "by row blocks of C (each GPU holding B), which needs no communication during the product; the "
            "benchmark measures one GPU's share." % args.gpus)
        return 2

    import numpy as np
    import torch

    from tiled_gemm_output_amd import inputs, tgemm

    if not os.path.exists(tgemm.LIBRARY):
        from tiled_gemm_output_amd import build as lib_build

        lib_build.build()
    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        return 1
    torch.cuda.set_device(0)
    if args.copy_probe:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return 0
    w = inputs.WORKLOADS[args.workload]
    if args.shape:
        import dataclasses

        M, N, K = (int(x) for x in args.shape.split(","))
        w = dataclasses.replace(w, name="%s_as_%dx%dx%d" % (w.name, M, N, K), M=M, N=N, K=K)
    dtype = tgemm.DTYPES[w.dtype]
    log("bench: workload %s M=%d N=%d K=%d dtype=%s" % (w.name, w.M, w.N, w.K, w.dtype))
    a, b = inputs.make(w)
    op_a = tgemm.OP_T if args.op[0] == "t" else tgemm.OP_N
    op_b = tgemm.OP_T if args.op[1] == "t" else tgemm.OP_N
    sa = np.ascontiguousarray(a.T) if op_a == tgemm.OP_T else a  # what is stored on the device
    sb = np.ascontiguousarray(b.T) if op_b == tgemm.OP_T else b
    lda, ldb = sa.shape[1], sb.shape[1]
    da = torch.from_numpy(sa.view(np.int16 if a.dtype == np.uint16 else np.int32)).cuda()
    db = torch.from_numpy(sb.view(np.int16 if b.dtype == np.uint16 else np.int32)).cuda()
    del sa, sb
    ob = tgemm.OUT_BYTES[dtype]
    dc = torch.empty((w.M, w.N), dtype=torch.int16 if ob == 2 else torch.int32, device="cuda")
    h = tgemm.gemm_create()
    if args.tile:
        tgemm.check(tgemm.gemm_set_tile(h, *[int(x) for x in args.tile.split(",")]))
    tgemm.check(tgemm.gemm_set_split_k(h, args.split_k), "gemm_set_split_k")
    plan = tgemm.gemm_plan_op(h, op_a, op_b, w.M, w.N, w.K, da.data_ptr(), lda, db.data_ptr(), ldb, dc.data_ptr(),
                              w.N, dtype)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step():
        tgemm.check(tgemm.gemm_run_op(h, op_a, op_b, w.M, w.N, w.K, da.data_ptr(), lda, db.data_ptr(), ldb,
                                      dc.data_ptr(), w.N, dtype, sp), "gemm_run_op")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: warmup done (%d steps), timing %d steps" % (args.warmup, args.steps))
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.graph:
        # The launches only enqueue kernels on the given stream (no allocation once the
        # warm-up has sized any split-K workspace, no memset), so they can be captured.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs = torch.cuda.current_stream().cuda_stream
            for _ in range(args.steps):
                tgemm.check(tgemm.gemm_run_op(h, op_a, op_b, w.M, w.N, w.K, da.data_ptr(), lda, db.data_ptr(), ldb,
                                              dc.data_ptr(), w.N, dtype, cs), "gemm_run_op (captured)")
        graph.replay()  # first replay uploads the graph; untimed
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_start.record(stream)
        graph.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = t_start.elapsed_time(t_end)
        per_launch_ms = [total_ms / args.steps]
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_start.record(stream)
        for i in range(args.steps):
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = t_start.elapsed_time(t_end)
        per_launch_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = total_ms / args.steps
    launch_ms = float(np.mean(per_launch_ms))
    flops = 2.0 * w.M * w.N * w.K
    value = flops / (ms_per_step * 1e-3) / 1e12
    log("bench: %.4f ms/step (events), %.4f ms/launch (mean), min %.4f, wall %.3f s" %
        (ms_per_step, launch_ms, min(per_launch_ms), wall))

    ib = 2 if dtype != tgemm.I32_I32 else 4
    compulsory = ib * (w.M * w.K + w.K * w.N) + ob * w.M * w.N
    intensity = flops / compulsory
    sha = kernel_source_sha()
    # the recorded counters are for the default launch (library's tile and split, no transposes)
    default_launch = args.op == "nn" and not args.tile and args.split_k == 0
    traffic = load_traffic(w.name, sha) if default_launch else None
    if intensity >= RIDGE:
        achieved = flops / (launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_16BIT_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_MFMA_16BIT_TFLOPS, "traffic": traffic}
    else:
        achieved = compulsory / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic}

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "bf16" if w.in_kind == "bf16" else w.in_kind,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "in": w.in_kind, "acc": "fp32" if ib == 2 else "i32",
                   "out": w.out_kind, "tile": [plan["tile_m"], plan["tile_n"], plan["tile_k"]],
                   "op": args.op, "kernel": plan["kernel_name"], "grid": plan["grid"], "split_k": plan["split_k"],
                   "tail_split_k": plan["tail_split_k"], "tail_m0": plan["tail_m0"], "threads": plan["threads"],
                   "vector_loads": plan["vector_loads"], "kernel_source_sha": sha,
                   "timing": "hip graph of the timed steps" if args.graph else "hip events around each launch"},
        "pct_of_mfma_peak": 100.0 * value / PEAK_MFMA_16BIT_TFLOPS,
        "launch_us": {"mean": 1e3 * launch_ms, "median": 1e3 * float(np.median(per_launch_ms)),
                      "min": 1e3 * float(np.min(per_launch_ms))},
        "roofline": roof,
        "cpu_baseline": None,
    }
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count}
    result["sclk"] = None
    # No clock window under rocprofv3: its launches would add thousands of profiled dispatches
    # to the counter files.
    profiled = "ROCPROFILER_LIBRARY_CTOR" in os.environ or "ROCPROF_OUTPUT_PATH" in os.environ
    if args.clock_window > 0 and not profiled:
        samples, watts, max_mhz = sample_clock_under_load(step, args.clock_window)
        if samples:
            med = float(np.median(samples))
            top = max_mhz or 2400.0
            peak_now = PEAK_MFMA_16BIT_TFLOPS * med / top
            result["sclk"] = {
                "source": "driver metrics table via amdsmi, in process (gfx clock, mean over XCDs; socket power), read "
                          "while the same launches continue for %.1f s after the timed region (readings of the first "
                          "%.1f s left out)" % (
                              CLOCK_SETTLE_S + args.clock_window, CLOCK_SETTLE_S),
                "median_mhz": med, "min_mhz": float(np.min(samples)), "max_mhz": float(np.max(samples)),
                "samples": len(samples), "max_clk_mhz": top,
                "mfma_peak_at_median_tflops": peak_now,
                "frac_of_peak_at_median": (flops / (launch_ms * 1e-3) / 1e12) / peak_now,
                "socket_power_w_median": float(np.median(watts)) if watts else None,
                "socket_power_w_max": float(np.max(watts)) if watts else None,
            }
    if not args.no_cpu_baseline:
        import oracle

        o = oracle.get()
        base, rows, ref = cpu_baseline(o, a, b, w, args.cpu_seconds)
        result["cpu_baseline"] = base
        got = dc[torch.from_numpy(rows).cuda()].cpu().numpy()
        if w.out_kind == "f32":
            gv = got.view(np.float32).astype(np.float64)
            rv = ref.astype(np.float64)
        else:
            gv = (got.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64) \
                if w.out_kind == "bf16" else got.view(np.float16).astype(np.float64)
            rv = (ref.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64) \
                if w.out_kind == "bf16" else ref.view(np.float16).astype(np.float64)
        scale = float(np.max(np.abs(rv)))
        err = np.abs(gv - rv)
        p_bits, emin = {"f32": (24, -126), "bf16": (8, -126), "f16": (11, -14)}[w.out_kind]
        ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(rv != 0, np.abs(rv), 1.0))), emin) - (p_bits - 1))
        ok = bool(np.all(err <= np.maximum(2e-3 * scale, ulp)))
        result["check"] = {"rows": int(len(rows)), "rule": "|C-R| <= max(2e-3*max|R|, 1 ulp of R)",
                           "passed": ok, "max_err_over_max_abs": float(err.max() / scale),
                           "max_err_ulps": float(np.max(err / ulp)),
                           "differing_elements": int(np.sum(got.view(np.int16 if ob == 2 else np.int32)
                                                            != ref.view(np.int16 if ob == 2 else np.int32)))}
    tgemm.gemm_destroy(h)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
