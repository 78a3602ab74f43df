"""Counter tests: what rocprofv3 counts on the GPU against the library's model.

Each case runs ``bench.py`` on one workload under ``rocprofv3 --pmc`` in a child
process (hard time limit, one counter group per run) and reads the per-dispatch
counters of the GEMM kernel:

* MFMA work: SQ_INSTS_VALU_MFMA_MOPS_{BF16,F16} x 512 flops equals the executed
  flops of gemm_model for the planned call exactly (2MNK plus the zero padding of
  partial tiles) -- the pages' 4,194,304 operations at 128^3 with the 16x16x32 tile
  ("Reading a matrix multiply through its tiles", "Count the repeated reads");
* traffic: L1-to-L2 read requests x 128 bytes equal the no-reuse count of the same
  section (A read once per column tile, B once per row tile) on the 256x256 tile;
* a plan with a split-K tail: the MFMA ops of its two launches per call equal the
  model's executed flops;
* LDS layout: no bank conflicts on the 256x256 tile (the Mojo puzzle page discusses
  conflict-free shared-memory access; here the XOR swizzles of both LDS tiles and of
  the epilogue staging).

A missing profiler or a run that produced no counters skips the case (the test is
about the counts, not the tool); a wrong count fails it.
"""
import csv
import glob
import os
import shutil
import subprocess
import sys

import pytest

from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = ("macro_tile_kernel", "small_tile_kernel")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if shutil.which("rocprofv3") is None:
        pytest.skip("rocprofv3 not found")


def per_dispatch(tmp_path, names, workload, tile=None, shape=None):
    """{dispatch id: {counter: value}} of the GEMM kernels over a bench.py run of 4 calls."""
    out = tmp_path / "prof"
    cmd = ["rocprofv3", "--pmc", *names, "-d", str(out), "-o", "c", "-f", "csv", "--", sys.executable,
           os.path.join(ROOT, "bench.py"), "--no-cpu-baseline", "--steps", "3", "--warmup", "1", "--workload", workload]
    if tile:
        cmd += ["--tile", ",".join(str(x) for x in tile)]
    if shape:
        cmd += ["--shape", ",".join(str(x) for x in shape)]
    print("counter case %s tile %s: %s" % (workload, tile, " ".join(names)), flush=True)
    try:
        r = subprocess.run(cmd, cwd="/tmp", capture_output=True, text=True, timeout=120,
                           env=dict(os.environ, TMPDIR="/tmp"))
    except subprocess.TimeoutExpired:
        pytest.skip("rocprofv3 did not finish in 120 s")
    files = glob.glob(str(out / "**" / "*counter_collection.csv"), recursive=True)
    if not files:
        pytest.skip("rocprofv3 produced no counters (exit %d): %s" % (r.returncode, r.stderr[-300:]))
    per = {}
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                if not any(k in row["Kernel_Name"] for k in KERNELS):
                    continue
                d = per.setdefault(int(row["Dispatch_Id"]), {})
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    assert per, "no dispatch of the GEMM kernel was counted"
    return per


def counters(tmp_path, names, workload, tile=None):
    """Mean per-dispatch value of each counter for the GEMM kernel (dispatches after the first)."""
    per = per_dispatch(tmp_path, names, workload, tile)
    keys = sorted(per)[1:] if len(per) > 1 else sorted(per)
    return {n: sum(per[k].get(n, 0.0) for k in keys) / len(keys) for n in names}


def model_of(workload, tile=None, shape=None, with_plan=False):
    """gemm_model of the call bench.py makes for a workload (its buffers are dense
    torch allocations: 256-byte aligned stand-in addresses give the same plan)."""
    w = inputs.WORKLOADS[workload]
    M, N, K = shape or (w.M, w.N, w.K)
    dtype = tgemm.DTYPES[w.dtype]
    h = tgemm.gemm_create()
    try:
        if tile:
            tgemm.check(tgemm.gemm_set_tile(h, *tile))
        plan = tgemm.gemm_plan(h, M, N, K, 256, K, 256, N, 256, N, dtype)
    finally:
        tgemm.gemm_destroy(h)
    m = tgemm.gemm_model(plan, M, N, K, dtype)
    return (m, plan) if with_plan else m


MFMA = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16"]


@pytest.mark.parametrize("workload,tile", [("square128_f16", (16, 16, 32)), ("ragged1000x777x333_bf16", (64, 64, 64)),
                                           ("square4096_bf16", None)], ids=str)
def test_mfma_work_is_the_model(tmp_path, workload, tile):
    c = counters(tmp_path, MFMA, workload, tile)
    got = 512.0 * (c[MFMA[0]] + c[MFMA[1]])
    want = model_of(workload, tile)["executed_flops"]
    assert got == want, "MFMA flops %.6g, model %.6g" % (got, want)


def test_no_lds_bank_conflicts_on_the_256_tile(tmp_path):
    c = counters(tmp_path, ["SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"], "square4096_bf16")
    assert c["SQ_INSTS_LDS"] > 0
    assert c["SQ_LDS_BANK_CONFLICT"] == 0


def test_l2_requests_are_the_pages_traffic_count(tmp_path):
    """The load schedule requests exactly the no-reuse count of "Count the repeated
    reads": A read once per column tile, B once per row tile (M K ceil(N / tn) +
    K N ceil(M / tm) elements), as whole 128-byte lines from L2."""
    c = counters(tmp_path, ["TCP_TCC_READ_REQ_sum"], "square4096_bf16")
    m = model_of("square4096_bf16")
    assert 128.0 * c["TCP_TCC_READ_REQ_sum"] == m["bytes_a"] + m["bytes_b"]


def test_mfma_work_of_a_split_k_tail(tmp_path):
    """A plan with a split-K tail (4352 x 4096 x 1024: 16 full tile rows, then 16 tiles
    in 4 K-slices) runs two GEMM launches per call: their MFMA ops together equal the
    model's executed flops of the call."""
    shape = (4352, 4096, 1024)
    m, plan = model_of("square4096_bf16", shape=shape, with_plan=True)
    assert plan["tail_split_k"] > 1
    per = per_dispatch(tmp_path, MFMA, "square4096_bf16", shape=shape)
    calls = 4  # bench.py --warmup 1 --steps 3
    assert len(per) == 2 * calls
    got = 512.0 * sum(d.get(MFMA[0], 0.0) + d.get(MFMA[1], 0.0) for d in per.values()) / calls
    assert got == m["executed_flops"], "MFMA flops %.6g, model %.6g" % (got, m["executed_flops"])
