"""The library's launches captured in a HIP graph: every replay gives the eager result.

gemm_run only enqueues kernels on the caller's stream (no allocation once a split-K
workspace exists, no memset), so a caller may capture it. Each case runs eagerly
first (which also sizes any workspace), captures the same call, and replays the graph
several times with eager work of the program in between (clearing C, another product
on the same handle, host synchronisations); every replay must reproduce the eager
bytes exactly, and the eager result must meet the accuracy rule against the oracle.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def o():
    return oracle.get()


# (M, N, K, dtype, forced tile or None, forced K-slices, operand-copy mode): the automatic
# 256x256 plan, a ragged edge-tile plan, split-K with its reduction kernel, a split-K tail
# after the full rounds (three kernels), the one-wave 16x16x32 tile, the int32 path, and
# plans that first copy A into aligned rows (alone, and before a split-K tail).
CASES = [
    (512, 512, 1024, tgemm.BF16_BF16, None, 0, 0),
    (4352, 4096, 1024, tgemm.BF16_BF16, None, 0, 0),
    (1000, 777, 333, tgemm.BF16_F32, (64, 64, 64), 0, 0),
    (128, 2048, 4096, tgemm.BF16_F32, None, 4, 0),
    (128, 128, 128, tgemm.F16_F32, (16, 16, 32), 0, 0),
    (96, 80, 70, tgemm.I32_I32, None, 0, 0),
    (1000, 1024, 1000, tgemm.BF16_BF16, None, 0, 1),
    (4352, 4096, 1000, tgemm.BF16_F32, None, 0, 1),
]


def _inputs(M, N, K, dtype, seed):
    return inputs.random_case(M, N, K, G.IN_KIND[dtype], seed)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%d-d%d" % c[:4])
def test_graph_replays_match_eager(o, case):
    M, N, K, dtype, tile, splits, repack = case
    print("graph case M=%d N=%d K=%d dtype=%d tile=%s split_k=%d repack=%d" % (M, N, K, dtype, tile, splits, repack),
          flush=True)
    a, b = _inputs(M, N, K, dtype, 7 + M)
    it = np.int32 if dtype == tgemm.I32_I32 else np.int16
    da, db = torch.from_numpy(a.view(it)).cuda(), torch.from_numpy(b.view(it)).cuda()
    ob = tgemm.OUT_BYTES[dtype]
    dc = torch.zeros((M, N), dtype=G.int_dtype(ob), device="cuda")
    h = tgemm.gemm_create()
    try:
        if tile:
            tgemm.check(tgemm.gemm_set_tile(h, *tile))
        tgemm.check(tgemm.gemm_set_split_k(h, splits))
        tgemm.check(tgemm.gemm_set_repack(h, repack))
        if repack:
            p = tgemm.gemm_plan(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N, dtype)
            assert p["repack"] & 1, p  # A (rows of K elements, not a multiple of 64) is copied
            assert M < 4352 or p["tail_split_k"] > 1, p  # and the larger case ends with a split-K tail

        def call(stream):
            tgemm.check(tgemm.gemm_run(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N, dtype, stream))

        call(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        eager = dc.cpu().numpy().copy()
        G.compare(eager, o.gemm(a, b, G.IN_KIND[dtype], G.OUT_KIND[dtype]), G.OUT_KIND[dtype])

        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call(torch.cuda.current_stream().cuda_stream)
        # a second product on the same handle between replays (eager work of the program)
        xa = torch.from_numpy(_inputs(64, 64, 64, dtype, 99)[0].view(it)).cuda()
        xc = torch.zeros((64, 64), dtype=G.int_dtype(ob), device="cuda")
        for r in range(4):
            dc.zero_()
            tgemm.check(tgemm.gemm_run(h, 64, 64, 64, xa.data_ptr(), 64, xa.data_ptr(), 64, xc.data_ptr(), 64, dtype,
                                       torch.cuda.current_stream().cuda_stream))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = dc.cpu().numpy()
            assert np.array_equal(got, eager), "replay %d differs from the eager result" % r
    finally:
        tgemm.gemm_destroy(h)


def test_graph_replay_after_workspace_growth(o):
    """A captured split-K call keeps the workspace it was captured with: a later eager
    call on the same handle that needs a larger one gets a new buffer (the old one is
    kept until gemm_destroy), so every replay still reproduces the eager result."""
    dtype = tgemm.BF16_F32
    (Ms, Ns, Ks), (Mb, Nb, Kb) = (128, 2048, 4096), (128, 8192, 8192)  # 4 and 16 MiB of fp32 partial tiles
    a, b = _inputs(Ms, Ns, Ks, dtype, 5)
    xa, xb = _inputs(Mb, Nb, Kb, dtype, 6)
    da, db = torch.from_numpy(a.view(np.int16)).cuda(), torch.from_numpy(b.view(np.int16)).cuda()
    dxa, dxb = torch.from_numpy(xa.view(np.int16)).cuda(), torch.from_numpy(xb.view(np.int16)).cuda()
    dc = torch.zeros((Ms, Ns), dtype=torch.int32, device="cuda")
    dxc = torch.zeros((Mb, Nb), dtype=torch.int32, device="cuda")
    h = tgemm.gemm_create()
    try:
        tgemm.check(tgemm.gemm_set_split_k(h, 4))

        def small(stream):
            tgemm.check(tgemm.gemm_run(h, Ms, Ns, Ks, da.data_ptr(), Ks, db.data_ptr(), Ns, dc.data_ptr(), Ns, dtype,
                                       stream))

        small(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        eager = dc.cpu().numpy().copy()
        G.compare(eager, o.gemm(a, b, "bf16", "f32").view(np.int32), "f32")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            small(torch.cuda.current_stream().cuda_stream)
        for r in range(3):
            # needs a larger workspace than the captured call's
            tgemm.check(tgemm.gemm_run(h, Mb, Nb, Kb, dxa.data_ptr(), Kb, dxb.data_ptr(), Nb, dxc.data_ptr(), Nb,
                                       dtype, torch.cuda.current_stream().cuda_stream))
            dc.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(dc.cpu().numpy(), eager), "replay %d differs from the eager result" % r
        G.compare(dxc.cpu().numpy(), o.gemm(xa, xb, "bf16", "f32").view(np.int32), "f32")
    finally:
        tgemm.gemm_destroy(h)
