"""gemm_run_op_noalloc: the C entry point that allocates nothing, against gemm_run_op.

The allocation-free call keeps split-K partial tiles in a fixed scratch array of
32 MiB per GPU instead of the handle's workspace. Its results must be those of
gemm_run_op for the same arguments -- bit for bit where both run the same kernels,
else to the accuracy rule against the oracle -- on calls in a row whose second input
is smaller (the scratch keeps the first call's partial tiles), and it must not
allocate device memory: a fresh handle's first split-K call leaves the free device
memory unchanged, and can be captured into a HIP graph with no call before it.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SCRATCH = 32 << 20


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def both(h, M, N, K, da, db, dtype, lda=None, ldb=None):
    """C from gemm_run_op and from gemm_run_op_noalloc (same handle, same stream)."""
    ob = tgemm.OUT_BYTES[dtype]
    lda, ldb = lda or K, ldb or N
    s = torch.cuda.current_stream().cuda_stream
    c_ref = torch.full((M, N), -1, dtype=G.int_dtype(ob), device="cuda")
    c_new = torch.full((M, N), -1, dtype=G.int_dtype(ob), device="cuda")
    tgemm.check(tgemm.gemm_run_op(h, tgemm.OP_N, tgemm.OP_N, M, N, K, da.data_ptr(), lda, db.data_ptr(), ldb,
                                  c_ref.data_ptr(), N, dtype, s), "gemm_run_op")
    tgemm.check(tgemm.gemm_run_op_noalloc(h, tgemm.OP_N, tgemm.OP_N, M, N, K, da.data_ptr(), lda, db.data_ptr(), ldb,
                                          c_new.data_ptr(), N, dtype, s), "gemm_run_op_noalloc")
    torch.cuda.synchronize()
    return c_ref.cpu().numpy(), c_new.cpu().numpy()


def test_two_calls_in_a_row_match_gemm_run_op(o):
    """Split-K products (partial tiles in the scratch array), the second one smaller,
    then a product that needs no scratch: bit-identical to gemm_run_op (same plan,
    same kernels) and within the accuracy rule of the oracle."""
    h = tgemm.gemm_create()
    try:
        for M, N, K, dtype in [(128, 8192, 8192, tgemm.BF16_F32), (64, 4096, 4096, tgemm.BF16_F32),
                               (1000, 777, 333, tgemm.BF16_BF16)]:
            print("noalloc case M=%d N=%d K=%d dtype=%d" % (M, N, K, dtype), flush=True)
            p = tgemm.gemm_plan(h, M, N, K, 1 << 20, K, 1 << 30, N, 1 << 34, N, dtype)
            if K >= 4096:
                assert p["split_k"] > 1 and p["split_k"] * M * N * 4 <= SCRATCH, p
            a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=M + K)
            ref, new = both(h, M, N, K, dev16(a), dev16(b), dtype)
            assert np.array_equal(new, ref)
            G.compare(new, o.gemm(a, b, G.IN_KIND[dtype], G.OUT_KIND[dtype]).view(G.np_int(tgemm.OUT_BYTES[dtype])),
                      G.OUT_KIND[dtype])
    finally:
        tgemm.gemm_destroy(h)


def test_tall_product_a_three_steps_ahead(o):
    """A tall, narrow product (the 256x256 tile with A loaded three K-steps ahead,
    ragged K): bit-identical to gemm_run_op, and the oracle's result on sampled rows."""
    h = tgemm.gemm_create()
    try:
        M, N, K, dtype = 16384, 1024, 200, tgemm.BF16_BF16
        p = tgemm.gemm_plan(h, M, N, K, 1 << 20, K, 1 << 30, N, 1 << 34, N, dtype)
        assert (p["tile_m"], p["split_k"], p["stages"]) == (256, 1, 3), p
        a, b = inputs.random_case(M, N, K, "bf16", seed=7)
        ref, new = both(h, M, N, K, dev16(a), dev16(b), dtype)
        assert np.array_equal(new, ref)
        rows, _ = inputs.sample_rows_cols(M, N, seed=7, block=256)
        G.compare(new[rows], o.gemm_rows(a, b, rows, "bf16", "bf16").view(np.int16), "bf16")
    finally:
        tgemm.gemm_destroy(h)


def test_split_k_tail_and_operand_copies(o):
    """A plan with a split-K tail whose partial tiles fit (run as gemm_run_op runs it)
    and a plan that copies A into aligned rows (not done here: the kernels read the
    unaligned rows, with the same sums in the same order): bit-identical results."""
    h = tgemm.gemm_create()
    try:
        M, N, K, dtype = 4352, 4096, 1024, tgemm.BF16_F32
        p = tgemm.gemm_plan(h, M, N, K, 1 << 20, K, 1 << 30, N, 1 << 34, N, dtype)
        assert p["tail_split_k"] > 1 and p["tail_split_k"] * (M - p["tail_m0"]) * N * 4 <= SCRATCH, p
        a, b = inputs.random_case(M, N, K, "bf16", seed=3)
        ref, new = both(h, M, N, K, dev16(a), dev16(b), dtype)
        assert np.array_equal(new, ref)
        rows = np.array([0, 1, 2047, 4095, 4096, 4200, M - 1], dtype=np.int64)
        G.compare(new[rows], o.gemm_rows(a, b, rows, "bf16", "f32").view(np.int32), "f32")

        M, N, K, dtype = 1000, 1024, 1000, tgemm.BF16_BF16
        tgemm.check(tgemm.gemm_set_repack(h, 1))
        a, b = inputs.random_case(M, N, K, "bf16", seed=4)
        da, db = dev16(a), dev16(b)
        p = tgemm.gemm_plan(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, 1 << 34, N, dtype)
        assert p["repack"] & 1, p
        ref, new = both(h, M, N, K, da, db, dtype)
        assert np.array_equal(new, ref)
    finally:
        tgemm.gemm_destroy(h)


def test_scratch_too_small_is_refused():
    """A call whose split-K partial tiles exceed the scratch array is refused before
    anything is enqueued: C keeps its contents."""
    h = tgemm.gemm_create()
    try:
        M, N, K = 1024, 1024, 4096
        tgemm.check(tgemm.gemm_set_split_k(h, 16))  # 16 x 1024 x 1024 x 4 bytes = 64 MiB
        a, b = inputs.random_case(M, N, K, "bf16", seed=5)
        da, db = dev16(a), dev16(b)
        c = torch.full((M, N), 0x1234, dtype=torch.int32, device="cuda")
        st = tgemm.gemm_run_op_noalloc(h, tgemm.OP_N, tgemm.OP_N, M, N, K, da.data_ptr(), K, db.data_ptr(), N,
                                       c.data_ptr(), N, tgemm.BF16_F32, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert st == tgemm.ERR_SCRATCH_TOO_SMALL, tgemm.gemm_status_string(st)
        assert "scratch" in tgemm.gemm_status_string(st)
        assert bool((c == 0x1234).all().item())
    finally:
        tgemm.gemm_destroy(h)


def test_no_device_allocation_and_graph_capture(o):
    """On a fresh handle the first split-K call allocates nothing (free device memory
    unchanged, while gemm_run_op's first split-K call takes its 16 MiB workspace), and
    the call can be captured into a HIP graph without any call before it; replays
    reproduce gemm_run_op's result."""
    M, N, K, dtype = 128, 8192, 8192, tgemm.BF16_F32
    a, b = inputs.random_case(M, N, K, "bf16", seed=6)
    da, db = dev16(a), dev16(b)
    c = torch.zeros((M, N), dtype=torch.int32, device="cuda")
    c_ref = torch.zeros((M, N), dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    h = tgemm.gemm_create()
    try:
        free0 = torch.cuda.mem_get_info()[0]
        tgemm.check(tgemm.gemm_run_op_noalloc(h, tgemm.OP_N, tgemm.OP_N, M, N, K, da.data_ptr(), K, db.data_ptr(), N,
                                              c.data_ptr(), N, dtype, s))
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        tgemm.check(tgemm.gemm_run_op(h, tgemm.OP_N, tgemm.OP_N, M, N, K, da.data_ptr(), K, db.data_ptr(), N,
                                      c_ref.data_ptr(), N, dtype, s))
        torch.cuda.synchronize()
        free2 = torch.cuda.mem_get_info()[0]
        print("free device memory: %d, after noalloc %d, after gemm_run_op %d" % (free0, free1, free2), flush=True)
        assert free0 - free1 < (4 << 20)
        assert free1 - free2 >= (16 << 20)  # the measure sees the workspace gemm_run_op allocates
        assert np.array_equal(c.cpu().numpy(), c_ref.cpu().numpy())
    finally:
        tgemm.gemm_destroy(h)

    h = tgemm.gemm_create()  # fresh: no workspace, nothing run before the capture
    try:
        c.zero_()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            tgemm.check(tgemm.gemm_run_op_noalloc(h, tgemm.OP_N, tgemm.OP_N, M, N, K, da.data_ptr(), K, db.data_ptr(),
                                                  N, c.data_ptr(), N, dtype, torch.cuda.current_stream().cuda_stream))
        want = c_ref.cpu().numpy()
        for r in range(3):
            c.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(c.cpu().numpy(), want), "replay %d" % r
        G.compare(want, o.gemm(a, b, "bf16", "f32").view(np.int32), "f32")
    finally:
        tgemm.gemm_destroy(h)
