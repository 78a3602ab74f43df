"""GPU: handles are independent, and calls run on the stream they are given.

Each handle owns its split-K and operand-copy workspaces; the library keeps no other
state between calls. Two handles driven from two streams at once (plans that use the
workspaces: a forced split-K, a split-K tail, operand copies) must reproduce their
one-at-a-time results bit for bit (the kernels are deterministic), and the oracle. A
call enqueued on a non-default stream runs after the caller's earlier work on that
stream (here the writes of its inputs) and before later work (a copy of C).
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@pytest.fixture(scope="module")
def o():
    return oracle.get()


class Problem:
    """Device inputs and output of one product; ``ld_pad`` pads the leading dimensions."""

    def __init__(self, torch, M, N, K, seed, ld_pad=0):
        self.M, self.N, self.K = M, N, K
        self.a, self.b = inputs.random_case(M, N, K, "bf16", seed=seed)
        self.lda, self.ldb, self.ldc = K + ld_pad, N + ld_pad, N
        da = torch.zeros((M, self.lda), dtype=torch.int16, device="cuda")
        db = torch.zeros((K, self.ldb), dtype=torch.int16, device="cuda")
        da[:, :K] = torch.from_numpy(self.a.view(np.int16)).cuda()
        db[:, :N] = torch.from_numpy(self.b.view(np.int16)).cuda()
        self.da, self.db = da, db
        self.dc = torch.zeros((M, N), dtype=torch.int32, device="cuda")

    def run(self, h, stream):
        tgemm.check(tgemm.gemm_run(h, self.M, self.N, self.K, self.da.data_ptr(), self.lda, self.db.data_ptr(),
                                   self.ldb, self.dc.data_ptr(), self.ldc, tgemm.BF16_F32, stream.cuda_stream),
                    "gemm_run")

    def plan(self, h):
        return tgemm.gemm_plan(h, self.M, self.N, self.K, self.da.data_ptr(), self.lda, self.db.data_ptr(), self.ldb,
                               self.dc.data_ptr(), self.ldc, tgemm.BF16_F32)


def test_two_handles_on_two_streams(torch, o):
    h1, h2 = tgemm.gemm_create(), tgemm.gemm_create()
    try:
        tgemm.check(tgemm.gemm_set_split_k(h1, 3), "gemm_set_split_k")
        tgemm.check(tgemm.gemm_set_repack(h2, 1), "gemm_set_repack")  # copy operands whose rows are off 128 B
        p1 = Problem(torch, 96, 201, 3001, seed=11)  # forced split-K: workspace of h1
        p2 = Problem(torch, 4352, 4096, 1024, seed=12, ld_pad=1)  # split-K tail and operand copies: h2's
        assert p1.plan(h1)["split_k"] == 3
        q2 = p2.plan(h2)
        assert q2["tail_split_k"] > 1 and q2["repack"] == 3, q2
        default = torch.cuda.current_stream()
        p1.run(h1, default)
        p2.run(h2, default)
        torch.cuda.synchronize()
        ref1, ref2 = p1.dc.clone(), p2.dc.clone()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        for it in range(6):
            p1.dc.zero_()
            p2.dc.zero_()
            torch.cuda.synchronize()
            for _ in range(3):  # several calls in flight on each stream
                p2.run(h2, s2)
                p1.run(h1, s1)
            torch.cuda.synchronize()
            assert torch.equal(p1.dc, ref1), "handle 1 on its stream, iteration %d" % it
            assert torch.equal(p2.dc, ref2), "handle 2 on its stream, iteration %d" % it
    finally:
        tgemm.gemm_destroy(h1)
        tgemm.gemm_destroy(h2)
    G.compare(ref1.cpu().numpy(), o.gemm(p1.a, p1.b, "bf16", "f32").view(np.int32), "f32")
    rows, cols = inputs.sample_rows_cols(p2.M, p2.N, seed=3, block=256)
    G.compare(ref2[torch.from_numpy(rows).cuda()].cpu().numpy(),
              o.gemm_rows(p2.a, p2.b, rows, "bf16", "f32").view(np.int32), "f32")
    G.compare(ref2[:, torch.from_numpy(cols).cuda()].cpu().numpy(),
              o.gemm_cols(p2.a, p2.b, cols, "bf16", "f32").view(np.int32), "f32")


def test_call_is_ordered_on_its_stream(torch, o):
    """Inputs written on a side stream, the product enqueued on it without a host
    synchronization, and C copied out on it: the copy sees the product of the new inputs."""
    h = tgemm.gemm_create()
    try:
        M, N, K = 1000, 777, 333
        p = Problem(torch, M, N, K, seed=21)
        a2, b2 = inputs.random_case(M, N, K, "bf16", seed=22)
        ha = torch.from_numpy(a2.view(np.int16)).pin_memory()
        hb = torch.from_numpy(b2.view(np.int16)).pin_memory()
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            p.da[:, :K].copy_(ha, non_blocking=True)
            p.db[:, :N].copy_(hb, non_blocking=True)
            p.run(h, s)
            out = p.dc.clone()
        s.synchronize()
        G.compare(out.cpu().numpy(), o.gemm(a2, b2, "bf16", "f32").view(np.int32), "f32")
    finally:
        tgemm.gemm_destroy(h)
