"""gemm_tune: the fastest measured plan for a shape is kept in the handle and used by
later calls; results stay those of the oracle whatever plan is chosen."""
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


class Dev:
    """A, B, C on the device for a logical M x K and K x N product (row-major, dense)."""

    def __init__(self, a, b, dtype):
        self.M, self.K = a.shape
        self.N = b.shape[1]
        it = np.int16 if a.dtype == np.uint16 else np.int32
        self.a = torch.from_numpy(a.view(it)).cuda()
        self.b = torch.from_numpy(b.view(it)).cuda()
        ob = tgemm.OUT_BYTES[dtype]
        self.c = torch.zeros((self.M, self.N), dtype=G.int_dtype(ob), device="cuda")
        self.dtype = dtype

    def args(self):
        return (self.M, self.N, self.K, self.a.data_ptr(), self.K, self.b.data_ptr(), self.N, self.c.data_ptr(),
                self.N, self.dtype)

    def tune(self, h, iters=3):
        return tgemm.gemm_tune(h, tgemm.OP_N, tgemm.OP_N, *self.args(), torch.cuda.current_stream().cuda_stream, iters)

    def plan(self, h):
        return tgemm.gemm_plan(h, *self.args())

    def run(self, h):
        tgemm.check(tgemm.gemm_run(h, *self.args(), torch.cuda.current_stream().cuda_stream))

    def time_us(self, h, n=20):
        for _ in range(3):
            self.run(h)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            self.run(h)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n


KEYS = ("kernel", "tile_m", "tile_n", "tile_k", "split_k", "stages", "grid", "tail_split_k", "tail_m0", "repack")


@pytest.mark.parametrize("shape,dtype", [((200, 136, 1000), tgemm.BF16_F32), ((520, 264, 2000), tgemm.BF16_BF16),
                                         ((1000, 777, 333), tgemm.BF16_F32), ((96, 96, 96), tgemm.F16_F16),
                                         ((4352, 4096, 1024), tgemm.BF16_BF16)],  # automatic plan with a tail
                         ids=str)
def test_tuned_plan_used_and_correct(o, shape, dtype):
    M, N, K = shape
    a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=M + K)
    d = Dev(a, b, dtype)
    g = tgemm.Gemm()
    try:
        best = d.tune(g.h)
        torch.cuda.synchronize()
        ref = o.gemm(a, b, G.IN_KIND[dtype], G.OUT_KIND[dtype]).view(G.np_int(tgemm.OUT_BYTES[dtype]))
        G.compare(d.c.cpu().numpy(), ref, G.OUT_KIND[dtype])            # C holds the product after tuning
        assert {k: best[k] for k in KEYS} == {k: d.plan(g.h)[k] for k in KEYS}
        d.c.zero_()
        d.run(g.h)                                                       # the tuned plan, run again
        torch.cuda.synchronize()
        G.compare(d.c.cpu().numpy(), ref, G.OUT_KIND[dtype])
        fresh = tgemm.gemm_plan(None, *d.args())                          # other handles: the automatic plan
        assert fresh["kernel"] in (3, 4)
    finally:
        g.close()


def test_tuning_does_not_lose_to_the_automatic_plan(o):
    """A shape whose automatic tile count quantizes badly on 256 compute units."""
    M = N = K = 3072
    a, b = inputs.random_case(M, N, K, "bf16", seed=3)
    d = Dev(a, b, tgemm.BF16_BF16)
    g = tgemm.Gemm()
    try:
        auto = d.plan(g.h)
        t_auto = d.time_us(g.h)
        best = d.tune(g.h, iters=5)
        t_best = d.time_us(g.h)
        print("3072^3 automatic %s %.1f us, tuned %s %.1f us" % (
            (auto["tile_m"], auto["tile_n"], auto["split_k"], auto["stages"]), t_auto,
            (best["tile_m"], best["tile_n"], best["split_k"], best["stages"]), t_best))
        assert t_best <= 1.15 * t_auto
        rows, cols = inputs.sample_rows_cols(M, N, seed=5, block=512)
        c = d.c.cpu().numpy()
        G.compare(c[rows], o.gemm_rows(a, b, rows, "bf16", "bf16").view(np.int16), "bf16")
        G.compare(c[:, cols], o.gemm_cols(a, b, cols, "bf16", "bf16").view(np.int16), "bf16")
    finally:
        g.close()


def test_forced_settings_win_and_nothing_to_tune():
    a, b = inputs.random_case(256, 256, 512, "bf16", seed=4)
    d = Dev(a, b, tgemm.BF16_F32)
    g = tgemm.Gemm()
    try:
        g.set_tile(64, 64, 64)
        p = d.tune(g.h)
        assert (p["tile_m"], p["tile_n"]) == (64, 64)
        g.set_tile(0, 0, 0)
        g.set_split_k(3)
        assert d.tune(g.h)["split_k"] == 3
        g.set_split_k(0)
        ai, bi = inputs.random_case(64, 64, 64, "i32", seed=5)
        di = Dev(ai, bi, tgemm.I32_I32)
        assert di.tune(g.h)["kernel_name"] == "int32_valu"
        with pytest.raises(tgemm.GemmError):
            d.tune(g.h, iters=0)
    finally:
        g.close()


@pytest.mark.parametrize("shape", [(1024, 1024, 1000), (520, 1000, 1032)], ids=str)
def test_tuning_tries_operand_copies(o, shape):
    """Rows off cache lines (lda = K = 1000, or ldb = N = 1000): the tuner also times
    the plans with those operands copied into aligned rows; whichever it keeps, the
    result is the oracle's, and copies only ever cover a misaligned operand."""
    M, N, K = shape
    misaligned = (1 if (2 * K) % 128 else 0) | (2 if (2 * N) % 128 else 0)
    a, b = inputs.random_case(M, N, K, "bf16", seed=M + N)
    d = Dev(a, b, tgemm.BF16_F32)
    g = tgemm.Gemm()
    try:
        best = d.tune(g.h)
        assert best["kernel"] == 4 and best["repack"] & ~misaligned == 0, best
        assert {k: best[k] for k in KEYS} == {k: d.plan(g.h)[k] for k in KEYS}
        print("%s: tuned plan tile %dx%d split %d stages %d repack %d" % (
            shape, best["tile_m"], best["tile_n"], best["split_k"], best["stages"], best["repack"]), flush=True)
        d.c.zero_()
        d.run(g.h)
        torch.cuda.synchronize()
        ref = o.gemm(a, b, "bf16", "f32").view(np.int32)
        G.compare(d.c.cpu().numpy(), ref, "f32")
        # a handle that forbids copies tunes without them
        tgemm.check(tgemm.gemm_set_repack(g.h, -1), "gemm_set_repack")
        assert d.tune(g.h)["repack"] == 0
    finally:
        g.close()
