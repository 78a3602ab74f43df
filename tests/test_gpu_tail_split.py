"""GPU parity of plans with a split-K tail.

When an automatic 256x256 plan has more than one round of tiles and its last round is
only partly full, the tile rows that fill whole rounds run first and the remaining
rows run as a second launch with each tile's K range cut into S slices, summed in
slice order by the reduction kernel. Both parts must give the oracle's result (bit
for bit on integer-valued inputs, whose fp32 sums are exact in any order); rows
before the tail come from the same kernel over the same K order as the plain plan,
so they must equal a forced-tile (no tail) run bit for bit.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu

N_, T_ = tgemm.OP_N, tgemm.OP_T


@pytest.fixture(scope="module")
def h():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = tgemm.gemm_create()
    yield g
    tgemm.gemm_destroy(g)


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def tail_plan(h, M, N, K, ops, dtype):
    lda = M if ops[0] == T_ else K
    ldb = K if ops[1] == T_ else N
    return tgemm.gemm_plan_op(h, ops[0], ops[1], M, N, K, 1 << 20, lda, 1 << 30, ldb, 1 << 34, N, dtype)


@pytest.mark.parametrize("ops", [(N_, N_), (T_, T_), (N_, T_)], ids=["NN", "TT", "NT"])
@pytest.mark.parametrize("shape", [(4352, 4096, 1024), (4608, 4096, 2048)], ids=str)
def test_tail_split_full_output(h, o, shape, ops):
    M, N, K = shape
    for n, dtype in enumerate([tgemm.BF16_F32, tgemm.F16_F16]):
        p = tail_plan(h, M, N, K, ops, dtype)
        assert p["tail_split_k"] > 1 and p["tail_m0"] > 0, p
        a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=M + K + n)
        print("tail split case %s %s dtype %d plan tail_m0 %d S %d" % (shape, ops, dtype, p["tail_m0"],
                                                                       p["tail_split_k"]), flush=True)
        c, dc = G.run(h, a, b, dtype, op_a=ops[0], op_b=ops[1])
        assert dc.untouched_outside()
        ref = o.gemm(a, b, G.IN_KIND[dtype], G.OUT_KIND[dtype]).view(G.np_int(tgemm.OUT_BYTES[dtype]))
        G.compare(c, ref, G.OUT_KIND[dtype])


def test_tail_split_integer_inputs_and_rows_before_the_tail(h, o):
    """Integer-valued inputs: exact. Float inputs: the rows before the tail equal a
    forced 256x256 run (one launch, no tail) bit for bit; the tail rows agree with it
    to the accuracy rule."""
    M, N, K = 4352, 4096, 1024
    p = tail_plan(h, M, N, K, (N_, N_), tgemm.BF16_F32)
    m0 = p["tail_m0"]
    assert p["tail_split_k"] > 1 and m0 == 4096
    a = inputs.draw((M, K), "small_int", "bf16", 81)
    b = inputs.draw((K, N), "small_int", "bf16", 82)
    c, _ = G.run(h, a, b, tgemm.BF16_F32)
    assert np.array_equal(c, o.gemm(a, b, "bf16", "f32").view(np.int32))
    a, b = inputs.random_case(M, N, K, "bf16", seed=83)
    c, _ = G.run(h, a, b, tgemm.BF16_F32)
    tgemm.check(tgemm.gemm_set_tile(h, 256, 256, 64), "gemm_set_tile")
    try:
        assert tail_plan(h, M, N, K, (N_, N_), tgemm.BF16_F32)["tail_split_k"] == 0  # forced tile: no tail
        c_plain, _ = G.run(h, a, b, tgemm.BF16_F32)
    finally:
        tgemm.gemm_set_tile(h, 0, 0, 0)
    assert np.array_equal(c[:m0], c_plain[:m0])
    G.compare(c[m0:], c_plain[m0:], "f32")


@pytest.mark.parametrize("shape", [(6000, 6000, 6000), (7000, 7000, 7000), (8193, 8193, 8193)], ids=str)
def test_tail_split_large_sampled(h, o, shape):
    """Large products whose last round is partly full, compared on sampled rows and
    columns (one per 256 plus the first and last: every tail tile row is sampled)."""
    import torch

    M, N, K = shape
    p = tail_plan(h, M, N, K, (N_, N_), tgemm.BF16_BF16)
    assert p["tail_split_k"] > 1, p
    a, b = inputs.random_case(M, N, K, "bf16", seed=M + 1)
    print("tail split large %s tail_m0 %d S %d" % (shape, p["tail_m0"], p["tail_split_k"]), flush=True)
    da = torch.from_numpy(a.view(np.int16)).cuda()
    db = torch.from_numpy(b.view(np.int16)).cuda()
    dc = torch.full((M, N), G.SENTINEL[2], dtype=torch.int16, device="cuda")
    tgemm.check(tgemm.gemm_run(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N, tgemm.BF16_BF16,
                               torch.cuda.current_stream().cuda_stream), "gemm_run")
    torch.cuda.synchronize()
    rows, cols = inputs.sample_rows_cols(M, N, seed=9, block=256)
    assert np.any(rows >= p["tail_m0"])
    got_r = dc[torch.from_numpy(rows).cuda()].cpu().numpy()
    got_c = dc[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    G.compare(got_r, o.gemm_rows(a, b, rows, "bf16", "bf16").view(np.int16), "bf16")
    G.compare(got_c, o.gemm_cols(a, b, cols, "bf16", "bf16").view(np.int16), "bf16")


def test_tail_split_tall_a_deep(h, o):
    """A tall, narrow product whose full rounds and split-K tail both run the 256x256
    tile with A loaded three K-steps ahead: integer-valued inputs exact on sampled rows
    (every tail row among them) and columns; float inputs give the rows before the
    tail bit for bit as a forced-tile run (one launch, no tail)."""
    import torch

    M, N, K = 17408, 1024, 2048
    p = tail_plan(h, M, N, K, (N_, N_), tgemm.BF16_F32)
    m0 = p["tail_m0"]
    assert (p["stages"], p["tail_split_k"] > 1, m0) == (3, True, 16384), p
    rows, cols = inputs.sample_rows_cols(M, N, seed=11, block=256)
    rows = np.unique(np.concatenate([rows, np.arange(m0, M, 97, dtype=rows.dtype), [M - 1]]))

    def run(a, b):
        da = torch.from_numpy(a.view(np.int16)).cuda()
        db = torch.from_numpy(b.view(np.int16)).cuda()
        dc = torch.full((M, N), G.SENTINEL[4], dtype=torch.int32, device="cuda")
        tgemm.check(tgemm.gemm_run(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N,
                                   tgemm.BF16_F32, torch.cuda.current_stream().cuda_stream), "gemm_run")
        torch.cuda.synchronize()
        return dc

    a = inputs.draw((M, K), "small_int", "bf16", 91)
    b = inputs.draw((K, N), "small_int", "bf16", 92)
    print("tall a-deep tail: tail_m0 %d S %d, integer inputs" % (m0, p["tail_split_k"]), flush=True)
    dc = run(a, b)
    assert np.array_equal(dc[torch.from_numpy(rows).cuda()].cpu().numpy(), o.gemm_rows(a, b, rows, "bf16", "f32").view(np.int32))
    assert np.array_equal(dc[:, torch.from_numpy(cols).cuda()].cpu().numpy(), o.gemm_cols(a, b, cols, "bf16", "f32").view(np.int32))
    a, b = inputs.random_case(M, N, K, "bf16", seed=93)
    c = run(a, b).cpu().numpy()
    G.compare(c[rows], o.gemm_rows(a, b, rows, "bf16", "f32").view(np.int32), "f32")
    tgemm.check(tgemm.gemm_set_tile(h, 256, 256, 64), "gemm_set_tile")
    try:
        q = tail_plan(h, M, N, K, (N_, N_), tgemm.BF16_F32)
        assert (q["tail_split_k"], q["stages"]) == (0, 3), q  # forced tile: no tail, same pipeline
        c_plain = run(a, b).cpu().numpy()
    finally:
        tgemm.gemm_set_tile(h, 0, 0, 0)
    assert np.array_equal(c[:m0], c_plain[:m0])


def tail_cases():
    """Tile counts of one or two full rounds plus a few tiles (ragged last tiles),
    random K, leading-dimension padding and operand forms."""
    rng = np.random.default_rng(4242)
    out = []
    for tm, tn in [(17, 16), (18, 16), (9, 32), (20, 13), (33, 8), (25, 21)]:
        M = 256 * (tm - 1) + int(rng.integers(1, 257))
        N = 256 * (tn - 1) + int(rng.integers(1, 257))
        K = int(rng.integers(1000, 3000))
        pad = int(rng.choice([0, 1, 8, 37]))
        ops = [(N_, N_), (T_, N_), (N_, T_), (T_, T_)][int(rng.integers(0, 4))]
        out.append((M, N, K, pad, ops))
    return out


@pytest.mark.parametrize("case", tail_cases(), ids=str)
def test_tail_and_copies_random(h, o, case):
    """Random shapes past one round of 256x256 tiles, with padded leading dimensions
    and transposed forms: whatever tail and operand copies the plan picks, the sampled
    rows and columns match the oracle and nothing outside C is written."""
    import torch

    M, N, K, pad, ops = case
    a, b = inputs.random_case(M, N, K, "bf16", seed=M + N + K)
    lda = (M if ops[0] == T_ else K) + pad
    ldb = (K if ops[1] == T_ else N) + pad
    sa = np.ascontiguousarray(a.T) if ops[0] == T_ else a
    sb = np.ascontiguousarray(b.T) if ops[1] == T_ else b
    da = G.DevMatrix(sa, sa.shape[0], sa.shape[1], lda, 0, 2, fill=G.SENTINEL[2])
    db = G.DevMatrix(sb, sb.shape[0], sb.shape[1], ldb, 0, 2, fill=G.SENTINEL[2])
    dc = G.DevMatrix(None, M, N, N + pad, 0, 2)
    p = tgemm.gemm_plan_op(h, ops[0], ops[1], M, N, K, da.ptr, da.ld, db.ptr, db.ld, dc.ptr, dc.ld, tgemm.BF16_BF16)
    print("tail/copies random %s plan tail %d m0 %d repack %d" % (case, p["tail_split_k"], p["tail_m0"], p["repack"]),
          flush=True)
    tgemm.check(tgemm.gemm_run_op(h, ops[0], ops[1], M, N, K, da.ptr, da.ld, db.ptr, db.ld, dc.ptr, dc.ld,
                                  tgemm.BF16_BF16, torch.cuda.current_stream().cuda_stream), "gemm_run_op")
    torch.cuda.synchronize()
    assert dc.untouched_outside()
    c = dc.host()
    rows, cols = inputs.sample_rows_cols(M, N, seed=M, block=256)
    G.compare(c[rows], o.gemm_rows(a, b, rows, "bf16", "bf16").view(np.int16), "bf16")
    G.compare(c[:, cols], o.gemm_cols(a, b, cols, "bf16", "bf16").view(np.int16), "bf16")
