"""GPU parity at operand sizes past 32-bit byte offsets (the largest sizes).

Every dimension fits int32 (the host rejects more), but an operand can still span
many GiB: tile origins are 64-bit addresses, and a buffer range is clamped at 2 GiB.
An offset that wrapped at 2^31 or 2^32 bytes would read a row that far away. Here the
large operand (5 GiB and more) is a block of 251 seeded rows repeated along its rows:
251 is prime, so rows 2^31 or 2^32 bytes apart hold different data, and sampled outputs
(one row or column per 256 plus the first and last) are compared with the oracle,
computed from the block on the host. A leading dimension too large for one buffer range
per tile is also covered: then the plan must name the element loader, and the result
must not change.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu

N_, T_ = tgemm.OP_N, tgemm.OP_T
PERIOD = 251


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@pytest.fixture(scope="module")
def h(torch):
    g = tgemm.gemm_create()
    yield g
    tgemm.gemm_destroy(g)


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def repeat_rows(torch, block, rows):
    """Device matrix of ``rows`` rows: row r is block[r % len(block)]."""
    d = torch.from_numpy(block.view(np.int16)).cuda()
    reps = -(-rows // block.shape[0])
    return d.repeat(reps, 1)[:rows].contiguous()


def run(torch, h, ops, M, N, K, A, lda, B, ldb, dtype, tile=None):
    tgemm.check(tgemm.gemm_set_tile(h, *(tile or (0, 0, 0))), "gemm_set_tile")
    try:
        p = tgemm.gemm_plan_op(h, ops[0], ops[1], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, 1 << 20, N, dtype)
        ob = tgemm.OUT_BYTES[dtype]
        C = torch.full((M, N), G.SENTINEL[ob], dtype=G.int_dtype(ob), device="cuda")
        print("large case %s %s lda %d ldb %d tile %s plan %s" % ((M, N, K), ops, lda, ldb, tile,
                                                                   {k: p[k] for k in ("tile_m", "tile_n", "vector_loads",
                                                                                      "split_k")}), flush=True)
        st = tgemm.gemm_run_op(h, ops[0], ops[1], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), N,
                               dtype, torch.cuda.current_stream().cuda_stream)
        tgemm.check(st, "gemm_run_op")
        torch.cuda.synchronize()
    finally:
        tgemm.gemm_set_tile(h, 0, 0, 0)
    return p, C


@pytest.mark.parametrize("tile", [None, (256, 256, 64)], ids=str)
def test_a_beyond_4gib(torch, h, o, tile):
    """A is 40000 x 65536 bf16 (5.2 GB), stored as given (K-contiguous rows)."""
    M, N, K = 40000, 64, 65536
    block = inputs.draw((PERIOD, K), "normal", "bf16", 11)
    b = inputs.draw((K, N), "normal", "bf16", 12)
    A = repeat_rows(torch, block, M)
    B = torch.from_numpy(b.view(np.int16)).cuda()
    p, C = run(torch, h, (N_, N_), M, N, K, A, K, B, N, tgemm.BF16_F32, tile)
    assert p["vector_loads"] == 1
    del A
    rows, _ = inputs.sample_rows_cols(M, N, seed=13, block=256)
    got = C[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = o.gemm_rows(block[rows % PERIOD], b, np.arange(len(rows)), "bf16", "f32")
    G.compare(got, ref.view(np.int32), "f32")


def test_transposed_a_beyond_4gib(torch, h, o):
    """A supplied transposed: stored K x M = 65536 x 40000 bf16 (5.2 GB), M-contiguous."""
    M, N, K = 40000, 64, 65536
    block_t = inputs.draw((PERIOD, M), "normal", "bf16", 21)  # stored row k = block_t[k % PERIOD]
    b = inputs.draw((K, N), "normal", "bf16", 22)
    At = repeat_rows(torch, block_t, K)
    B = torch.from_numpy(b.view(np.int16)).cuda()
    p, C = run(torch, h, (T_, N_), M, N, K, At, M, B, N, tgemm.BF16_F32)
    assert p["vector_loads"] == 1
    del At
    rows, _ = inputs.sample_rows_cols(M, N, seed=23, block=256)
    # logical A[m][k] = stored[k][m] = block_t[k % PERIOD][m]
    a_sub = np.ascontiguousarray(np.tile(block_t[:, rows].T, (1, -(-K // PERIOD)))[:, :K])
    got = C[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = o.gemm_rows(a_sub, b, np.arange(len(rows)), "bf16", "f32")
    G.compare(got, ref.view(np.int32), "f32")


def test_transposed_b_beyond_4gib(torch, h, o):
    """B supplied transposed: stored N x K = 40000 x 65536 bf16 (5.2 GB); C's columns sampled."""
    M, N, K = 64, 40000, 65536
    a = inputs.draw((M, K), "normal", "bf16", 31)
    block = inputs.draw((PERIOD, K), "normal", "bf16", 32)  # stored row n = block[n % PERIOD]
    A = torch.from_numpy(a.view(np.int16)).cuda()
    Bt = repeat_rows(torch, block, N)
    p, C = run(torch, h, (N_, T_), M, N, K, A, K, Bt, K, tgemm.BF16_BF16)
    assert p["vector_loads"] == 1
    del Bt
    _, cols = inputs.sample_rows_cols(M, N, seed=33, block=256)
    got = C[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    b_sub = np.ascontiguousarray(block[cols % PERIOD].T)  # K x len(cols)
    ref = o.gemm_cols(a, b_sub, np.arange(len(cols)), "bf16", "bf16")
    G.compare(got, ref.view(np.int16), "bf16")


def test_int32_beyond_4gib(torch, h, o):
    """int32 A of 20000 x 65536 (5.2 GB): the VALU path's 64-bit strides; bit-exact."""
    M, N, K = 20000, 8, 65536
    rng = np.random.default_rng(41)
    block = rng.integers(-(2**31), 2**31, size=(PERIOD, K), dtype=np.int64).astype(np.int32)
    b = rng.integers(-(2**31), 2**31, size=(K, N), dtype=np.int64).astype(np.int32)
    dblock = torch.from_numpy(block).cuda()
    A = dblock.repeat(-(-M // PERIOD), 1)[:M].contiguous()
    B = torch.from_numpy(b).cuda()
    p, C = run(torch, h, (N_, N_), M, N, K, A, K, B, N, tgemm.I32_I32)
    del A
    rows, _ = inputs.sample_rows_cols(M, N, seed=43, block=256)
    got = C[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.int32)
    ref = o.gemm_rows(block[rows % PERIOD], b, np.arange(len(rows)), "i32", "i32")
    assert np.array_equal(got, ref.view(np.int32))


@pytest.mark.parametrize("tile,vec", [((256, 256, 64), 0), ((64, 64, 64), 1)], ids=str)
def test_leading_dimension_beyond_buffer_range(torch, h, o, tile, vec):
    """lda = 2^22 + 2^16 elements: 255 rows of it span more than one 2 GiB buffer
    range, so a 256-row tile takes the element loader and a 64-row tile the direct
    loads; the 5.1 GB buffer around the 600 x 64 matrix holds NaN."""
    M, N, K = 600, 96, 64
    lda = (1 << 22) + (1 << 16)
    a, b = inputs.random_case(M, N, K, "bf16", seed=51)
    buf = torch.full(((M - 1) * lda + K + 8,), G.SENTINEL[2], dtype=torch.int16, device="cuda")
    buf.as_strided((M, K), (lda, 1)).copy_(torch.from_numpy(a.view(np.int16)).cuda())
    B = torch.from_numpy(b.view(np.int16)).cuda()
    p, C = run(torch, h, (N_, N_), M, N, K, buf, lda, B, N, tgemm.BF16_F32, tile)
    assert p["vector_loads"] == vec
    del buf
    ref = o.gemm(a, b, "bf16", "f32")
    G.compare(C.cpu().numpy().view(np.int32), ref.view(np.int32), "f32")
