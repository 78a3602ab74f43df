"""GPU parity of operand copies into aligned rows (gemm_set_repack).

An operand whose rows do not start on 128-byte boundaries can be copied first into
rows padded to a multiple of 64 elements in the handle's workspace. The product
kernels then see the same values in the same order, so every case must give results
identical bit for bit to the same call without copies (mode -1), and the oracle's
result; the plan must flag exactly the operands whose rows are off 128-byte
boundaries (mode 1). The buffers around A and B hold NaN, as in the ragged-load
tests, and C must be untouched outside its window.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu

N_, T_ = tgemm.OP_N, tgemm.OP_T
OPS_ALL = [(N_, N_), (N_, T_), (T_, N_), (T_, T_)]
OP_IDS = {(N_, N_): "NN", (N_, T_): "NT", (T_, N_): "TN", (T_, T_): "TT"}
NAN = G.SENTINEL[2]


@pytest.fixture(scope="module")
def h():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = tgemm.gemm_create()
    yield g
    tgemm.gemm_set_repack(g, 0)
    tgemm.gemm_destroy(g)


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def layout(M, N, K, ops, pad, offs):
    la = (M if ops[0] == T_ else K) + pad
    lb = (K if ops[1] == T_ else N) + pad
    return la, lb


def expected_bits(ops, M, N, K, la, lb, offs):
    """Operands whose rows are off 128-byte boundaries (bit 0 A, bit 1 B); the test
    buffers start 256-byte aligned, so only the element offsets and strides count."""
    bits = 0
    if (2 * offs[0]) % 128 or (2 * la) % 128:
        bits |= 1
    if (2 * offs[1]) % 128 or (2 * lb) % 128:
        bits |= 2
    return bits


def run_modes(h, a, b, dtype, ops, la, lb, ldc, offs, tile=None, splits=0):
    """(C with copies, C without) for one call; checks the plan's flags."""
    M, K = a.shape
    N = b.shape[1]
    tgemm.check(tgemm.gemm_set_tile(h, *(tile or (0, 0, 0))), "gemm_set_tile")
    tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
    out = []
    try:
        for mode in (1, -1):
            tgemm.check(tgemm.gemm_set_repack(h, mode), "gemm_set_repack")
            p = tgemm.gemm_plan_op(h, ops[0], ops[1], M, N, K, (1 << 20) + 2 * offs[0], la, (1 << 24) + 2 * offs[1],
                                   lb, (1 << 28), ldc, dtype)
            want = expected_bits(ops, M, N, K, la, lb, offs) if mode == 1 else 0
            assert p["kernel_name"] == "mfma_macro_tile" and p["vector_loads"] == 1, p
            assert p["repack"] == want, (p, want)
            print("repack case %s %s lda %d ldb %d offs %s mode %d bits %d" %
                  ((M, N, K), OP_IDS[ops], la, lb, offs, mode, p["repack"]), flush=True)
            c, dc = G.run(h, a, b, dtype, lda=la, ldb=lb, ldc=ldc, offs=offs, op_a=ops[0], op_b=ops[1], ab_fill=NAN)
            assert dc.untouched_outside(), "kernel wrote outside C"
            out.append(c)
    finally:
        tgemm.gemm_set_repack(h, 0)
        tgemm.gemm_set_tile(h, 0, 0, 0)
        tgemm.gemm_set_split_k(h, 0)
    return out


CASES = [
    (1000, 777, 333, 0, (0, 0, 0)),
    (999, 1001, 1003, 3, (1, 3, 0)),
    (257, 129, 6, 1, (0, 0, 0)),
    (17, 19, 1, 0, (0, 0, 0)),
    (300, 5, 3, 0, (5, 7, 0)),
    (130, 70, 777, 2, (2, 6, 1)),
    (512, 384, 256, 0, (4, 0, 0)),  # 8-byte aligned A, aligned B
    (256, 300, 200, 0, (0, 0, 0)),  # 16-byte but not 128-byte aligned rows
]


@pytest.mark.parametrize("ops", OPS_ALL, ids=lambda x: OP_IDS[x])
@pytest.mark.parametrize("case", CASES, ids=str)
def test_copies_change_nothing(h, o, case, ops):
    M, N, K, pad, offs = case
    la, lb = layout(M, N, K, ops, pad, offs)
    for n, dtype in enumerate([tgemm.BF16_F32, tgemm.F16_F16]):
        a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=M + 3 * N + 5 * K + n)
        with_copies, without = run_modes(h, a, b, dtype, ops, la, lb, N + pad, offs)
        assert np.array_equal(with_copies, without)
        ref = o.gemm(a, b, G.IN_KIND[dtype], G.OUT_KIND[dtype]).view(G.np_int(tgemm.OUT_BYTES[dtype]))
        G.compare(with_copies, ref, G.OUT_KIND[dtype])


@pytest.mark.parametrize("ops", [(N_, N_), (T_, T_)], ids=["NN", "TT"])
def test_copies_with_split_k_and_tail(h, o, ops):
    """Copies followed by a forced split-K launch, and by a plan with a split-K tail."""
    for (M, N, K), pad, offs, splits in [((96, 201, 3001), 1, (1, 0, 0), 3), ((4352, 4096, 1024), 1, (0, 1, 0), 0)]:
        la, lb = layout(M, N, K, ops, pad, offs)
        a, b = inputs.random_case(M, N, K, "bf16", seed=K)
        with_copies, without = run_modes(h, a, b, tgemm.BF16_F32, ops, la, lb, N, offs, splits=splits)
        assert np.array_equal(with_copies, without)
        G.compare(with_copies, o.gemm(a, b, "bf16", "f32").view(np.int32), "f32")


def test_automatic_copy_at_8191(h, o):
    """8191^3 bf16 (odd leading dimensions): the automatic plan copies A; the result
    equals the call without copies bit for bit and the oracle on sampled rows and columns."""
    import torch

    M = N = K = 8191
    a, b = inputs.random_case(M, N, K, "bf16", seed=8191)
    da = torch.from_numpy(a.view(np.int16)).cuda()
    db = torch.from_numpy(b.view(np.int16)).cuda()
    outs = []
    try:
        for mode in (0, -1):
            tgemm.check(tgemm.gemm_set_repack(h, mode))
            p = tgemm.gemm_plan(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, 1 << 28, N, tgemm.BF16_BF16)
            assert p["repack"] == (1 if mode == 0 else 0), p
            dc = torch.full((M, N), G.SENTINEL[2], dtype=torch.int16, device="cuda")
            tgemm.check(tgemm.gemm_run(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N,
                                       tgemm.BF16_BF16, torch.cuda.current_stream().cuda_stream), "gemm_run")
            torch.cuda.synchronize()
            outs.append(dc)
    finally:
        tgemm.gemm_set_repack(h, 0)
    assert torch.equal(outs[0], outs[1])
    rows, cols = inputs.sample_rows_cols(M, N, seed=5, block=256)
    got_r = outs[0][torch.from_numpy(rows).cuda()].cpu().numpy()
    got_c = outs[0][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    G.compare(got_r, o.gemm_rows(a, b, rows, "bf16", "bf16").view(np.int16), "bf16")
    G.compare(got_c, o.gemm_cols(a, b, cols, "bf16", "bf16").view(np.int16), "bf16")


def test_set_repack_arguments(h):
    assert tgemm.gemm_set_repack(h, 2) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_set_repack(h, -2) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_set_repack(None, 0) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_set_repack(h, 0) == tgemm.OK
