"""GPU parity of the transposed-operand forms, C = op(A) @ op(B) (gemm_run_op).

The device holds the transpose of a transposed operand (A as K x M, B as N x K);
the oracle computes on the logical M x K and K x N matrices, so the layouts are
checked against the plain definition, not against each other. Then, because the
two staging paths deliver the same values to the same MFMA lanes, the four forms
must also agree with one another bit for bit for a fixed tile.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu

N_, T_ = tgemm.OP_N, tgemm.OP_T
OPS = [(N_, T_), (T_, N_), (T_, T_)]
OPS_ALL = [(N_, N_)] + OPS
OP_IDS = {(N_, N_): "NN", (N_, T_): "NT", (T_, N_): "TN", (T_, T_): "TT"}


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


def configure(h, tile=None, splits=0):
    tgemm.check(tgemm.gemm_set_tile(h, *(tile or (0, 0, 0))), "gemm_set_tile")
    tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")


def run(h, a, b, dtype, ops, tile=None, splits=0, **layout):
    configure(h, tile, splits)
    try:
        return G.run(h, a, b, dtype, op_a=ops[0], op_b=ops[1], **layout)
    finally:
        configure(h)


def ref_bits(o, a, b, dtype):
    return o.gemm(a, b, G.IN_KIND[dtype], G.OUT_KIND[dtype]).view(G.np_int(tgemm.OUT_BYTES[dtype]))


def check(h, o, a, b, dtype, ops, tile=None, splits=0, **layout):
    c, dc = run(h, a, b, dtype, ops, tile, splits, **layout)
    assert dc.untouched_outside(), "kernel wrote outside C"
    return c, G.compare(c, ref_bits(o, a, b, dtype), G.OUT_KIND[dtype])


TILES = [None, (16, 16, 32), (64, 64, 64), (128, 128, 64), (256, 128, 64), (256, 256, 64)]
# element loader (ragged, odd extents), direct loads with a ragged K tail, direct loads with K % 64 == 0
SHAPES = [(1000, 777, 333), (520, 264, 136), (512, 384, 256), (33, 40, 72)]


@pytest.mark.parametrize("ops", OPS, ids=lambda x: OP_IDS[x])
@pytest.mark.parametrize("tile", TILES, ids=str)
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_transposed_forms(h, o, ops, tile, shape):
    M, N, K = shape
    for n, dtype in enumerate([tgemm.BF16_F32, tgemm.F16_F16, tgemm.BF16_BF16, tgemm.F16_F32]):
        if tile is not None and n > 1:
            continue  # forced tiles: two formats are enough
        a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=M + 3 * N + 5 * K + n)
        check(h, o, a, b, dtype, ops, tile)


@pytest.mark.parametrize("ops", OPS, ids=lambda x: OP_IDS[x])
def test_transposed_vector_path_taken(h, ops):
    """The aligned shapes above really use the 16-byte loads in every form."""
    M, N, K = 512, 384, 256
    p = tgemm.gemm_plan_op(h, ops[0], ops[1], M, N, K, 1 << 20, M if ops[0] == T_ else K, 1 << 22,
                           K if ops[1] == T_ else N, 1 << 24, N, tgemm.BF16_F32)
    assert p["vector_loads"] == 1 and p["kernel_name"] == "mfma_macro_tile"


@pytest.mark.parametrize("tile", [None, (16, 16, 32), (64, 64, 64), (256, 256, 64)], ids=str)
@pytest.mark.parametrize("shape", [(300, 200, 150), (256, 256, 256), (257, 129, 8), (1, 1, 1)], ids=str)
def test_forms_agree_bit_for_bit(h, o, tile, shape):
    """Same fragments in the same lanes: NN, NT, TN and TT give identical bits."""
    M, N, K = shape
    a, b = inputs.random_case(M, N, K, "bf16", seed=17 + M)
    outs = [run(h, a, b, tgemm.BF16_F32, ops, tile)[0] for ops in OPS_ALL]
    for c in outs[1:]:
        assert np.array_equal(outs[0], c)
    G.compare(outs[0], ref_bits(o, a, b, tgemm.BF16_F32), "f32")


@pytest.mark.parametrize("ops", OPS, ids=lambda x: OP_IDS[x])
def test_transposed_integer_inputs_bit_exact(h, o, ops):
    for M, N, K in [(300, 200, 150), (256, 512, 1024), (33, 520, 72)]:
        for dtype, kind in [(tgemm.BF16_F32, "bf16"), (tgemm.F16_F16, "f16")]:
            a = inputs.draw((M, K), "small_int", kind, 61 + M)
            b = inputs.draw((K, N), "small_int", kind, 67 + N)
            c, dc = run(h, a, b, dtype, ops)
            assert dc.untouched_outside()
            assert np.array_equal(c, ref_bits(o, a, b, dtype)), (M, N, K, dtype)


@pytest.mark.parametrize("ops", OPS, ids=lambda x: OP_IDS[x])
@pytest.mark.parametrize("tile", [None, (3, 3, 3), (16, 16, 64), (32, 8, 7)], ids=str)
def test_transposed_int32(h, o, ops, tile):
    a, b = inputs.random_case(77, 45, 61, "i32", seed=5)
    c, dc = run(h, a, b, tgemm.I32_I32, ops, tile)
    assert dc.untouched_outside()
    assert np.array_equal(c.view(np.int32), ref_bits(o, a, b, tgemm.I32_I32).view(np.int32))


@pytest.mark.parametrize("ops", OPS, ids=lambda x: OP_IDS[x])
def test_transposed_padded_and_offset(h, o, ops):
    """Leading dimensions beyond the stored row length and element offsets (the
    element loader for unaligned pointers, the direct loads for aligned ones)."""
    for (M, N, K), pad, offs in [((200, 136, 1000), 8, (0, 0, 0)), ((130, 70, 777), 3, (1, 2, 5)),
                                 ((256, 256, 512), 16, (8, 8, 0))]:
        a, b = inputs.random_case(M, N, K, "bf16", seed=M + pad)
        lda = (M if ops[0] == T_ else K) + pad
        ldb = (K if ops[1] == T_ else N) + pad
        check(h, o, a, b, tgemm.BF16_BF16, ops, lda=lda, ldb=ldb, ldc=N + pad, offs=offs)


@pytest.mark.parametrize("ops", OPS, ids=lambda x: OP_IDS[x])
@pytest.mark.parametrize("splits", [0, 3, 8])
def test_transposed_split_k(h, o, ops, splits):
    for M, N, K in [(64, 512, 4096), (96, 200, 3000), (128, 1024, 2048)]:
        a, b = inputs.random_case(M, N, K, "bf16", seed=K + splits)
        check(h, o, a, b, tgemm.BF16_F32, ops, splits=splits)


@pytest.mark.parametrize("name,ops", [("square8192_bf16", (N_, T_)), ("square8192_bf16", (T_, N_)),
                                      ("square8192_bf16", (T_, T_)), ("skinny128x8192x8192_bf16", (N_, T_)),
                                      ("tall16384x1024x8192_bf16", (T_, N_))], ids=str)
def test_transposed_large_sampled(h, o, name, ops):
    """Full-size products in the forms real callers use most (weights stored N x K),
    compared on sampled rows and columns."""
    import torch

    w = inputs.WORKLOADS[name]
    a, b = inputs.make(w)
    dtype = tgemm.DTYPES[w.dtype]
    sa = np.ascontiguousarray(a.T) if ops[0] == T_ else a
    sb = np.ascontiguousarray(b.T) if ops[1] == T_ else b
    da = torch.from_numpy(sa.view(np.int16)).cuda()
    db = torch.from_numpy(sb.view(np.int16)).cuda()
    ob = tgemm.OUT_BYTES[dtype]
    dc = torch.full((w.M, w.N), G.SENTINEL[ob], dtype=G.int_dtype(ob), device="cuda")
    tgemm.check(tgemm.gemm_run_op(h, ops[0], ops[1], w.M, w.N, w.K, da.data_ptr(), sa.shape[1], db.data_ptr(),
                                  sb.shape[1], dc.data_ptr(), w.N, dtype, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    rows, cols = inputs.sample_rows_cols(w.M, w.N, seed=w.index + 1, block=512)
    kind_in, kind_out = G.IN_KIND[dtype], G.OUT_KIND[dtype]
    got_r = dc[torch.from_numpy(rows).cuda()].cpu().numpy()
    got_c = dc[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    G.compare(got_r, o.gemm_rows(a, b, rows, kind_in, kind_out).view(G.np_int(ob)), kind_out)
    G.compare(got_c, o.gemm_cols(a, b, cols, kind_in, kind_out).view(G.np_int(ob)), kind_out)
