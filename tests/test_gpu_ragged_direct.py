"""GPU parity of the direct 16-byte loads on ragged and unaligned operands.

The macro-tile kernel loads whole 16-byte chunks of a stored row at any 2-byte
alignment. A chunk that runs past the end of a stored row brings in the row's
padding or the start of the next row: those values land at reduction positions past
K, which the kernel clears once the last K-tile has landed, or at tile rows / columns
past M or N, whose outputs are never stored. The matrix's last row is guarded by the
buffer range check (the range is shortened by 2 bytes when the row length is odd,
and the last element is written into LDS separately).

Every case here fills the A and B buffers around the matrices (row padding, the
elements before an offset pointer, the guard after the end) with a NaN pattern: a
value from outside a matrix that reached a stored output would make it NaN. Outputs
are compared with the oracle in full (rule of gpu_util; bit-exact for
integer-valued inputs); the plan must name the direct loads, so the cases cannot
silently pass on the element loader.
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
NAN = G.SENTINEL[2]  # a NaN in bf16 and in f16


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


def stored(M, N, K, ops):
    """(rows, row length) of the stored A and B for the forms."""
    sa = (K, M) if ops[0] == T_ else (M, K)
    sb = (N, K) if ops[1] == T_ else (K, N)
    return sa, sb


def plan(h, M, N, K, ops, lda, ldb, ldc, offs, dtype):
    # 256-byte aligned stand-in bases plus the element offsets: the same alignment
    # classes as the test buffers (torch allocations are 256-byte aligned)
    return tgemm.gemm_plan_op(h, ops[0], ops[1], M, N, K, (1 << 20) + 2 * offs[0], lda, (1 << 24) + 2 * offs[1], ldb,
                              (1 << 28) + tgemm.OUT_BYTES[dtype] * offs[2], ldc, dtype)


def check(h, o, M, N, K, ops, dtype, pad=0, offs=(0, 0, 0), tile=None, splits=0, kind="normal", seed=0):
    (ra, la), (rb, lb) = stored(M, N, K, ops)
    lda, ldb, ldc = la + pad, lb + pad, N + pad
    tgemm.check(tgemm.gemm_set_tile(h, *(tile or (0, 0, 0))), "gemm_set_tile")
    tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
    try:
        p = plan(h, M, N, K, ops, lda, ldb, ldc, offs, dtype)
        assert p["kernel_name"] == "mfma_macro_tile" and p["vector_loads"] == 1, p
        in_kind = G.IN_KIND[dtype]
        if kind == "normal":
            a, b = inputs.random_case(M, N, K, in_kind, seed=seed)
        else:
            a = inputs.draw((M, K), kind, in_kind, seed)
            b = inputs.draw((K, N), kind, in_kind, seed + 1)
        print("ragged direct case %s %s pad %d offs %s tile %s splits %d dtype %d" %
              ((M, N, K), OP_IDS[ops], pad, offs, tile, splits, dtype), flush=True)
        c, dc = G.run(h, a, b, dtype, lda=lda, ldb=ldb, ldc=ldc, offs=offs, op_a=ops[0], op_b=ops[1], ab_fill=NAN)
    finally:
        tgemm.gemm_set_tile(h, 0, 0, 0)
        tgemm.gemm_set_split_k(h, 0)
    assert dc.untouched_outside(), "kernel wrote outside C"
    ref = o.gemm(a, b, G.IN_KIND[dtype], G.OUT_KIND[dtype]).view(G.np_int(tgemm.OUT_BYTES[dtype]))
    assert not np.isnan(G.values(c, G.OUT_KIND[dtype])).any(), "a value from outside the matrices reached C"
    if kind != "normal":
        assert np.array_equal(c, ref)
        return None
    return G.compare(c, ref, G.OUT_KIND[dtype])


# (M, N, K, row padding, element offsets of A, B, C)
CASES = [
    (1000, 777, 333, 0, (0, 0, 0)),   # odd K and N
    (999, 1001, 1003, 3, (1, 3, 0)),  # everything odd, odd strides, 2-byte aligned pointers
    (257, 129, 6, 1, (0, 0, 0)),      # K = 6: one chunk per row straddles the end
    (17, 19, 1, 0, (0, 0, 0)),        # K = 1: a stored row of one element
    (300, 5, 3, 0, (5, 7, 0)),
    (130, 70, 777, 2, (2, 6, 1)),
    (64, 64, 72, 0, (4, 0, 0)),       # 8-byte aligned A
]


@pytest.mark.parametrize("ops", OPS_ALL, ids=lambda x: OP_IDS[x])
@pytest.mark.parametrize("case", CASES, ids=str)
def test_ragged_direct_loads(h, o, case, ops):
    M, N, K, pad, offs = case
    for n, dtype in enumerate([tgemm.BF16_F32, tgemm.F16_F16]):
        check(h, o, M, N, K, ops, dtype, pad, offs, seed=M + 3 * N + 5 * K + n)


@pytest.mark.parametrize("ops", OPS_ALL, ids=lambda x: OP_IDS[x])
@pytest.mark.parametrize("tile", [(256, 256, 64), (128, 128, 64), (64, 64, 64)], ids=str)
def test_ragged_direct_loads_forced_tiles(h, o, tile, ops):
    for M, N, K, pad, offs in [(1000, 777, 333, 0, (0, 0, 0)), (299, 301, 203, 1, (1, 1, 0))]:
        check(h, o, M, N, K, ops, tgemm.BF16_BF16, pad, offs, tile=tile, seed=K)


@pytest.mark.parametrize("ops", OPS_ALL, ids=lambda x: OP_IDS[x])
def test_ragged_direct_loads_integer_inputs_bit_exact(h, o, ops):
    for M, N, K, pad, offs in [(999, 1001, 1003, 3, (1, 3, 0)), (257, 129, 6, 1, (0, 0, 0))]:
        check(h, o, M, N, K, ops, tgemm.BF16_F32, pad, offs, kind="small_int", seed=M)


@pytest.mark.parametrize("ops", OPS_ALL, ids=lambda x: OP_IDS[x])
@pytest.mark.parametrize("splits", [0, 3, 8])
def test_ragged_direct_loads_split_k(h, o, ops, splits):
    for M, N, K in [(128, 1023, 2049), (96, 201, 3001)]:
        check(h, o, M, N, K, ops, tgemm.BF16_F32, 1, (1, 0, 0), splits=splits, seed=K + splits)


def test_ragged_direct_loads_four_stages(h, o):
    """The 4-stage pipeline (a single round of workgroups in K-slices, long K) on ragged extents."""
    for (M, N, K), ops in [((1100, 1002, 6000), (N_, N_)), ((1099, 1001, 6001), (T_, T_))]:
        (ra, la), (rb, lb) = stored(M, N, K, ops)
        p = plan(h, M, N, K, ops, la, lb, N, (0, 0, 0), tgemm.BF16_BF16)
        assert p["stages"] == 4, p
        check(h, o, M, N, K, ops, tgemm.BF16_BF16, seed=K)


@pytest.mark.parametrize("shape", [(4095, 4095, 4096), (8191, 8191, 8191)], ids=str)
def test_ragged_direct_loads_large_sampled(h, o, shape):
    """Large ragged products (the shapes whose element-loader times were far behind
    the aligned ones), compared on sampled rows and columns."""
    import torch

    M, N, K = shape
    a, b = inputs.random_case(M, N, K, "bf16", seed=M + K)
    p = plan(h, M, N, K, (N_, N_), K, N, N, (0, 0, 0), tgemm.BF16_BF16)
    assert p["vector_loads"] == 1, p
    print("ragged direct large %s" % (shape,), flush=True)
    da = torch.from_numpy(a.view(np.int16)).cuda()
    db = torch.from_numpy(b.view(np.int16)).cuda()
    dc = torch.full((M, N), G.SENTINEL[2], dtype=torch.int16, device="cuda")
    tgemm.check(tgemm.gemm_run(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N, tgemm.BF16_BF16,
                               torch.cuda.current_stream().cuda_stream), "gemm_run")
    torch.cuda.synchronize()
    rows, cols = inputs.sample_rows_cols(M, N, seed=7, block=256)
    got_r = dc[torch.from_numpy(rows).cuda()].cpu().numpy()
    got_c = dc[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    G.compare(got_r, o.gemm_rows(a, b, rows, "bf16", "bf16").view(np.int16), "bf16")
    G.compare(got_c, o.gemm_cols(a, b, cols, "bf16", "bf16").view(np.int16), "bf16")
