"""The C ABI on the host: the library loads, exports every symbol the header
declares, and its argument checks and planning (pure host code) behave as
documented in include/tgemm.h. No kernel is launched here."""
import ctypes
import os
import re

import pytest

from tiled_gemm_output_amd import tgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tgemm.h")

NN = ctypes.c_void_p(0x1000)  # a non-null pointer value; never dereferenced by host code


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return tgemm.load()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert declared == sorted(tgemm.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(8):
        assert tgemm.gemm_status_string(s).startswith("GEMM_")
    assert tgemm.gemm_status_string(99) == "unknown status"


def ok_args(M=64, N=48, K=32):
    return [M, N, K, NN, K, NN, N, NN, N]


@pytest.mark.parametrize("dtype", range(5))
def test_valid_args(dtype):
    assert tgemm.gemm_check_args(*ok_args(), dtype) == tgemm.OK


@pytest.mark.parametrize(
    "patch,expected",
    [
        ({0: -1}, tgemm.ERR_INVALID_ARG),            # M < 0
        ({1: -5}, tgemm.ERR_INVALID_ARG),            # N < 0
        ({2: -1}, tgemm.ERR_INVALID_ARG),            # K < 0
        ({4: 31}, tgemm.ERR_INVALID_ARG),            # lda < K
        ({6: 47}, tgemm.ERR_INVALID_ARG),            # ldb < N
        ({8: 47}, tgemm.ERR_INVALID_ARG),            # ldc < N
        ({3: None}, tgemm.ERR_INVALID_ARG),          # A null with elements
        ({5: None}, tgemm.ERR_INVALID_ARG),          # B null with elements
        ({7: None}, tgemm.ERR_INVALID_ARG),          # C null with elements
        ({0: 2**31}, tgemm.ERR_INVALID_ARG),         # dimension beyond int32
        ({1: 2**30 + 1, 6: 2**30 + 1, 8: 2**30 + 1}, tgemm.ERR_INVALID_ARG),  # N beyond 2^30
        ({2: 2**30 + 1, 4: 2**30 + 1}, tgemm.ERR_INVALID_ARG),               # K beyond 2^30
    ],
)
def test_bad_args(patch, expected):
    args = ok_args()
    for i, v in patch.items():
        args[i] = v
    assert tgemm.gemm_check_args(*args, tgemm.BF16_BF16) == expected


def test_transposed_operand_strides():
    """gemm_check_args_op: a transposed A is stored K x M (lda >= M), a transposed B
    N x K (ldb >= K); op values other than N/T are invalid."""
    M, N, K = 64, 48, 32
    ck = tgemm.gemm_check_args_op
    for op_a in (tgemm.OP_N, tgemm.OP_T):
        for op_b in (tgemm.OP_N, tgemm.OP_T):
            lda = M if op_a == tgemm.OP_T else K
            ldb = K if op_b == tgemm.OP_T else N
            assert ck(op_a, op_b, M, N, K, NN, lda, NN, ldb, NN, N, tgemm.BF16_F32) == tgemm.OK
            assert ck(op_a, op_b, M, N, K, NN, lda - 1, NN, ldb, NN, N, tgemm.BF16_F32) == tgemm.ERR_INVALID_ARG
            assert ck(op_a, op_b, M, N, K, NN, lda, NN, ldb - 1, NN, N, tgemm.BF16_F32) == tgemm.ERR_INVALID_ARG
    # lda = K = 32 < M = 64 is too short for a transposed A; fine untransposed
    assert ck(tgemm.OP_T, tgemm.OP_N, M, N, K, NN, K, NN, N, NN, N, tgemm.BF16_F32) == tgemm.ERR_INVALID_ARG
    assert ck(tgemm.OP_N, tgemm.OP_N, M, N, K, NN, K, NN, N, NN, N, tgemm.BF16_F32) == tgemm.OK
    for bad in (2, -1):
        assert ck(bad, tgemm.OP_N, M, N, K, NN, K, NN, N, NN, N, tgemm.BF16_F32) == tgemm.ERR_INVALID_ARG
        assert ck(tgemm.OP_N, bad, M, N, K, NN, K, NN, N, NN, N, tgemm.BF16_F32) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_run_op(None, tgemm.OP_T, tgemm.OP_N, M, N, K, NN, M, NN, N, NN, N, tgemm.BF16_F32,
                             None) == tgemm.ERR_INVALID_ARG
    # gemm_check_args is the (N, N) case
    assert tgemm.gemm_check_args(*ok_args(), tgemm.BF16_F32) == ck(tgemm.OP_N, tgemm.OP_N, *ok_args(), tgemm.BF16_F32)


def test_largest_dimensions_accepted():
    assert tgemm.gemm_check_args(2**30, 8, 8, NN, 8, NN, 8, NN, 8, tgemm.BF16_F32) == tgemm.OK
    assert tgemm.gemm_check_args(2**30 + 1, 8, 8, NN, 8, NN, 8, NN, 8, tgemm.BF16_F32) == tgemm.ERR_INVALID_ARG


def test_unknown_dtype():
    assert tgemm.gemm_check_args(*ok_args(), 5) == tgemm.ERR_UNSUPPORTED_DTYPE
    assert tgemm.gemm_check_args(*ok_args(), -1) == tgemm.ERR_UNSUPPORTED_DTYPE


def test_null_pointers_allowed_for_empty_matrices():
    # M == 0: A and C have no elements
    assert tgemm.gemm_check_args(0, 8, 8, None, 8, NN, 8, None, 8, tgemm.F16_F32) == tgemm.OK
    # K == 0: A and B have no elements, C is zero-filled
    assert tgemm.gemm_check_args(4, 8, 0, None, 1, None, 8, NN, 8, tgemm.F16_F32) == tgemm.OK
    assert tgemm.gemm_check_args(4, 8, 0, None, 1, None, 8, None, 8, tgemm.F16_F32) == tgemm.ERR_INVALID_ARG


def test_null_or_unknown_handle():
    assert tgemm.gemm_destroy(None) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_set_tile(None, 16, 16, 32) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_set_split_k(None, 2) == tgemm.ERR_INVALID_ARG
    p = tgemm.GemmPlan()
    assert tgemm.load().gemm_tune(None, 0, 0, *ok_args(), tgemm.BF16_F32, None, 5, ctypes.byref(p)) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_run(None, *ok_args(), tgemm.BF16_BF16, None) == tgemm.ERR_INVALID_ARG
    bogus = ctypes.c_void_p(0xDEADBEEF0)
    assert tgemm.gemm_destroy(bogus) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_run(bogus, *ok_args(), tgemm.BF16_BF16, None) == tgemm.ERR_INVALID_ARG


def test_create_without_gpu():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    h = ctypes.c_void_p()
    assert tgemm.load().gemm_create(ctypes.byref(h)) == tgemm.ERR_NO_DEVICE
    assert tgemm.load().gemm_create(None) == tgemm.ERR_INVALID_ARG


def plan(M, N, K, dtype, A=0x10000, lda=None, B=0x20000, ldb=None, ldc=None):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tgemm.gemm_plan(None, M, N, K, ctypes.c_void_p(A), max(lda, 1), ctypes.c_void_p(B), max(ldb, 1),
                           ctypes.c_void_p(0x30000), max(ldc, 1), dtype)


def test_plan_auto_tiles():
    p = plan(8192, 8192, 8192, tgemm.BF16_BF16)
    assert (p["tile_m"], p["tile_n"], p["tile_k"]) == (256, 256, 64)
    assert p["kernel_name"] == "mfma_macro_tile" and p["vector_loads"] == 1 and p["grid"] == 32 * 32
    p = plan(96, 96, 96, tgemm.BF16_F32)
    assert p["kernel_name"] == "mfma_macro_tile" and p["vector_loads"] == 1
    p = plan(9, 9, 9, tgemm.I32_I32)
    assert p["kernel_name"] == "int32_valu"


def test_plan_tile_by_rounds_of_workgroups():
    """With fewer than 256 tiles of 256x256, the tile with the fewest rounds of
    workgroups times per-round work (scaled by each tile's cost per flop) wins."""
    def tile(M, N, K):
        p = plan(M, N, K, tgemm.BF16_BF16)
        return p["tile_m"], p["tile_n"], p["split_k"], p["stages"]
    assert tile(3072, 3072, 3072) == (256, 256, 1, 2)   # 144 tiles in one round, not 288 of 256x128 in two
    assert tile(3584, 3584, 3584) == (256, 256, 1, 2)   # 196 tiles
    assert tile(3072, 4096, 1024) == (256, 256, 1, 2)
    assert tile(2560, 2560, 2560)[:2] == (256, 128)     # 100 of 256x256 would leave 156 CUs idle; 200 of 256x128
    assert tile(2048, 4096, 2048)[:2] == (256, 128)     # one full round of 256x128, not 512 of 128x128
    assert tile(1024, 1024, 1024) == (64, 64, 1, 4)     # short K: 256 tiles of 64x64, 16 K-tiles each
    assert tile(512, 512, 512) == (64, 64, 1, 4)        # 8 K-tiles
    assert tile(1536, 1536, 1536)[:2] == (128, 128)     # 144 tiles of 128x128
    assert tile(128, 8192, 8192)[:3] == (128, 128, 4)   # long K: one row of 128x128 tiles reads B once
    assert tile(64, 4096, 4096)[:3] == (64, 64, 4)
    assert tile(16384, 1024, 8192)[:2] == (256, 256)    # 256 tiles: a full round


def test_plan_split_k():
    # few C tiles and a long K: the reduction is cut into K-slices
    p = plan(128, 8192, 8192, tgemm.BF16_BF16)
    assert (p["tile_m"], p["tile_n"], p["grid"]) == (128, 128, 64)
    assert p["split_k"] == 4  # 256 workgroups: one per compute unit
    p = plan(64, 64, 4096, tgemm.BF16_F32)   # one 64x64 tile, 64 K-tiles -> 16 slices of 4
    assert p["grid"] == 1 and p["split_k"] == 16
    p = plan(64, 64, 448, tgemm.F16_F16)     # 7 K-tiles: too short to split
    assert p["split_k"] == 1
    p = plan(96, 96, 2000, tgemm.BF16_F32)   # four 64x64 tiles, 32 K-tiles (ragged) -> 8 slices of 4
    assert p["split_k"] == 8
    # enough tiles, the integer path, empty products: no split
    for args in ((8192, 8192, 8192, tgemm.BF16_BF16), (4096, 4096, 4096, tgemm.BF16_BF16),
                 (9, 9, 9000, tgemm.I32_I32), (0, 64, 4096, tgemm.BF16_F32), (64, 64, 0, tgemm.BF16_F32)):
        assert plan(*args)["split_k"] == 1, args


def test_plan_stages():
    """The deep pipeline (4 stages of each operand) when the launch has at most one
    workgroup per compute unit (256) and every K-slice has at least 8 K-tiles, except
    for unsplit 128x128 tiles; 3 A stages and 2 B stages for 256x256 tiles over a C
    at most 4 tile columns wide with at least 4 times as many tile rows (split or
    not); the default one (2 A stages, 3 B stages) otherwise."""
    assert plan(8192, 8192, 8192, tgemm.BF16_BF16)["stages"] == 2             # 1024 workgroups
    assert plan(16384, 1024, 8192, tgemm.BF16_F32)["stages"] == 3             # 64 x 4 tiles
    assert plan(16384, 1024, 8192, tgemm.BF16_F32, A=0x10001)["stages"] == 2  # odd address: element loader
    assert plan(12288, 1024, 8192, tgemm.BF16_F32)["stages"] == 3             # 48 x 4 tiles
    assert plan(16384, 768, 8192, tgemm.BF16_F32)["stages"] == 3              # 64 x 3 tiles
    p = plan(20480, 1024, 4096, tgemm.BF16_F32)                                # 80 x 4, a split-K tail
    assert (p["split_k"], p["stages"], p["tail_split_k"]) == (1, 3, 4)
    assert plan(16384, 1280, 8192, tgemm.BF16_F32)["stages"] == 2             # 64 x 5 tiles
    assert plan(2048, 16384, 4096, tgemm.BF16_BF16)["stages"] == 2            # 8 x 64 tiles
    p = plan(1024, 1024, 65536, tgemm.BF16_BF16)                               # 16 tiles of 256x256 x 16 slices
    assert (p["tile_m"], p["split_k"], p["stages"]) == (256, 16, 2)
    p = plan(16384, 512, 8192, tgemm.BF16_BF16)                                # 64 x 2 tiles x 2 slices
    assert (p["tile_m"], p["split_k"], p["stages"]) == (256, 2, 3)
    p = plan(128, 8192, 8192, tgemm.BF16_F32)                                  # 64 tiles x 4 slices of 32 K-tiles
    assert (p["grid"] * p["split_k"], p["stages"]) == (256, 4)
    p = plan(768, 768, 8192, tgemm.BF16_BF16)                                  # 36 tiles of 128x128 x 7 slices
    assert (p["tile_m"], p["grid"] * p["split_k"], p["stages"]) == (128, 252, 4)
    p = plan(1792, 1792, 1096, tgemm.BF16_BF16)                                # 196 unsplit tiles of 128x128
    assert (p["tile_m"], p["grid"], p["split_k"], p["stages"]) == (128, 196, 1, 2)
    p = plan(1024, 1024, 1096, tgemm.BF16_BF16)                                # 256 tiles of 64x64, 18 K-tiles (ragged K)
    assert (p["tile_m"], p["grid"], p["split_k"], p["stages"]) == (64, 256, 1, 4)
    assert plan(1024, 1024, 900, tgemm.BF16_BF16)["stages"] == 4              # 15 K-tiles
    assert plan(1024, 1024, 448, tgemm.BF16_BF16)["stages"] == 2              # 7 K-tiles: too short
    assert plan(1024, 1024, 1096, tgemm.BF16_BF16, A=0x10001)["stages"] == 2  # odd address: element loader
    assert plan(9, 9, 9, tgemm.I32_I32)["stages"] == 1
    assert plan(0, 9, 9, tgemm.BF16_F32)["stages"] == 0


def test_plan_tail_split():
    """Automatic 256x256 plans with more than one round of tiles (256, one per compute
    unit) whose last round is partly full: the tile rows that fill whole rounds run
    first, then the remaining rows as a second launch with each tile's K range in S
    slices (S x tail tiles <= 256 workgroups), when the estimate beats one more round."""
    p = plan(6000, 6000, 6000, tgemm.BF16_BF16)  # 24 x 24 = 576 tiles = 2 rounds + 64
    # 21 tile rows = 504 tiles in 2 rounds; 3 rows x 24 = 72 tiles x 3 slices = 216 workgroups
    assert (p["tile_m"], p["grid"], p["split_k"], p["tail_m0"], p["tail_split_k"]) == (256, 576, 1, 21 * 256, 3)
    p = plan(7000, 7000, 7000, tgemm.BF16_BF16)  # 28 x 28 = 784 = 3 rounds + 16
    assert (p["tail_m0"], p["tail_split_k"]) == (27 * 256, 9)  # 1 row x 28 tiles x 9 slices = 252
    p = plan(4352, 4096, 1024, tgemm.BF16_F32)  # 17 x 16 = 272: 16 rows, then 16 tiles x 4 slices
    assert (p["tail_m0"], p["tail_split_k"]) == (4096, 4)  # 16 K-tiles: at most 16 / 4 slices
    for shape in [(8192, 8192, 8192), (4096, 4096, 4096), (16384, 1024, 8192), (8191, 8191, 8191),
                  (4352, 4096, 256),  # 4 K-tiles: too short to split
                  (2048, 2048, 8192), (128, 8192, 8192)]:
        p = plan(*shape, tgemm.BF16_BF16)
        assert (p["tail_split_k"], p["tail_m0"]) == (0, 0), shape


def test_plan_repack():
    """Automatic operand copies: an operand whose rows do not start on 128-byte
    boundaries is copied into aligned rows when the estimated time saved (13% of the
    product's for a K-contiguous operand, 5% for an M/N-contiguous one) exceeds the
    copy's (one read and one write at 6 TB/s)."""
    assert plan(8192, 8192, 8192, tgemm.BF16_BF16)["repack"] == 0           # aligned rows
    assert plan(6000, 6000, 6000, tgemm.BF16_BF16)["repack"] == 1           # 12000-byte rows: A only pays
    assert plan(10000, 10000, 10000, tgemm.BF16_BF16)["repack"] == 3        # both pay at this size
    assert plan(8191, 8191, 8191, tgemm.BF16_BF16)["repack"] == 1
    assert plan(4095, 4095, 4096, tgemm.BF16_BF16)["repack"] == 0           # B only, and it does not pay
    assert plan(8192, 8192, 8192, tgemm.BF16_BF16, A=0x10040)["repack"] == 1  # base 64 bytes off a line
    assert plan(8192, 8192, 8192, tgemm.BF16_BF16, lda=8200)["repack"] == 1
    assert plan(1000, 777, 333, tgemm.BF16_F32)["repack"] == 0              # too small to pay
    assert plan(8191, 8191, 8191, tgemm.BF16_BF16, A=0x10001)["repack"] == 0  # element loader: no copies
    p = plan(6000, 6000, 6000, tgemm.BF16_BF16)
    m = tgemm.gemm_model(p, 6000, 6000, 6000, tgemm.BF16_BF16)
    tail_ws = 8.0 * p["tail_split_k"] * (6000 - p["tail_m0"]) * 6000
    assert m["bytes_workspace"] == tail_ws + 2 * 2 * 6000 * 6000  # A read and written once


def test_plan_vector_loads_need_alignment():
    """The macro-tile kernel's direct loads need 2-byte aligned A and B only (whole
    16-byte chunks at 2-byte alignment; chunks past a row end are dealt with in the
    kernel); the one-wave 16x16x32 kernel needs 16-byte aligned A, B, strides and
    contiguous extents."""
    assert plan(1000, 777, 333, tgemm.BF16_F32)["vector_loads"] == 1        # K, N not multiples of 8
    assert plan(256, 256, 256, tgemm.BF16_F32, A=0x10002)["vector_loads"] == 1  # A 2-byte aligned
    assert plan(256, 256, 256, tgemm.BF16_F32, A=0x10001)["vector_loads"] == 0  # A not 2-byte aligned
    assert plan(256, 256, 256, tgemm.BF16_F32, lda=260)["vector_loads"] == 1
    assert plan(256, 256, 256, tgemm.BF16_F32, lda=257)["vector_loads"] == 1


def plan_op(op_a, op_b, M, N, K, dtype, A=0x10000, lda=None, B=0x20000, ldb=None):
    lda = (M if op_a == tgemm.OP_T else K) if lda is None else lda
    ldb = (K if op_b == tgemm.OP_T else N) if ldb is None else ldb
    return tgemm.gemm_plan_op(None, op_a, op_b, M, N, K, ctypes.c_void_p(A), max(lda, 1), ctypes.c_void_p(B),
                              max(ldb, 1), ctypes.c_void_p(0x30000), max(N, 1), dtype)


def test_plan_transposed_vector_loads():
    """Direct loads for every operand form, whatever the extents (the one-wave
    kernel's strict rule: contiguous extents in whole 8-element chunks -- K for A and
    M for a transposed A; N for B and K for a transposed B)."""
    T, Nn = tgemm.OP_T, tgemm.OP_N
    for op_a, op_b, M, N, K in [(Nn, T, 8192, 8192, 8192), (T, T, 256, 256, 256), (T, Nn, 100, 256, 256),
                                (Nn, Nn, 100, 256, 256), (Nn, T, 256, 100, 256), (Nn, Nn, 256, 100, 256),
                                (Nn, T, 256, 256, 100), (T, Nn, 256, 256, 100), (T, T, 99, 101, 103)]:
        assert plan_op(op_a, op_b, M, N, K, tgemm.BF16_F32)["vector_loads"] == 1, (op_a, op_b, M, N, K)
    # same tile and split choice as the untransposed product
    for op_a in (Nn, T):
        for op_b in (Nn, T):
            p = plan_op(op_a, op_b, 128, 8192, 8192, tgemm.BF16_F32)
            assert (p["tile_m"], p["tile_n"], p["split_k"]) == (128, 128, 4)


def test_plan_empty_and_zero_k():
    assert plan(0, 16, 16, tgemm.BF16_F32)["kernel_name"] == "none"
    assert plan(16, 0, 16, tgemm.BF16_F32)["kernel_name"] == "none"
    assert plan(16, 16, 0, tgemm.BF16_F32)["kernel_name"] == "zero_fill"


def test_plan_rejects_bad_arguments():
    with pytest.raises(tgemm.GemmError) as e:
        plan(-1, 16, 16, tgemm.BF16_F32)
    assert e.value.status == tgemm.ERR_INVALID_ARG
