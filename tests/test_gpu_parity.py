"""GPU parity: the HIP library (through its C ABI) against the oracle.

Every case runs through gemm_run on the device and is compared with the oracle on
the same seeded inputs (tiled_gemm_output_amd/inputs.py): bit-exact for int32 and
for integer-valued float inputs, the accuracy rule of gpu_util otherwise. Full
outputs are compared at the small workloads and a randomized sweep of ragged
shapes, leading dimensions and pointer offsets; at the large workloads the
sampled rows and columns (one per 128-block plus the first and last) are compared,
in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tests import oracle_pins
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu


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


def set_tile(h, tile):
    tgemm.check(tgemm.gemm_set_tile(h, *(tile or (0, 0, 0))), "gemm_set_tile")


def oracle_ref(o, a, b, dtype):
    return o.gemm(a, b, G.IN_KIND[dtype], G.OUT_KIND[dtype])


def check_full(h, o, a, b, dtype, tile=None, splits=0, **layout):
    set_tile(h, tile)
    tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
    try:
        c, dc = G.run(h, a, b, dtype, **layout)
    finally:
        set_tile(h, None)
        tgemm.gemm_set_split_k(h, 0)
    assert dc.untouched_outside(), "kernel wrote outside C"
    ref = oracle_ref(o, a, b, dtype)
    if dtype == tgemm.I32_I32:
        return G.compare(c.view(np.int32), ref.view(np.int32), "i32")
    return G.compare(c, ref.view(G.np_int(tgemm.OUT_BYTES[dtype])), G.OUT_KIND[dtype])


# ---------------------------------------------------------------- the workloads

def test_worked_example_9x9(h, o):
    """The puzzle page's example with its 3x3 tiles: bit-exact, and equal to the closed form."""
    a, b = inputs.worked_example()
    for tile in [(3, 3, 3), None]:
        set_tile(h, tile)
        c, dc = G.run(h, a, b, tgemm.I32_I32)
        set_tile(h, None)
        assert dc.untouched_outside()
        assert np.array_equal(c.astype(np.int64), oracle_pins.worked_closed_form())
        assert np.array_equal(c, o.gemm(a, b, "i32", "i32"))


def test_square128_f16_16x16x32(h, o):
    w = inputs.WORKLOADS["square128_f16"]
    a, b = inputs.make(w)
    st = check_full(h, o, a, b, tgemm.F16_F32, tile=w.tile)
    assert st["normwise"] < 1e-5
    set_tile(h, w.tile)
    p = tgemm.gemm_plan(h, 128, 128, 128, 1 << 20, 128, 1 << 21, 128, 1 << 22, 128, tgemm.F16_F32)
    set_tile(h, None)
    assert p["kernel_name"] == "mfma_16x16x32_one_wave" and p["grid"] == 64 and p["vector_loads"] == 1


@pytest.mark.parametrize("name", ["ragged96_bf16", "ragged1000x777x333_bf16"])
@pytest.mark.parametrize("dtype", [tgemm.BF16_F32, tgemm.BF16_BF16])
@pytest.mark.parametrize("forced", [True, False])
def test_ragged_edge_tiles(h, o, name, dtype, forced):
    w = inputs.WORKLOADS[name]
    a, b = inputs.make(w)
    check_full(h, o, a, b, dtype, tile=w.tile if forced else None)


LARGE = ["square4096_bf16", "square8192_bf16", "tall16384x1024x8192_bf16", "skinny128x8192x8192_bf16"]


def sampled_check(h, o, a, b, dtype, rows, cols, exact=False):
    """Run at full size; compare the sampled rows and columns with the oracle."""
    import torch

    M, K = a.shape
    N = b.shape[1]
    ob = tgemm.OUT_BYTES[dtype]
    da = torch.from_numpy(a.view(np.int16)).cuda()
    db = torch.from_numpy(b.view(np.int16)).cuda()
    dc = torch.full((M, N), G.SENTINEL[ob], dtype=G.int_dtype(ob), device="cuda")
    st = tgemm.gemm_run(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N, dtype,
                        torch.cuda.current_stream().cuda_stream)
    tgemm.check(st, "gemm_run")
    torch.cuda.synchronize()
    kind_in, kind_out = G.IN_KIND[dtype], G.OUT_KIND[dtype]
    got_r = dc[torch.from_numpy(rows).cuda()].cpu().numpy()
    got_c = dc[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    ref_r = o.gemm_rows(a, b, rows, kind_in, kind_out).view(G.np_int(ob))
    ref_c = o.gemm_cols(a, b, cols, kind_in, kind_out).view(G.np_int(ob))
    if exact:
        assert np.array_equal(got_r, ref_r) and np.array_equal(got_c, ref_c)
        return {}
    s1 = G.compare(got_r, ref_r, kind_out)
    s2 = G.compare(got_c, ref_c, kind_out)
    return {"rows": s1, "cols": s2}


@pytest.mark.parametrize("name", LARGE)
def test_large_workloads_sampled(h, o, name):
    w = inputs.WORKLOADS[name]
    a, b = inputs.make(w)
    rows, cols = inputs.sample_rows_cols(w.M, w.N, seed=w.index, block=256)
    sampled_check(h, o, a, b, tgemm.DTYPES[w.dtype], rows, cols)


@pytest.mark.parametrize("dtype", [tgemm.F16_F16, tgemm.F16_F32])
def test_large_f16_sampled(h, o, dtype):
    """fp16 inputs at the full 8192^3 size (N(0, 1) draws rounded to fp16; the sums, up to
    a few hundred, stay far inside fp16's range), on sampled rows and columns."""
    a, b = inputs.random_case(8192, 8192, 8192, "f16", seed=8192 + dtype)
    rows, cols = inputs.sample_rows_cols(8192, 8192, seed=dtype, block=512)
    print("large f16 8192^3 dtype %d" % dtype, flush=True)
    sampled_check(h, o, a, b, dtype, rows, cols)


@pytest.mark.parametrize("name", ["square8192_bf16", "skinny128x8192x8192_bf16"])
def test_large_exact_integer_inputs(h, o, name):
    """Integer-valued inputs in [-8, 8]: every fp32 partial sum is exact, so the
    sampled outputs must match the oracle bit for bit at full size."""
    w = inputs.WORKLOADS[name]
    a = inputs.draw((w.M, w.K), "small_int", "bf16", 101)
    b = inputs.draw((w.K, w.N), "small_int", "bf16", 102)
    rows, cols = inputs.sample_rows_cols(w.M, w.N, seed=7, block=512)
    sampled_check(h, o, a, b, tgemm.DTYPES[w.dtype], rows, cols, exact=True)


# ---------------------------------------------------------------- exact classes

TILES_FLOAT = [(16, 16, 32), (64, 64, 64), (128, 128, 64), (256, 128, 64), (256, 256, 64), None]


@pytest.mark.parametrize("tile", TILES_FLOAT, ids=str)
@pytest.mark.parametrize("shape", [(300, 200, 150), (256, 256, 256), (33, 520, 72), (1, 1, 1), (257, 129, 8)], ids=str)
def test_integer_inputs_bit_exact(h, o, tile, shape):
    M, N, K = shape
    for dtype, kind in [(tgemm.BF16_F32, "bf16"), (tgemm.F16_F32, "f16"), (tgemm.BF16_BF16, "bf16")]:
        a = inputs.draw((M, K), "small_int", kind, 11 + M)
        b = inputs.draw((K, N), "small_int", kind, 13 + N)
        set_tile(h, tile)
        c, dc = G.run(h, a, b, dtype)
        set_tile(h, None)
        assert dc.untouched_outside()
        ref = oracle_ref(o, a, b, dtype).view(G.np_int(tgemm.OUT_BYTES[dtype]))
        assert np.array_equal(c, ref), (dtype, tile, shape)


def test_identity_and_zero(h, o):
    rng = np.random.default_rng(5)
    a = inputs.to_bits(rng.standard_normal((130, 96)).astype(np.float32), "bf16")
    eye = inputs.to_bits(np.eye(96, dtype=np.float32), "bf16")
    c, _ = G.run(h, a, eye, tgemm.BF16_BF16)
    assert np.array_equal(c.view(np.uint16), a)
    z = np.zeros_like(a)
    c, _ = G.run(h, z, eye, tgemm.BF16_F32)
    assert not np.any(G.values(c, "f32"))


# ---------------------------------------------------------------- sweep

def sweep_cases():
    rng = np.random.default_rng(2026)
    cases = []
    dtypes = [tgemm.BF16_F32, tgemm.BF16_BF16, tgemm.F16_F32, tgemm.F16_F16, tgemm.I32_I32]
    for n in range(40):
        M, N, K = (int(x) for x in rng.integers(1, 301, size=3))
        dtype = dtypes[n % len(dtypes)]
        pad = [0, 1, 8][n % 3]
        offs = (0, 0, 0) if n % 4 == 0 else tuple(int(x) for x in rng.integers(0, 9, size=3))
        cases.append((M, N, K, dtype, pad, offs))
    # aligned shapes that take the direct-load path, and K not a multiple of 64
    cases += [(512, 384, 200, tgemm.BF16_F32, 0, (0, 0, 0)), (520, 264, 136, tgemm.BF16_BF16, 8, (0, 0, 0)),
              (1024, 1024, 64, tgemm.F16_F32, 0, (0, 0, 0)), (768, 512, 1000, tgemm.BF16_F32, 0, (0, 0, 0))]
    return cases


@pytest.mark.parametrize("case", sweep_cases(), ids=str)
def test_random_sweep(h, o, case):
    M, N, K, dtype, pad, offs = case
    kind = G.IN_KIND[dtype]
    a, b = inputs.random_case(M, N, K, kind, seed=M * 7 + N * 3 + K)
    check_full(h, o, a, b, dtype, lda=K + pad, ldb=N + pad, ldc=N + pad, offs=offs)


@pytest.mark.parametrize("tile", [(3, 3, 3), (1, 1, 1), (16, 16, 64), (32, 8, 7), (32, 32, 32), None], ids=str)
def test_int32_tiles(h, o, tile):
    a, b = inputs.random_case(77, 45, 61, "i32", seed=3)
    check_full(h, o, a, b, tgemm.I32_I32, tile=tile)


# ---------------------------------------------------------------- degenerate cases

def test_k_zero_fills_zeros(h, o):
    import torch

    for dtype in [tgemm.BF16_F32, tgemm.BF16_BF16, tgemm.I32_I32]:
        ob = tgemm.OUT_BYTES[dtype]
        dc = G.DevMatrix(None, 37, 21, 24, 3, ob)
        st = tgemm.gemm_run(h, 37, 21, 0, None, 1, None, 21, dc.ptr, dc.ld, dtype,
                            torch.cuda.current_stream().cuda_stream)
        tgemm.check(st)
        torch.cuda.synchronize()
        assert not np.any(dc.host()) and dc.untouched_outside()


def test_empty_output_launches_nothing(h):
    import torch

    dc = G.DevMatrix(None, 4, 4, 4, 0, 4)
    for M, N in [(0, 4), (4, 0)]:
        st = tgemm.gemm_run(h, M, N, 5, dc.ptr, 5, dc.ptr, max(N, 1), dc.ptr, max(N, 1), tgemm.BF16_F32,
                            torch.cuda.current_stream().cuda_stream)
        assert st == tgemm.OK
    torch.cuda.synchronize()
    assert np.all(dc.host() == dc.fill)


def test_unsupported_forced_tile(h):
    tgemm.check(tgemm.gemm_set_tile(h, 48, 48, 48))
    try:
        st = tgemm.gemm_run(h, 64, 64, 64, 1 << 20, 64, 1 << 21, 64, 1 << 22, 64, tgemm.BF16_F32, None)
        assert st == tgemm.ERR_UNSUPPORTED_TILE
    finally:
        tgemm.gemm_set_tile(h, 0, 0, 0)


def test_repeatable_and_side_stream(h, o):
    """Same inputs twice (second time on a non-default stream): identical bits."""
    import torch

    a, b = inputs.random_case(1024, 768, 1536, "bf16", seed=9)
    c1, _ = G.run(h, a, b, tgemm.BF16_F32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c2, _ = G.run(h, a, b, tgemm.BF16_F32, stream=s)
    assert np.array_equal(c1, c2)
    G.compare(c1, oracle_ref(o, a, b, tgemm.BF16_F32).view(np.int32), "f32")


# ---------------------------------------------------------------- split-K

def plan_of(h, M, N, K, dtype, splits=0, tile=None):
    """gemm_plan for dense row-major operands under a forced split count / tile."""
    set_tile(h, tile)
    tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
    try:
        return tgemm.gemm_plan(h, M, N, K, 1 << 20, K, 1 << 21, N, 1 << 22, N, dtype)
    finally:
        set_tile(h, None)
        tgemm.gemm_set_split_k(h, 0)


SPLIT_SHAPES = [(200, 136, 1000), (130, 70, 777), (256, 256, 4096), (64, 512, 640), (1, 8, 2048)]


@pytest.mark.parametrize("splits", [2, 3, 5, 16, 64])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=str)
def test_split_k_forced(h, o, shape, splits):
    """K cut into slices (ragged last slice, ragged K tail, element and direct
    loaders), fp32 partial tiles summed in slice order, one rounding at the end."""
    M, N, K = shape
    nk = -(-K // 64)
    for n, dtype in enumerate([tgemm.BF16_BF16, tgemm.F16_F32, tgemm.BF16_F32, tgemm.F16_F16]):
        p = plan_of(h, M, N, K, dtype, splits)
        assert p["kernel_name"] == "mfma_macro_tile"
        per = -(-nk // min(splits, nk))
        assert p["split_k"] == -(-nk // per) and p["split_k"] <= splits
        a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=31 * splits + n)
        check_full(h, o, a, b, dtype, splits=splits)


@pytest.mark.parametrize("shape,splits", [((1100, 2000, 8200), 3), ((2048, 1024, 8192), 4), ((1100, 2000, 4000), 3),
                                          ((2048, 2048, 4096), 1), ((768, 768, 8192), 7), ((128, 8192, 8192), 4),
                                          ((257, 2440, 3976), 4), ((251, 2033, 11048), 8)],
                         ids=str)
def test_automatic_split_of_one_round(h, o, shape, splits):
    """Automatic plans of at most one round of 128x128 tiles take the K-slice count of
    the library's estimate: 144 tiles over 129 or 63 K-tiles in 3 slices, 128 tiles
    over 128 K-tiles in 4 (two workgroups on every compute unit), a full round over 64
    K-tiles unsplit, 768x768 with 128 K-tiles as 36 tiles of 128x128 in 7 slices (not
    144 unsplit 64x64 tiles), the HBM-bound 128-row product in 4; 257 x 2440 over 63
    K-tiles as 60 tiles in 4 slices and 251 x 2033 over 173 K-tiles as 32 tiles in 8
    (not 64x64 tiles; one-row and ragged last tile rows). Sampled rows and
    columns against the oracle: integer-valued inputs bit for bit, N(0, 1) inputs to
    the accuracy rule."""
    M, N, K = shape
    p = plan_of(h, M, N, K, tgemm.BF16_F32)
    print("automatic one-round split %s: tile %dx%d split %d stages %d" % (
        shape, p["tile_m"], p["tile_n"], p["split_k"], p["stages"]), flush=True)
    assert (p["tile_m"], p["tile_n"]) == (128, 128) and p["split_k"] == splits, p
    rows, cols = inputs.sample_rows_cols(M, N, seed=11, block=128)
    a = inputs.draw((M, K), "small_int", "bf16", 201)
    b = inputs.draw((K, N), "small_int", "bf16", 202)
    sampled_check(h, o, a, b, tgemm.BF16_F32, rows, cols, exact=True)
    a, b = inputs.random_case(M, N, K, "bf16", seed=203)
    sampled_check(h, o, a, b, tgemm.BF16_F32, rows, cols)


@pytest.mark.parametrize("shape,tile,splits", [
    ((128, 4096, 2048), (128, 128, 64), 0), ((4096, 128, 2048), (128, 128, 64), 0),
    ((100, 3000, 1000), (128, 128, 64), 3), ((3000, 100, 1000), (128, 128, 64), 1),
    ((64, 8192, 640), (64, 64, 64), 0), ((8192, 64, 640), (64, 64, 64), 2),
    ((200, 5000, 1500), (256, 256, 64), 0), ((256, 3000, 700), (256, 128, 64), 0)], ids=str)
def test_single_tile_row_or_column(h, o, shape, tile, splits):
    """C covered by one row or one column of tiles: the workgroups keep the hardware's
    order (no panel is shared, so nothing is grouped on an XCD), with and without
    split-K. Every output against the oracle: integer-valued inputs bit for bit,
    N(0, 1) inputs to the accuracy rule."""
    M, N, K = shape
    p = plan_of(h, M, N, K, tgemm.BF16_F32, splits=splits, tile=tile)
    print("single tile row/column %s: tile %dx%d split %d grid %d" % (
        shape, p["tile_m"], p["tile_n"], p["split_k"], p["grid"]), flush=True)
    assert -(-M // p["tile_m"]) == 1 or -(-N // p["tile_n"]) == 1, p
    for dtype, kind in [(tgemm.BF16_F32, "bf16"), (tgemm.F16_F16, "f16")]:
        a = inputs.draw((M, K), "small_int", kind, 301)
        b = inputs.draw((K, N), "small_int", kind, 302)
        set_tile(h, tile)
        tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
        try:
            c, dc = G.run(h, a, b, dtype)
        finally:
            set_tile(h, None)
            tgemm.gemm_set_split_k(h, 0)
        assert dc.untouched_outside(), "kernel wrote outside C"
        assert np.array_equal(c, oracle_ref(o, a, b, dtype).view(G.np_int(tgemm.OUT_BYTES[dtype]))), (shape, dtype)
        a, b = inputs.random_case(M, N, K, kind, seed=303)
        check_full(h, o, a, b, dtype, tile=tile, splits=splits)


@pytest.mark.parametrize("ldc_pad,c_off", [(0, 0), (1, 0), (4, 1), (3, 2)], ids=str)
def test_split_reduction_per_tile_layouts(h, o, ldc_pad, c_off):
    """The per-tile split-K reduction (one row of 128x128 tiles, a multiple of 8 of them,
    in the hardware's order) with C rows padded and C offset from its allocation, so
    that some rows or the base leave the four-element alignment of its vector stores:
    every output format, integer-valued inputs, bit for bit against the oracle."""
    M, N, K = 128, 2048, 3000
    p = plan_of(h, M, N, K, tgemm.BF16_F32, splits=3, tile=(128, 128, 64))
    assert (p["grid"], p["split_k"]) == (16, 3), p
    for dtype, kind in [(tgemm.BF16_F32, "bf16"), (tgemm.BF16_BF16, "bf16"), (tgemm.F16_F16, "f16"), (tgemm.F16_F32, "f16")]:
        a = inputs.draw((M, K), "small_int", kind, 501)
        b = inputs.draw((K, N), "small_int", kind, 502)
        set_tile(h, (128, 128, 64))
        tgemm.check(tgemm.gemm_set_split_k(h, 3), "gemm_set_split_k")
        try:
            c, dc = G.run(h, a, b, dtype, ldc=N + ldc_pad, offs=(0, 0, c_off))
        finally:
            set_tile(h, None)
            tgemm.gemm_set_split_k(h, 0)
        assert dc.untouched_outside(), "kernel wrote outside C"
        assert np.array_equal(c, oracle_ref(o, a, b, dtype).view(G.np_int(tgemm.OUT_BYTES[dtype]))), (dtype, ldc_pad, c_off)


@pytest.mark.parametrize("shape", [(2600, 1900, 8300), (1000, 1000, 42000)], ids=str)
def test_automatic_split_of_few_256_tiles(h, o, shape):
    """At most 128 tiles of 256x256 with slices of at least 40 K-tiles: the automatic
    plan is 256x256 with S = 256 / tiles (at most 16) K-slices, ragged extents and K
    tail included. Sampled rows and columns against the oracle (integer-valued inputs
    bit for bit, N(0, 1) inputs to the accuracy rule)."""
    M, N, K = shape
    p = plan_of(h, M, N, K, tgemm.BF16_BF16)
    tiles = -(-M // 256) * -(-N // 256)
    print("automatic 256x256 split %s: tiles %d split %d" % (shape, tiles, p["split_k"]), flush=True)
    assert (p["tile_m"], p["tile_n"]) == (256, 256) and p["split_k"] == min(256 // tiles, 16), p
    rows, cols = inputs.sample_rows_cols(M, N, seed=13, block=256)
    a = inputs.draw((M, K), "small_int", "bf16", 211)
    b = inputs.draw((K, N), "small_int", "bf16", 212)
    sampled_check(h, o, a, b, tgemm.BF16_BF16, rows, cols, exact=True)
    a, b = inputs.random_case(M, N, K, "bf16", seed=213)
    sampled_check(h, o, a, b, tgemm.BF16_BF16, rows, cols)


@pytest.mark.parametrize("splits", [0, 4, 7])
def test_split_k_integer_inputs_bit_exact(h, o, splits):
    """Integer-valued inputs: every partial sum is exact, so the split result must
    equal the oracle bit for bit, whatever the slicing."""
    for M, N, K in [(96, 200, 3000), (128, 8192 // 8, 4096), (33, 40, 1100)]:
        for dtype, kind in [(tgemm.BF16_F32, "bf16"), (tgemm.F16_F16, "f16")]:
            a = inputs.draw((M, K), "small_int", kind, 41 + M)
            b = inputs.draw((K, N), "small_int", kind, 43 + N)
            tgemm.check(tgemm.gemm_set_split_k(h, splits))
            try:
                c, dc = G.run(h, a, b, dtype)
            finally:
                tgemm.gemm_set_split_k(h, 0)
            assert dc.untouched_outside()
            ref = oracle_ref(o, a, b, dtype).view(G.np_int(tgemm.OUT_BYTES[dtype]))
            assert np.array_equal(c, ref), (M, N, K, dtype, splits)


def test_split_k_deterministic_and_workspace_reuse(h, o):
    """Automatic split: identical bits on repeated calls; the handle's workspace
    grows for a larger product and is reused by a smaller one."""
    small = inputs.random_case(64, 128, 2048, "bf16", seed=51)
    large = inputs.random_case(128, 1024, 4096, "bf16", seed=52)
    assert plan_of(h, 64, 128, 2048, tgemm.BF16_F32)["split_k"] > 1
    assert plan_of(h, 128, 1024, 4096, tgemm.BF16_F32)["split_k"] > 1
    outs = []
    for a, b in [small, large, small, large]:
        c, _ = G.run(h, a, b, tgemm.BF16_F32)
        outs.append(c)
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])
    for (a, b), c in zip([small, large], outs[:2]):
        G.compare(c, oracle_ref(o, a, b, tgemm.BF16_F32).view(np.int32), "f32")


def test_split_k_setting_limits(h, o):
    assert tgemm.gemm_set_split_k(h, -1) == tgemm.ERR_INVALID_ARG
    assert tgemm.gemm_set_split_k(h, 65) == tgemm.ERR_INVALID_ARG
    # more slices than K-tiles: lowered to one slice per K-tile
    assert plan_of(h, 64, 64, 100, tgemm.BF16_F32, splits=64)["split_k"] == 2
    # 1 turns the automatic split off; other kernels ignore the setting
    assert plan_of(h, 128, 8192, 8192, tgemm.BF16_BF16, splits=1)["split_k"] == 1
    assert plan_of(h, 64, 64, 4096, tgemm.BF16_F32, splits=8, tile=(16, 16, 32))["split_k"] == 1
    assert plan_of(h, 64, 64, 4096, tgemm.I32_I32, splits=8)["split_k"] == 1
    a, b = inputs.random_case(64, 64, 4096, "bf16", seed=61)
    check_full(h, o, a, b, tgemm.BF16_F32, tile=(16, 16, 32), splits=8)
    check_full(h, o, a, b, tgemm.BF16_F32, splits=1)
    # a forced tile with a forced split
    check_full(h, o, a, b, tgemm.BF16_BF16, tile=(128, 128, 64), splits=6)


# ---------------------------------------------------------------- 4-stage pipeline

DEEP = [(1100, 1000, 6000), (1000, 1000, 1096), (1000, 1000, 4096), (136, 2056, 4096), (200, 968, 8000)]


@pytest.mark.parametrize("shape", DEEP, ids=str)
def test_deep_pipeline(h, o, shape):
    """Launches of at most one workgroup per compute unit run the 4-stage twin of
    the tile (64x64, or 128x128 cut into K-slices; K-tile counts that are not a
    multiple of the 4-step stage cycle, ragged K tails, edge tiles): random inputs to the accuracy rule,
    integer-valued inputs bit for bit, in every format and in the transposed forms."""
    M, N, K = shape
    for n, dtype in enumerate([tgemm.BF16_BF16, tgemm.F16_F32, tgemm.BF16_F32, tgemm.F16_F16]):
        p = plan_of(h, M, N, K, dtype)
        assert p["stages"] == 4, p
        a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=K + n)
        check_full(h, o, a, b, dtype)
    for kind, dtype in [("bf16", tgemm.BF16_F32), ("f16", tgemm.F16_F16)]:
        a = inputs.draw((M, K), "small_int", kind, 71)
        b = inputs.draw((K, N), "small_int", kind, 73)
        for ops in [(tgemm.OP_N, tgemm.OP_N), (tgemm.OP_N, tgemm.OP_T), (tgemm.OP_T, tgemm.OP_T)]:
            c, dc = G.run(h, a, b, dtype, op_a=ops[0], op_b=ops[1])
            assert dc.untouched_outside()
            assert np.array_equal(c, oracle_ref(o, a, b, dtype).view(G.np_int(tgemm.OUT_BYTES[dtype]))), ops


def test_deep_pipeline_forced_tile(h, o):
    """A forced 64x64 tile, or a forced 128x128 tile cut into K-slices, also gets the
    4-stage pipeline when the launch is small (an unsplit 128x128 tile keeps two A
    stages and three B stages)."""
    for tile, splits in [((128, 128, 64), 2), ((64, 64, 64), 0)]:
        p = plan_of(h, 520, 264, 2000, tgemm.BF16_F32, splits=splits, tile=tile)
        assert p["stages"] == 4 and (p["tile_m"], p["tile_n"]) == tile[:2]
        a, b = inputs.random_case(520, 264, 2000, "bf16", seed=tile[0])
        check_full(h, o, a, b, tgemm.BF16_F32, tile=tile, splits=splits)
    assert plan_of(h, 520, 264, 2000, tgemm.BF16_F32, tile=(128, 128, 64))["stages"] == 2


# ---------------------------------------------------------------- 3 A stages, 2 B stages

ADEEP = [(1100, 250, 6000), (2100, 300, 1096), (3100, 520, 2000), (2065, 257, 777), (1030, 60, 4104),
         (1300, 200, 4027)]


@pytest.mark.parametrize("shape", ADEEP, ids=str)
def test_a_deep_pipeline(h, o, shape):
    """The unsplit 256x256 tile over a C at most four tile columns wide and four times
    as tall loads A three K-steps ahead into three A stages and B two ahead into two
    (K-tile counts with every remainder of its 6-step stage cycle, ragged K tails, edge
    tiles): random inputs to the accuracy rule in every format, integer-valued inputs
    bit for bit in all four operand forms."""
    M, N, K = shape
    tile = (256, 256, 64)
    for n, dtype in enumerate([tgemm.BF16_BF16, tgemm.F16_F32, tgemm.BF16_F32, tgemm.F16_F16]):
        p = plan_of(h, M, N, K, dtype, tile=tile)
        assert (p["stages"], p["split_k"]) == (3, 1), p
        a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=K + 7 * n)
        check_full(h, o, a, b, dtype, tile=tile)
    for kind, dtype in [("bf16", tgemm.BF16_F32), ("f16", tgemm.F16_F16)]:
        a = inputs.draw((M, K), "small_int", kind, 81)
        b = inputs.draw((K, N), "small_int", kind, 83)
        ref = oracle_ref(o, a, b, dtype).view(G.np_int(tgemm.OUT_BYTES[dtype]))
        set_tile(h, tile)
        try:
            for ops in [(tgemm.OP_N, tgemm.OP_N), (tgemm.OP_N, tgemm.OP_T), (tgemm.OP_T, tgemm.OP_N),
                        (tgemm.OP_T, tgemm.OP_T)]:
                print("a-deep %s %s ops %s" % (shape, kind, ops), flush=True)
                c, dc = G.run(h, a, b, dtype, op_a=ops[0], op_b=ops[1])
                assert dc.untouched_outside()
                assert np.array_equal(c, ref), ops
        finally:
            set_tile(h, None)


@pytest.mark.parametrize("shape,splits", [((2100, 300, 6000), 3), ((1300, 200, 4027), 2), ((3100, 520, 2000), 5)],
                         ids=str)
def test_a_deep_split_k(h, o, shape, splits):
    """Three A stages in K-slices (a forced 256x256 tile over a tall, narrow C, forced
    slice counts, ragged K): integer-valued inputs bit for bit in two operand forms,
    random inputs to the accuracy rule."""
    M, N, K = shape
    tile = (256, 256, 64)
    p = plan_of(h, M, N, K, tgemm.BF16_F32, splits=splits, tile=tile)
    assert (p["stages"], p["split_k"]) == (3, splits), p
    a = inputs.draw((M, K), "small_int", "bf16", 61)
    b = inputs.draw((K, N), "small_int", "bf16", 62)
    ref = oracle_ref(o, a, b, tgemm.BF16_F32).view(np.int32)
    set_tile(h, tile)
    tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
    try:
        for ops in [(tgemm.OP_N, tgemm.OP_N), (tgemm.OP_T, tgemm.OP_T)]:
            print("a-deep split %s S %d ops %s" % (shape, splits, ops), flush=True)
            c, dc = G.run(h, a, b, tgemm.BF16_F32, op_a=ops[0], op_b=ops[1])
            assert dc.untouched_outside()
            assert np.array_equal(c, ref), ops
    finally:
        set_tile(h, None)
        tgemm.gemm_set_split_k(h, 0)
    a, b = inputs.random_case(M, N, K, "bf16", seed=K + splits)
    check_full(h, o, a, b, tgemm.BF16_BF16, tile=tile, splits=splits)


def a_deep_cases():
    """Random tall, narrow products that take three A stages on the forced 256x256 tile
    (at most 4 tile columns, at least 4 times as many tile rows): ragged M, N and K,
    leading-dimension padding, C offsets, every operand form and format."""
    rng = np.random.default_rng(777)
    dtypes = [tgemm.BF16_F32, tgemm.BF16_BF16, tgemm.F16_F32, tgemm.F16_F16]
    ops = [(tgemm.OP_N, tgemm.OP_N), (tgemm.OP_T, tgemm.OP_N), (tgemm.OP_N, tgemm.OP_T), (tgemm.OP_T, tgemm.OP_T)]
    cases = []
    for n in range(12):
        tn = int(rng.integers(1, 3))
        tm = 4 * tn + int(rng.integers(0, 2))
        M = 256 * (tm - 1) + int(rng.integers(1, 257))
        N = 256 * (tn - 1) + int(rng.integers(1, 257))
        K = int(rng.integers(65, 1500))
        pad = [0, 1, 8, 37][n % 4]
        coff = int(rng.integers(0, 9)) if n % 3 else 0
        cases.append((M, N, K, dtypes[n % 4], pad, coff, ops[(n // 2) % 4]))
    return cases


@pytest.mark.parametrize("case", a_deep_cases(), ids=str)
def test_a_deep_random(h, o, case):
    M, N, K, dtype, pad, coff, op = case
    p = plan_of(h, M, N, K, dtype, tile=(256, 256, 64))
    assert p["stages"] == 3, (case, p)
    a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=M + 3 * N + 7 * K)
    lda = (M if op[0] == tgemm.OP_T else K) + pad
    ldb = (K if op[1] == tgemm.OP_T else N) + pad
    print("a-deep random %s" % (case,), flush=True)
    check_full(h, o, a, b, dtype, tile=(256, 256, 64), lda=lda, ldb=ldb, ldc=N + pad, offs=(0, 0, coff),
               op_a=op[0], op_b=op[1])


# Two seeded shapes per branch of the automatic plan (tile, K-slices or not, pipeline, split-K
# tail), drawn from M in [100, 17000), N in [100, 9000), K in [64, 12000); the plan each one
# takes is pinned, so that a planner change that moves one shows up here.
AUTO_BRANCHES = [
    ((4630, 326, 1943), (64, 64, False, 2, False)),
    ((3076, 360, 327), (64, 64, False, 2, False)),
    ((2987, 139, 2570), (64, 64, False, 4, False)),
    ((240, 2586, 2652), (64, 64, False, 4, False)),
    ((3278, 121, 6258), (64, 64, True, 4, False)),
    ((465, 484, 4438), (64, 64, True, 4, False)),
    ((592, 6188, 3428), (128, 128, False, 2, False)),
    ((609, 5890, 6252), (128, 128, False, 2, False)),
    ((1852, 1230, 7266), (128, 128, True, 2, False)),
    ((1715, 633, 10028), (128, 128, True, 2, False)),
    ((143, 2665, 5655), (128, 128, True, 4, False)),
    ((218, 3498, 5076), (128, 128, True, 4, False)),
    ((1337, 4370, 3563), (256, 128, False, 2, False)),
    ((7032, 558, 3016), (256, 128, False, 2, False)),
    ((10719, 3285, 488), (256, 256, False, 2, False)),
    ((14474, 5504, 827), (256, 256, False, 2, False)),
    ((9429, 3744, 2837), (256, 256, False, 2, True)),
    ((3207, 5928, 6132), (256, 256, False, 2, True)),
    ((16426, 726, 9337), (256, 256, False, 3, False)),
    ((10947, 876, 304), (256, 256, False, 3, False)),
    ((1372, 3793, 10997), (256, 256, True, 2, False)),
    ((1542, 4169, 6705), (256, 256, True, 2, False)),
    ((10298, 522, 8356), (256, 256, True, 3, False)),
    ((11573, 492, 6177), (256, 256, True, 3, False)),
]


@pytest.mark.parametrize("shape,branch", AUTO_BRANCHES, ids=str)
def test_automatic_plan_branches(h, o, shape, branch):
    """Every branch of the automatic plan on ragged shapes of medium to large size (dense
    row-major operands, bf16 in and out): sampled rows and columns (one per 256, the
    first and the last) against the oracle."""
    import torch

    M, N, K = shape
    p = plan_of(h, M, N, K, tgemm.BF16_BF16)
    got = (p["tile_m"], p["tile_n"], p["split_k"] > 1, p["stages"], p["tail_split_k"] > 0)
    assert got == branch, (shape, p)
    a, b = inputs.random_case(M, N, K, "bf16", seed=M + N + K)
    print("plan branch %s %s" % (shape, branch), flush=True)
    da = torch.from_numpy(a.view(np.int16)).cuda()
    db = torch.from_numpy(b.view(np.int16)).cuda()
    dc = torch.full((M, N), G.SENTINEL[2], dtype=torch.int16, device="cuda")
    tgemm.check(tgemm.gemm_run(h, M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N, tgemm.BF16_BF16,
                               torch.cuda.current_stream().cuda_stream), "gemm_run")
    torch.cuda.synchronize()
    rows, cols = inputs.sample_rows_cols(M, N, seed=M, block=256)
    G.compare(dc[torch.from_numpy(rows).cuda()].cpu().numpy(), o.gemm_rows(a, b, rows, "bf16", "bf16").view(np.int16), "bf16")
    G.compare(dc[:, torch.from_numpy(cols).cuda()].cpu().numpy(), o.gemm_cols(a, b, cols, "bf16", "bf16").view(np.int16),
              "bf16")


# ---------------------------------------------------------------- output rounding edge cases

def test_output_rounding_edge_values(h, o):
    """One RNE rounding into bf16/f16: products that land exactly halfway between
    two output values (ties to even), values near the top of the f16 range, and
    bf16 results in the subnormal range (below 2^-126), against the oracle's
    exact rounding, element for element."""
    rng = np.random.default_rng(99)
    M, N, K = 64, 64, 32
    # halfway cases: a = 1 + 2^-8 (exact in bf16), b = e_0 + e_1 -> 1 + 2^-8 + 1 + 2^-8 etc.
    base = (1.0 + rng.integers(0, 128, size=(M, K)) / 128.0).astype(np.float32)
    base[: M // 2, 1] = 1.0  # these rows sum to a0 + 2^-8: exactly halfway between two bf16 values
    ones = np.zeros((K, N), dtype=np.float32)
    ones[0, :] = 1.0
    ones[1, :] = 2.0 ** -8   # half an ulp of bf16 in [1, 2)
    for dtype in (tgemm.BF16_BF16, tgemm.F16_F16):
        kind = "bf16" if dtype == tgemm.BF16_BF16 else "f16"
        aa = inputs.to_bits(base, kind)
        bb = inputs.to_bits(ones, kind)
        c, _ = G.run(h, aa, bb, dtype)
        ref = oracle_ref(o, aa, bb, dtype).view(np.int16)
        assert np.array_equal(c.view(np.int16), ref), dtype
    # large f16 results (sums near 60000) and tiny bf16 results (2^-130 scale)
    big = inputs.to_bits(rng.uniform(0.5, 1.0, size=(M, K)).astype(np.float32) * 64, "f16")
    bigb = inputs.to_bits(rng.uniform(0.5, 1.0, size=(K, N)).astype(np.float32) * 30, "f16")
    c, _ = G.run(h, big, bigb, tgemm.F16_F16)
    G.compare(c, oracle_ref(o, big, bigb, tgemm.F16_F16).view(np.int16), "f16")
    tiny = inputs.to_bits((rng.standard_normal((M, K)) * 2.0 ** -70).astype(np.float32), "bf16")
    tinyb = inputs.to_bits((rng.standard_normal((K, N)) * 2.0 ** -62).astype(np.float32), "bf16")
    c, _ = G.run(h, tiny, tinyb, tgemm.BF16_BF16)
    G.compare(c, oracle_ref(o, tiny, tinyb, tgemm.BF16_BF16).view(np.int16), "bf16")


# Regression: at the barrier that ends a K-step, the last fragment reads of the current
# stage may still be in flight (those consumed by the MFMAs after the barrier), so the
# refill issued right after it must go to a stage no wave still reads. Refills that
# land at once -- a K-tile past the end (a zero-length buffer), the lanes past K of a
# partial last K-tile -- are where a violation shows: one-K-tile split-K slices run
# after another product (which leaves data in LDS) lost the last substep of a slice in
# some runs, with the 64x64 tile (one MFMA block row per wave, so B's last fragments
# too are read after the barrier). Each case is repeated with a different product in
# between; every run must give the same bits, and those must meet the accuracy rule.
@pytest.mark.parametrize("shape,splits", [((256, 256, 4096), 64), ((256, 256, 4104), 0), ((128, 512, 2056), 8)],
                         ids=str)
def test_refill_after_barrier_repeatable(h, o, shape, splits):
    M, N, K = shape
    print("refill case M=%d N=%d K=%d splits=%d" % (M, N, K, splits), flush=True)
    a, b = inputs.random_case(M, N, K, "bf16", seed=97)
    xa, xb = inputs.random_case(M, N, 2048, "bf16", seed=98)
    ref = oracle_ref(o, a, b, tgemm.BF16_F32)
    first = None
    for r in range(12):
        check_full(h, o, xa, xb, tgemm.BF16_F32, splits=16)  # leaves other data in every CU's LDS
        set_tile(h, (64, 64, 64))
        tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
        try:
            c, _ = G.run(h, a, b, tgemm.BF16_F32)
        finally:
            set_tile(h, None)
            tgemm.gemm_set_split_k(h, 0)
        if first is None:
            first = c.copy()
            G.compare(c, ref.view(np.int32), "f32")
        else:
            assert np.array_equal(c, first), "run %d differs from the first run" % r


# Interior tiles are stored as 16-byte chunks staged through LDS, at whatever
# alignment C's base and row stride give them (2-byte aligned for 16-bit outputs);
# edge tiles element by element. Every combination must give the oracle's result and
# leave everything outside C untouched (neighbouring tiles share the 4-byte words
# and cache lines at their boundary when the row start is not 16-byte aligned).
@pytest.mark.parametrize("dtype,ldc_pad,c_off", [
    (tgemm.BF16_BF16, 0, 0), (tgemm.BF16_BF16, 4, 0), (tgemm.BF16_BF16, 8, 0), (tgemm.BF16_BF16, 0, 1),
    (tgemm.BF16_BF16, 0, 8), (tgemm.BF16_F32, 0, 0), (tgemm.BF16_F32, 1, 0), (tgemm.BF16_F32, 4, 0),
    (tgemm.BF16_F32, 0, 2), (tgemm.F16_F16, 0, 0), (tgemm.F16_F16, 4, 0)], ids=str)
@pytest.mark.parametrize("tile", [None, (128, 128, 64), (64, 64, 64)], ids=str)
def test_store_paths(h, o, dtype, ldc_pad, c_off, tile):
    M, N, K = 512, 512, 192
    a, b = inputs.random_case(M, N, K, G.IN_KIND[dtype], seed=71 + ldc_pad + c_off)
    check_full(h, o, a, b, dtype, tile=tile, ldc=N + ldc_pad, offs=(0, 0, c_off))


# Many launches of the same product, every output compared bit for bit with the
# first (on the device): the kernels are deterministic, so a stage refill landing
# over a fragment read still in flight (or any other race) would show up as a
# difference. The first output is also checked against the oracle on sampled rows.
@pytest.mark.parametrize("name,reps", [("square4096_bf16", 300), ("skinny128x8192x8192_bf16", 1500),
                                       ("ragged1000x777x333_bf16", 1500)])
def test_many_launches_identical(h, o, name, reps):
    torch = pytest.importorskip("torch")
    w = inputs.WORKLOADS[name]
    print("repeat case %s x %d" % (name, reps), flush=True)
    a, b = inputs.make(w)
    dtype = tgemm.DTYPES[w.dtype]
    ob = tgemm.OUT_BYTES[dtype]
    da, db = torch.from_numpy(a.view(np.int16)).cuda(), torch.from_numpy(b.view(np.int16)).cuda()
    c0 = torch.empty((w.M, w.N), dtype=G.int_dtype(ob), device="cuda")
    c1 = torch.empty_like(c0)
    sp = torch.cuda.current_stream().cuda_stream

    def run(c):
        tgemm.check(tgemm.gemm_run(h, w.M, w.N, w.K, da.data_ptr(), w.K, db.data_ptr(), w.N, c.data_ptr(), w.N,
                                   dtype, sp), "gemm_run")

    run(c0)
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(reps):
        c1.fill_(0x55)
        run(c1)
        bad += (c1 != c0).any().to(torch.int64)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0, "%d of %d launches differ from the first" % (int(bad.item()), reps)
    rows, _ = inputs.sample_rows_cols(w.M, w.N, seed=5)
    got = c0[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = o.gemm_rows(a, b, rows, w.in_kind, w.out_kind)
    G.compare(got, ref.view(G.np_int(ob)), w.out_kind)


# Pointers at odd byte addresses (the ABI accepts any alignment): A and B then go
# through the element loader, and C (not aligned to its element size) through the
# element-by-element epilogue; both must give the oracle's result.
@pytest.mark.parametrize("dtype", [tgemm.BF16_BF16, tgemm.BF16_F32], ids=["bf16_out", "f32_out"])
@pytest.mark.parametrize("shape", [(300, 200, 150), (257, 129, 64), (1, 1, 1)], ids=str)
def test_odd_byte_addresses(h, o, shape, dtype):
    import torch

    M, N, K = shape
    a, b = inputs.random_case(M, N, K, "bf16", seed=M + N + K)
    ob = tgemm.OUT_BYTES[dtype]
    # byte buffers: each matrix starts one byte into its buffer; the rest holds a fill pattern
    ba = torch.full((2 * M * K + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    bb = torch.full((2 * K * N + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    bc = torch.full((ob * M * N + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    ba[1:1 + 2 * M * K].copy_(torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)).cuda())
    bb[1:1 + 2 * K * N].copy_(torch.from_numpy(np.ascontiguousarray(b).view(np.uint8).reshape(-1)).cuda())
    p = tgemm.gemm_plan(h, M, N, K, ba.data_ptr() + 1, K, bb.data_ptr() + 1, N, bc.data_ptr() + 1, N, dtype)
    assert p["vector_loads"] == 0, p
    print("odd byte addresses %s dtype %d" % (shape, dtype), flush=True)
    tgemm.check(tgemm.gemm_run(h, M, N, K, ba.data_ptr() + 1, K, bb.data_ptr() + 1, N, bc.data_ptr() + 1, N, dtype,
                               torch.cuda.current_stream().cuda_stream), "gemm_run")
    torch.cuda.synchronize()
    host = bc.cpu().numpy()
    assert host[0] == 0x5A and np.all(host[1 + ob * M * N:] == 0x5A), "wrote outside C"
    c = host[1:1 + ob * M * N].copy().view(G.np_int(ob)).reshape(M, N)
    ref = oracle_ref(o, a, b, dtype).view(G.np_int(ob))
    G.compare(c, ref, G.OUT_KIND[dtype])


@pytest.mark.parametrize("tile,tall", [((64, 64, 64), False), ((128, 128, 64), False), ((256, 128, 64), False),
                                       ((256, 256, 64), False), ((256, 256, 64), True)], ids=str)
def test_k_step_counts(h, o, tile, tall):
    """Stage bookkeeping at the smallest K-step counts: 1 to 13 K-tiles (every remainder
    of the 6-step stage cycles, before and after one or two whole cycles; full, and with
    a partial last K-tile), 2 x 2 ragged tiles, or 9 x 2 (tall: the 256x256 tile with
    three A stages and two B stages), integer-valued inputs (exact in any order): every
    run matches the oracle bit for bit and a second run repeats it."""
    tm, tn, tk = tile
    M, N = (8 * tm + 17, tn + 5) if tall else (tm + 17, tn + 5)
    if tile == (256, 256, 64):
        assert plan_of(h, M, N, 13 * tk, tgemm.BF16_F32, tile=tile)["stages"] == (3 if tall else 2)
    for nk in range(1, 14):
        for K in (tk * nk, tk * nk - 13):
            a = inputs.draw((M, K), "small_int", "bf16", 100 + K)
            b = inputs.draw((K, N), "small_int", "bf16", 200 + K)
            ref = oracle_ref(o, a, b, tgemm.BF16_F32).view(np.int32)
            set_tile(h, tile)
            try:
                print("k-steps tile %s K %d" % (tile, K), flush=True)
                c1, _ = G.run(h, a, b, tgemm.BF16_F32)
                c2, _ = G.run(h, a, b, tgemm.BF16_F32)
            finally:
                set_tile(h, None)
            assert np.array_equal(c1, ref), (tile, K)
            assert np.array_equal(c2, c1), (tile, K)


@pytest.mark.parametrize("tile", [(64, 64, 64), (128, 128, 64)], ids=str)
def test_k_step_counts_four_stages(h, o, tile):
    """The 4-stage twins (launches of at most 256 workgroups with at least 8 K-tiles per
    slice; the 128x128 tile cut into two K-slices): K-tile counts per slice from the
    threshold up, every remainder of the 4-step stage cycle, exact against the oracle."""
    tm, tn, tk = tile
    M, N = 2 * tm + 3, 3 * tn - 7
    splits = 2 if tm == 128 else 0
    seen = set()
    for nk in (8, 9, 10, 11, 12, 16, 17, 18, 19):
        for K in (tk * nk * max(splits, 1), tk * nk * max(splits, 1) - 5):
            a = inputs.draw((M, K), "small_int", "f16", 300 + K)
            b = inputs.draw((K, N), "small_int", "f16", 400 + K)
            ref = oracle_ref(o, a, b, tgemm.F16_F32).view(np.int32)
            set_tile(h, tile)
            tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
            try:
                p = tgemm.gemm_plan(h, M, N, K, 1 << 20, K, 1 << 30, N, 1 << 34, N, tgemm.F16_F32)
                seen.add(p["stages"])
                print("4-stage k-steps tile %s K %d splits %d stages %d" % (tile, K, splits, p["stages"]), flush=True)
                c, _ = G.run(h, a, b, tgemm.F16_F32)
            finally:
                set_tile(h, None)
                tgemm.gemm_set_split_k(h, 0)
            assert np.array_equal(c, ref), (tile, K, p["stages"])
    assert 4 in seen, seen


@pytest.mark.parametrize("shape", [(1, 1, 1 << 20), (100000, 1, 512), (1, 100000, 512), (3, 70000, 3),
                                   (70000, 3, 5), (2, 2, 300001)], ids=str)
def test_degenerate_shapes(h, o, shape):
    """One output with a reduction of 2^20, a single column or row of 100,000 outputs,
    and thin products with K of 3 to 300,001: the whole C against the oracle, nothing
    written outside C; with integer-valued inputs, bit for bit."""
    M, N, K = shape
    print("degenerate %s" % (shape,), flush=True)
    a, b = inputs.random_case(M, N, K, "bf16", seed=M + 7 * N + K)
    c, dc = G.run(h, a, b, tgemm.BF16_F32)
    assert dc.untouched_outside()
    G.compare(c, oracle_ref(o, a, b, tgemm.BF16_F32).view(np.int32), "f32")
    if K <= 300001:
        ai = inputs.draw((M, K), "small_int", "bf16", 5 + M)
        bi = inputs.draw((K, N), "small_int", "bf16", 6 + N)
        c, _ = G.run(h, ai, bi, tgemm.BF16_F32)
        assert np.array_equal(c, oracle_ref(o, ai, bi, tgemm.BF16_F32).view(np.int32))
