"""GPU parity with IEEE special values in the inputs and overflow of the output.

The plain definition C[i][j] = sum_k A[i][k] B[k][j] also fixes what infinities and
NaNs in A or B give: a NaN poisons every sum it enters (its row of C, or its column),
an infinity times a nonzero value is an infinity of the product's sign, an infinity
times zero is NaN, and infinities of both signs in one sum give NaN. The oracle sums in
binary64 under the same IEEE rules, so the NaN positions and the infinities of C must
match it exactly; every finite element follows the accuracy rule. Sums beyond the
output format's largest finite value round to an infinity on both sides (fp16 output:
65504 + 16 rounds to even, i.e. up to infinity; 65504 + 15 stays 65504). Subnormal
inputs and fp32 subnormal results keep their values (no flush to zero): with inputs
whose products and sums are exact in fp32, C equals the oracle bit for bit.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tiled_gemm_output_amd import inputs, tgemm

pytestmark = pytest.mark.gpu

N_, T_ = tgemm.OP_N, tgemm.OP_T
FLOAT_DTYPES = [tgemm.BF16_F32, tgemm.BF16_BF16, tgemm.F16_F32, tgemm.F16_F16]
BITS = {
    "bf16": {"pinf": 0x7F80, "ninf": 0xFF80, "nan": 0x7FC0, "one": 0x3F80},
    "f16": {"pinf": 0x7C00, "ninf": 0xFC00, "nan": 0x7E00, "one": 0x3C00},
}


@pytest.fixture(scope="module")
def h():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = tgemm.gemm_create()
    yield g
    tgemm.gemm_set_tile(g, 0, 0, 0)
    tgemm.gemm_set_split_k(g, 0)
    tgemm.gemm_destroy(g)


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def plant(a, b, kind):
    """Special values at fixed positions of op(A) (M x K) and op(B) (K x N) bits."""
    s = BITS[kind]
    a, b = a.copy(), b.copy()
    a[5, 7] = s["pinf"]
    b[7, :10] = 0  # row 5: NaN in columns 0-9 (inf * 0), +-inf elsewhere
    a[9, 3] = s["nan"]  # row 9: NaN everywhere
    a[20, 11], a[20, 12] = s["pinf"], s["ninf"]
    b[11, :], b[12, :] = s["one"], s["one"]  # row 20: inf - inf = NaN everywhere
    b[4, 40] = s["nan"]  # column 40: NaN everywhere
    b[30, 50] = s["ninf"]  # column 50: -+inf by the sign of A[i, 30]
    return a, b


def check_special(c_bits, ref_bits, kind):
    c = G.values(c_bits, kind)
    r = G.values(ref_bits, kind)
    assert np.array_equal(np.isnan(c), np.isnan(r)), "NaN positions differ: %d vs %d" % (
        int(np.isnan(c).sum()), int(np.isnan(r).sum()))
    inf = np.isinf(r)
    assert np.array_equal(np.isinf(c), inf), "infinity positions differ"
    assert np.array_equal(c[inf], r[inf]), "infinity signs differ"
    fin = np.isfinite(r)
    scale = float(np.max(np.abs(r[fin]))) if fin.any() else 0.0
    err = np.abs(c[fin] - r[fin])
    allowed = np.maximum(G.TOL * scale, G.ulp(r[fin], kind))
    assert int(np.sum(err > allowed)) == 0, "finite elements beyond the accuracy rule"
    return int(np.isnan(r).sum()), int(inf.sum())


@pytest.mark.parametrize("ops", [(N_, N_), (T_, T_)], ids=["NN", "TT"])
@pytest.mark.parametrize("plan", [
    ((64, 64, 64), None, 0),  # small output
    ((300, 260, 200), None, 0),  # automatic plan, ragged tiles
    ((1030, 1100, 700), (256, 256, 64), 0),  # the 256x256 kernel, ragged
    ((300, 260, 2000), (128, 128, 64), 3),  # split-K: specials inside one slice's partial sums
], ids=["64^3", "300x260x200", "1030x1100x700-t256", "300x260x2000-splitk3"])
def test_special_values_propagate(h, o, plan, ops):
    (M, N, K), tile, splits = plan
    for n, dtype in enumerate(FLOAT_DTYPES):
        kind, okind = G.IN_KIND[dtype], G.OUT_KIND[dtype]
        a, b = inputs.random_case(M, N, K, kind, seed=M + N + K + n)
        a, b = plant(a, b, kind)
        ref = o.gemm(a, b, kind, okind).view(G.np_int(tgemm.OUT_BYTES[dtype]))
        tgemm.check(tgemm.gemm_set_tile(h, *(tile or (0, 0, 0))), "gemm_set_tile")
        tgemm.check(tgemm.gemm_set_split_k(h, splits), "gemm_set_split_k")
        try:
            print("special values %s %s dtype %d tile %s splits %d" % ((M, N, K), ops, dtype, tile, splits), flush=True)
            c, dc = G.run(h, a, b, dtype, op_a=ops[0], op_b=ops[1])
        finally:
            tgemm.gemm_set_tile(h, 0, 0, 0)
            tgemm.gemm_set_split_k(h, 0)
        assert dc.untouched_outside()
        nans, infs = check_special(c, ref, okind)
        assert nans >= 2 * N + M - 2 and infs > 0  # the planted rows and column are there


@pytest.mark.parametrize("dtype", [tgemm.F16_F16, tgemm.BF16_BF16, tgemm.BF16_F32])
def test_output_overflow(h, o, dtype):
    """Row sums that land just below, at and beyond the output format's largest finite
    value: fp16 65504 + 15 (-> 65504) and 65504 + 16 (tie -> infinity); bf16/fp32 2^127 +
    2^127 (-> infinity, the fp32 sum overflows as well)."""
    kind, okind = G.IN_KIND[dtype], G.OUT_KIND[dtype]
    M, N, K = 70, 40, 90
    x = np.zeros((M, K), np.float32)
    bmat = np.zeros((K, N), np.float32)
    bmat[0, :] = 1.0
    bmat[1, :] = 1.0
    if kind == "f16":
        x[:, 0] = 65504.0
        x[0::2, 1] = 15.0
        x[1::2, 1] = 16.0
        x[3, 1] = -16.0
    else:
        x[:, 0] = 2.0 ** 127
        x[0::2, 1] = 2.0 ** 127
        x[1::2, 1] = -(2.0 ** 126)
    a, b = inputs.to_bits(x, kind), inputs.to_bits(bmat, kind)
    ref = o.gemm(a, b, kind, okind).view(G.np_int(tgemm.OUT_BYTES[dtype]))
    r = G.values(ref, okind)
    if okind == "f16":
        assert np.isinf(r[1::2]).sum() == (M // 2 - 1) * N and np.all(r[0::2] == 65504.0)
    else:
        assert np.all(np.isinf(r[0::2])) and np.all(np.isfinite(r[1::2]))
    c, dc = G.run(h, a, b, dtype)
    assert dc.untouched_outside()
    check_special(c, ref, okind)


@pytest.mark.parametrize("dtype", FLOAT_DTYPES)
@pytest.mark.parametrize("tile", [None, (256, 256, 64), (16, 16, 32)], ids=["auto", "t256", "t16"])
def test_subnormal_inputs_and_outputs(h, o, dtype, tile):
    """Subnormal inputs count at their value (gradual underflow, no flush to zero): fp16
    2^-20 and 2^-24 (subnormal in fp16, normal in fp32 once multiplied by 1), bf16 2^-130
    times 2^100 (normal product); and fp32 results below 2^-126 (bf16 2^-70 x 2^-72,
    summed) are kept as fp32 subnormals."""
    kind, okind = G.IN_KIND[dtype], G.OUT_KIND[dtype]
    M, N, K = 96, 80, 100
    rng = np.random.default_rng(dtype)
    x = np.zeros((M, K), np.float32)
    y = np.zeros((K, N), np.float32)
    if kind == "f16":
        x[:, :] = np.float32(2.0 ** -20) * rng.integers(1, 16, size=(M, K)).astype(np.float32)  # subnormal in fp16
        x[0::3, :] = np.float32(2.0 ** -24)  # the smallest fp16 subnormal
        y[:, :] = rng.integers(-3, 4, size=(K, N)).astype(np.float32)
    else:
        x[:, :] = np.float32(2.0 ** -130) * rng.integers(1, 8, size=(M, K)).astype(np.float32)  # subnormal in bf16
        y[:, :] = np.float32(2.0 ** 100) * rng.integers(-3, 4, size=(K, N)).astype(np.float32)
        x[0::4, :] = np.float32(2.0 ** -70) * rng.integers(1, 8, size=(M // 4, K)).astype(np.float32)
        y[:, 0::5] = np.float32(2.0 ** -72) * rng.integers(-3, 4, size=(K, N // 5)).astype(np.float32)
    a, b = inputs.to_bits(x, kind), inputs.to_bits(y, kind)
    # the stored inputs are exactly the intended values
    assert np.array_equal(G.values(a, kind if kind == "f16" else "bf16"), x.astype(np.float64))
    ref = o.gemm(a, b, kind, okind).view(G.np_int(tgemm.OUT_BYTES[dtype]))
    r = G.values(ref, okind)
    if kind == "bf16" and okind == "f32":
        sub = (np.abs(r) < 2.0 ** -126) & (r != 0)
        assert sub.sum() > 0  # some results are fp32 subnormals
    tgemm.check(tgemm.gemm_set_tile(h, *(tile or (0, 0, 0))), "gemm_set_tile")
    try:
        print("subnormals dtype %d tile %s" % (dtype, tile), flush=True)
        c, dc = G.run(h, a, b, dtype)
    finally:
        tgemm.gemm_set_tile(h, 0, 0, 0)
    assert dc.untouched_outside()
    # exact: every product and partial sum is exact in fp32 (integer multiples of one power of two)
    cv = G.values(c, okind)
    assert np.array_equal(cv, r), "max |C - R| %g at |R| %g" % (np.max(np.abs(cv - r)), np.max(np.abs(r)))
