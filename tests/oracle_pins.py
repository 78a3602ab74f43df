"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each ``check_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch. ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` runs them on builds with planted mistakes and
expects each mistake to be caught. Nothing here calls the GPU library.

Independent references used (never the oracle's own formula retyped):
* the worked example's inputs as printed (tests/golden/worked_example_9x9.txt) and
  the closed form of its product, derived by hand from A[i][k] = 9i + k, B = 2A:
  C[i][j] = 2 * sum_k (9i + k)(9k + j) = 3672 + 5832 i + 72 j + 162 i j
  (sum_k k = 36, sum_k k^2 = 204 over k = 0..8);
* exact rational arithmetic (fractions.Fraction) for brute force on tiny shapes,
  with round-to-nearest-even done on rationals;
* numpy / torch format conversions and numpy's matmul as library routines;
* the pages' printed counts (tests/golden/page_counts.json).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# format parameters: significand bits (incl. implicit), min normal exponent, max exponent
FMT = {"f16": (11, -14, 15), "bf16": (8, -126, 127), "f32": (24, -126, 127)}


# ---------------------------------------------------------------------------
# independent helpers

def load_worked_example():
    a, b, cur = [], [], None
    with open(os.path.join(GOLDEN, "worked_example_9x9.txt")) as f:
        for line in f:
            s = line.strip()
            if not s or s.startswith("#"):
                continue
            if s in ("A", "B"):
                cur = a if s == "A" else b
                continue
            cur.append([int(x) for x in s.split()])
    return np.array(a, dtype=np.int32), np.array(b, dtype=np.int32)


def page_counts():
    with open(os.path.join(GOLDEN, "page_counts.json")) as f:
        return json.load(f)


def worked_closed_form():
    i = np.arange(9, dtype=np.int64)[:, None]
    j = np.arange(9, dtype=np.int64)[None, :]
    return 3672 + 5832 * i + 72 * j + 162 * i * j


def rne_fraction(q: Fraction, fmt: str):
    """Round an exact rational to the nearest value of ``fmt`` (ties to even),
    with gradual underflow and overflow to infinity. Returns a Fraction or +-inf."""
    p, emin, emax = FMT[fmt]
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * v


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def values(bits, kind):
    return f16_values(bits) if kind == "f16" else bf16_values(bits)


def _wrap32(x: int) -> int:
    x &= 0xFFFFFFFF
    return x - (1 << 32) if x >= (1 << 31) else x


# ---------------------------------------------------------------------------
# pins

def check_worked_example(o):
    """Page's 9x9 example: inputs as printed, product against the closed form."""
    from tiled_gemm_output_amd import inputs

    a_page, b_page = load_worked_example()
    a_gen, b_gen = inputs.worked_example()
    assert np.array_equal(a_page, a_gen) and np.array_equal(b_page, b_gen), "generator differs from the page"
    c = o.gemm(a_page, b_page, "i32", "i32").astype(np.int64)
    cf = worked_closed_form()
    assert np.array_equal(c, cf), "9x9 product differs from the closed form"
    assert c[0, 0] == 3672 and c[0, 8] == 4248 and c[8, 0] == 50328 and c[8, 8] == 61272
    assert int(c.sum()) == 2420280 and int(np.trace(c)) == 278640
    # the example also holds in float: every value < 2^24 is exact in fp32
    assert np.array_equal(c, 2 * (a_page.astype(np.int64) @ a_page.astype(np.int64)))
    cnt = page_counts()["worked_example_k_tiles"]
    assert o.tile_count(cnt["size"], cnt["tile"]) == cnt["value"]


def check_bruteforce_int(o, seed=7):
    """Every (M, N, K) in [1..7]^3 against exact Python integers reduced mod 2^32."""
    rng = np.random.default_rng(seed)
    for M in range(1, 8):
        for N in range(1, 8):
            for K in range(1, 8):
                a = rng.integers(-(2**31), 2**31, size=(M, K), dtype=np.int64).astype(np.int32)
                b = rng.integers(-(2**31), 2**31, size=(K, N), dtype=np.int64).astype(np.int32)
                c = o.gemm(a, b, "i32", "i32")
                al, bl = a.tolist(), b.tolist()
                for i in range(M):
                    for j in range(N):
                        s = sum(al[i][k] * bl[k][j] for k in range(K))
                        assert int(c[i, j]) == _wrap32(s), (M, N, K, i, j)


def _exact_inputs(rng, shape, kind):
    """Small integers times small powers of two: every product and every sum of a
    few of them is exact in binary64, so the exact rational result is known."""
    from tiled_gemm_output_amd import inputs

    v = rng.integers(-64, 65, size=shape).astype(np.float32) * np.exp2(rng.integers(-6, 1, size=shape)).astype(np.float32)
    return inputs.to_bits(v, kind)


def check_bruteforce_float(o, seed=11, kinds=("bf16", "f16")):
    """Tiny ragged shapes, exact rational sums, RNE to every output format."""
    rng = np.random.default_rng(seed)
    for kind in kinds:
        for M in range(1, 8, 2):
            for N in range(1, 8, 3):
                for K in range(1, 8):
                    a = _exact_inputs(rng, (M, K), kind)
                    b = _exact_inputs(rng, (K, N), kind)
                    av, bv = values(a, kind), values(b, kind)
                    exact = [[sum((Fraction(float(av[i, k])) * Fraction(float(bv[k, j])) for k in range(K)), Fraction(0))
                              for j in range(N)] for i in range(M)]
                    c64 = o.gemm(a, b, kind, "f64")
                    c32 = o.gemm(a, b, kind, "f32")
                    cbf = o.gemm(a, b, kind, "bf16")
                    ch = o.gemm(a, b, kind, "f16")
                    for i in range(M):
                        for j in range(N):
                            q = exact[i][j]
                            assert Fraction(float(c64[i, j])) == q, ("f64", kind, M, N, K)
                            assert float(c32[i, j]) == float(rne_fraction(q, "f32")), ("f32", kind, M, N, K)
                            assert float(bf16_values(cbf[i:i + 1, j:j + 1])[0, 0]) == float(rne_fraction(q, "bf16")), ("bf16", kind)
                            assert float(f16_values(ch[i:i + 1, j:j + 1])[0, 0]) == float(rne_fraction(q, "f16")), ("f16", kind)


def check_decode_exhaustive(o):
    """All 65536 patterns of each 16-bit format against numpy (binary16) and torch (bfloat16)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for kind in ("f16", "bf16"):
        got = o.decode(bits, kind)
        ref = values(bits, kind)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), kind
        assert np.array_equal(got[~nan], ref[~nan]), kind
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), kind


def _probe_doubles(rng, n):
    """Doubles over the whole range that matters for the narrow formats, plus
    exact midpoints between neighbouring narrow values (the ties)."""
    mant = rng.random(n) + 0.5
    exps = rng.integers(-150, 140, size=n)
    x = np.ldexp(mant, exps) * np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return x


def check_encode_f16(o, seed=3):
    """binary64 -> binary16 RNE against numpy's correctly rounded conversion,
    including every tie between neighbouring binary16 values."""
    rng = np.random.default_rng(seed)
    x = _probe_doubles(rng, 20000)
    x[rng.integers(0, len(x), 200)] = 0.0
    # ties: midpoints of consecutive finite binary16 values (both signs)
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    lo = f16_values(h[:-1])
    hi = f16_values(h[1:])
    mids = (lo + hi) / 2.0  # exact in binary64
    x = np.concatenate([x, mids, -mids, mids + np.spacing(mids), mids - np.spacing(mids), [65504.0, 65519.99, 65520.0, 1e6]])
    got = o.encode(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), int(np.sum(got != ref))


def check_encode_special(o):
    """Non-finite values and signed zeros: NaN stays NaN (the quiet NaN with the
    input's sign), infinities keep their sign, -0.0 stays -0.0, in every output
    format. Expected bits from numpy's binary64 -> binary16 / binary32 conversions;
    for bfloat16, the upper half of the binary32 pattern (bfloat16 is binary32's
    upper half, and these values need no rounding)."""
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0])
    with np.errstate(invalid="ignore"):
        f32 = x.astype(np.float32).view(np.uint32)
        want = {
            "f16": x.astype(np.float16).view(np.uint16),
            "f32": f32,
            "bf16": (f32 >> 16).astype(np.uint16),
        }
    # the patterns themselves: quiet NaN, infinity and zero of each format, sign bit set for the negatives
    assert [hex(v) for v in want["f16"]] == ["0x7e00", "0xfe00", "0x7c00", "0xfc00", "0x0", "0x8000"]
    assert [hex(v) for v in want["f32"]] == ["0x7fc00000", "0xffc00000", "0x7f800000", "0xff800000", "0x0",
                                             "0x80000000"]
    assert [hex(v) for v in want["bf16"]] == ["0x7fc0", "0xffc0", "0x7f80", "0xff80", "0x0", "0x8000"]
    for kind, ref in want.items():
        got = o.encode(x, kind)
        assert np.array_equal(got, ref), (kind, [hex(v) for v in got], [hex(v) for v in ref])
    # an infinite or NaN input flows through the product as in IEEE binary64
    a = np.array([[np.inf, 1.0], [np.nan, 0.0], [1.0, -0.0]])
    b = np.array([[2.0], [3.0]])
    for kind, enc in (("bf16", "bf16"), ("f16", "f16")):
        ab = np.asarray(o.encode(a.ravel(), enc), dtype=np.uint16).reshape(a.shape)
        bb = np.asarray(o.encode(b.ravel(), enc), dtype=np.uint16).reshape(b.shape)
        c = o.gemm(ab, bb, kind, "f32").astype(np.float64)
        assert c[0, 0] == np.inf and np.isnan(c[1, 0]) and c[2, 0] == 2.0, c


def check_encode_f32(o, seed=4):
    rng = np.random.default_rng(seed)
    x = np.ldexp(rng.random(20000) + 0.5, rng.integers(-160, 135, size=20000))
    x *= np.where(rng.random(20000) < 0.5, -1.0, 1.0)
    f = rng.random(5000).astype(np.float32) + np.float32(1)
    mids = (f.astype(np.float64) + np.nextafter(f, np.float32(3)).astype(np.float64)) / 2.0
    x = np.concatenate([x, mids, -mids])
    got = o.encode(x, "f32")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, ref), int(np.sum(got != ref))


def check_encode_bf16(o, seed=5):
    """binary64 -> bfloat16 RNE. (1) binary32-representable inputs against torch's
    binary32 -> bfloat16 conversion (a single rounding, so it is the reference);
    (2) arbitrary doubles against RNE on exact rationals -- this catches double
    rounding through binary32; (3) hand-made ties."""
    from tiled_gemm_output_amd import inputs

    rng = np.random.default_rng(seed)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, size=20000))).astype(np.float32)
    f = f[np.isfinite(f)]
    got = o.encode(f.astype(np.float64), "bf16")
    ref = inputs.f32_to_bf16_bits(f)
    assert np.array_equal(got, ref), int(np.sum(got != ref))
    x = _probe_doubles(rng, 3000)
    got = o.encode(x, "bf16")
    for xi, gi in zip(x.tolist(), got.tolist()):
        r = rne_fraction(Fraction(xi), "bf16")
        gv = float(bf16_values(np.array([[gi]], dtype=np.uint16))[0, 0])
        assert gv == float(r), (xi, gi)
    one = 1.0
    cases = {
        one + 2.0**-8: 0x3F80,             # exact tie between 1 and 1 + 2^-7 -> even (1)
        one + 2.0**-8 + 2.0**-40: 0x3F81,  # just above the tie -> up (double rounding would give 1)
        one + 3 * 2.0**-8: 0x3F82,         # tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
        -(one + 2.0**-8 + 2.0**-40): 0xBF81,
        2.0**128 * (1 - 2.0**-9): 0x7F80,  # tie between the largest finite and 2^128 -> infinity
        2.0**-133: 0x0001,                 # smallest subnormal
        2.0**-134: 0x0000,                 # tie between 0 and the smallest subnormal -> 0
        3 * 2.0**-135: 0x0001,
    }
    for xv, bits in cases.items():
        assert int(o.encode([xv], "bf16")[0]) == bits, (xv, hex(bits))


def check_against_numpy_matmul(o, seed=21):
    """Non-square random products against numpy's float64 matmul of the decoded
    inputs (a library routine, different summation order): agreement to within the
    binary64 summation bound catches a transposed operand, a wrong index or a
    dropped term."""
    rng = np.random.default_rng(seed)
    from tiled_gemm_output_amd import inputs

    for kind, (M, N, K) in [("bf16", (37, 29, 53)), ("f16", (23, 41, 19)), ("bf16", (5, 64, 130))]:
        a = inputs.to_bits(rng.standard_normal((M, K)).astype(np.float32), kind)
        b = inputs.to_bits(rng.standard_normal((K, N)).astype(np.float32), kind)
        av, bv = values(a, kind), values(b, kind)
        ref = av @ bv
        bound = K * 2.0**-52 * (np.abs(av) @ np.abs(bv))
        c = o.gemm(a, b, kind, "f64")
        assert np.all(np.abs(c - ref) <= bound + 1e-300), kind
        c32 = o.gemm(a, b, kind, "f32")
        assert np.all(np.abs(c32 - ref) <= 2.0**-24 * np.abs(ref) + bound * 2 + 1e-300), kind
    # integers: numpy int64 matmul reduced mod 2^32
    a = rng.integers(-(2**31), 2**31, size=(19, 33), dtype=np.int64).astype(np.int32)
    b = rng.integers(-(2**31), 2**31, size=(33, 11), dtype=np.int64).astype(np.int32)
    ref = ((a.astype(np.int64) @ b.astype(np.int64)) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    assert np.array_equal(o.gemm(a, b, "i32", "i32"), ref)


def check_special_cases(o, seed=31):
    """Identity, zero and K = 1 (outer product) are exact in every format."""
    from tiled_gemm_output_amd import inputs

    rng = np.random.default_rng(seed)
    for kind in ("bf16", "f16"):
        a = inputs.to_bits(rng.standard_normal((13, 17)).astype(np.float32), kind)
        eye = inputs.to_bits(np.eye(17, dtype=np.float32), kind)
        assert np.array_equal(o.gemm(a, eye, kind, kind), a), kind
        assert np.array_equal(o.gemm(a, eye, kind, "f32"), values(a, kind).astype(np.float32)), kind
        z = np.zeros((13, 17), dtype=np.uint16)
        assert not np.any(o.gemm(z, eye, kind, "f32")), kind
        col = inputs.to_bits(rng.standard_normal((9, 1)).astype(np.float32), kind)
        row = inputs.to_bits(rng.standard_normal((1, 7)).astype(np.float32), kind)
        outer = (values(col, kind) @ values(row, kind)).astype(np.float32)  # one exact product per entry
        assert np.array_equal(o.gemm(col, row, kind, "f32"), outer), kind
    eye_i = np.eye(6, dtype=np.int32)
    a = rng.integers(-(2**31), 2**31, size=(4, 6), dtype=np.int64).astype(np.int32)
    assert np.array_equal(o.gemm(a, eye_i, "i32", "i32"), a)


def check_sampled_and_strided(o, seed=41):
    """Sampled rows/columns and non-dense leading dimensions agree with the full product."""
    from tiled_gemm_output_amd import inputs

    rng = np.random.default_rng(seed)
    big_a = inputs.to_bits(rng.standard_normal((40, 50)).astype(np.float32), "bf16")
    big_b = inputs.to_bits(rng.standard_normal((45, 60)).astype(np.float32), "bf16")
    a, b = big_a[:31, :37], big_b[:37, :43]  # views with lda = 50, ldb = 60
    full = o.gemm(np.ascontiguousarray(a), np.ascontiguousarray(b), "bf16", "f64")
    assert np.array_equal(o.gemm(a, b, "bf16", "f64"), full)
    rows, cols = np.array([0, 5, 30]), np.array([0, 7, 42])
    assert np.array_equal(o.gemm_rows(a, b, rows, "bf16", "f64"), full[rows])
    assert np.array_equal(o.gemm_cols(a, b, cols, "bf16", "f64"), full[:, cols])
    ia = rng.integers(-1000, 1000, size=(12, 9)).astype(np.int32)
    ib = rng.integers(-1000, 1000, size=(9, 14)).astype(np.int32)
    fi = o.gemm(ia, ib, "i32", "i32")
    assert np.array_equal(o.gemm_rows(ia, ib, [3, 11], "i32", "i32"), fi[[3, 11]])
    assert np.array_equal(o.gemm_cols(ia, ib, [0, 13], "i32", "i32"), fi[:, [0, 13]])


def check_counts(o, seed=51):
    """The pages' printed counts, and the closed forms of the no-reuse model
    against the tile-by-tile walk on random shapes."""
    pc = page_counts()
    assert o.ops(128, 128, 128) == pc["ops_128_cubed"]["value"]
    t = pc["traffic_128_cubed_16x16x32"]
    a, b, c = o.traffic_bytes(128, 128, 128, t["tile_m"], t["tile_n"], t["tile_k"], t["input_bytes"], t["output_bytes"])
    assert (a, b, c) == (t["A_kib"] * 1024, t["B_kib"] * 1024, t["C_kib"] * 1024)
    assert a + b + c == t["total_kib"] * 1024
    for tk in pc["traffic_tile_k_invariant"]["tile_k_values"]:
        assert o.traffic_bytes(128, 128, 128, 16, 16, tk, 2, 4) == (a, b, c)
    fp = pc["footprint_16x16x32"]
    fa, fb, fc = o.footprint_bytes(16, 16, 32, 2, 4)
    assert (fa, fb, fc) == (fp["A_kib"] * 1024, fp["B_kib"] * 1024, fp["C_kib"] * 1024)
    assert fa + fb + fc == fp["total_kib"] * 1024
    e = pc["edge_96_by_64"]
    assert o.tile_count(96, 64) == e["full"] + e["partial"]
    assert o.tile_range(0, 64, 96) == (0, 64) and o.tile_range(1, 64, 96) == (64, 64 + e["partial_size"])
    tr = pc["tile_4_over_10"]["ranges"]
    assert o.tile_count(10, 4) == len(tr)
    assert [list(o.tile_range(i, 4, 10)) for i in range(len(tr))] == tr
    # closed forms ("Count the repeated reads"): A = M*K*ceil(N/tn), B = K*N*ceil(M/tm), C = M*N
    rng = np.random.default_rng(seed)
    for _ in range(200):
        M, N, K = (int(x) for x in rng.integers(1, 300, size=3))
        tm, tn, tk = (int(x) for x in rng.integers(1, 80, size=3))
        ea, eb, ec = o.traffic_elems(M, N, K, tm, tn, tk)
        assert ea == M * K * (-(-N // tn)) and eb == K * N * (-(-M // tm)) and ec == M * N, (M, N, K, tm, tn, tk)
        pa, pb, pcc = o.traffic_elems(M, N, K, tm, tn, tk, padded=True)
        nm, nn, nk = -(-M // tm), -(-N // tn), -(-K // tk)
        assert (pa, pb, pcc) == (nm * nn * nk * tm * tk, nm * nn * nk * tk * tn, nm * nn * tm * tn)
        assert pa >= ea and pb >= eb and pcc >= ec
    # the ragged workloads: actual-range count vs the padded overestimate (tile 64, bf16 in, fp32 out)
    assert sum(o.traffic_bytes(96, 96, 96, 64, 64, 64, 2, 4)) == 96 * 96 * 2 * 2 + 96 * 96 * 2 * 2 + 96 * 96 * 4
    assert sum(o.traffic_bytes(96, 96, 96, 64, 64, 64, 2, 4, padded=True)) == 8 * 4096 * 2 * 2 + 4 * 4096 * 4
    assert o.ops(1000, 777, 333) == 517482000


ALL_CHECKS = [
    check_worked_example,
    check_encode_special,
    check_bruteforce_int,
    check_bruteforce_float,
    check_decode_exhaustive,
    check_encode_f16,
    check_encode_f32,
    check_encode_bf16,
    check_against_numpy_matmul,
    check_special_cases,
    check_sampled_and_strided,
    check_counts,
]
