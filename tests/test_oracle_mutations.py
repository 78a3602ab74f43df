"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle.c, makes one plausible mistake in the copy (a dropped
term, a wrong sign or index, a transposed operand, a wrong rounding rule, a wrong
count), compiles it, and runs the pins of oracle_pins.py on that build in a
child process. The test passes when at least one pin fails (or the child dies).
"""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

MUTATIONS = {
    # the product
    "dropped_last_k_float": ("for (int64_t k = 0; k < K; ++k) {\n      double a", "for (int64_t k = 0; k < K - 1; ++k) {\n      double a"),
    "dropped_last_k_int": ("for (int64_t k = 0; k < K; ++k) {\n        uint32_t a", "for (int64_t k = 0; k < K - 1; ++k) {\n        uint32_t a"),
    "wrong_sign": ("acc[c] += a * lut[brow[c]];", "acc[c] -= a * lut[brow[c]];"),
    "transposed_b_int": ("acc[c] += a * brow[c];", "acc[c] += a * B[c * jb->ldb + k];"),
    "a_row_index_off": ("double a = lut[A[i * jb->lda + k]];", "double a = lut[A[i * jb->lda + (k + 1) % K]];"),
    "sampled_rows_ignored": ("int64_t i = jb->rows ? jb->rows[idx] : idx;\n    for (int64_t c = 0; c < nc; ++c) acc[c] = 0.0;",
                             "int64_t i = idx;\n    for (int64_t c = 0; c < nc; ++c) acc[c] = 0.0;"),
    "acc_in_float": ("double* acc = (double*)calloc", "float* acc = (float*)calloc"),
    # formats
    "f16_bias": ("ldexp((double)(f + 1024), e - 15 - 10)", "ldexp((double)(f + 1024), e - 16 - 10)"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_fraction_bits": ("ldexp((double)(f + 128), e - 127 - 7)", "ldexp((double)(f + 128), e - 127 - 8)"),
    "ties_away": ("double r = nearbyint(ldexp(ax, -q));", "double r = round(ldexp(ax, -q));"),
    "double_rounding": ("double r = nearbyint(ldexp(ax, -q));", "double r = nearbyint(ldexp((double)(float)ax, -q));"),
    "no_subnormals": ("if (lead < emin) lead = emin;", "if (0) lead = emin;"),
    "nan_encoded_as_inf": ("if (isnan(x)) return sign_bit | (exp_all << fbits) | (1u << (fbits - 1));",
                           "if (isnan(x)) return sign_bit | (exp_all << fbits);"),
    "inf_sign_dropped": ("if (isinf(x)) return sign_bit | (exp_all << fbits);", "if (isinf(x)) return exp_all << fbits;"),
    "negative_zero_dropped": ("if (ax == 0.0) return sign_bit;", "if (ax == 0.0) return 0;"),
    # counts
    "ops_halved": ("return 2 * M * N * K;", "return M * N * K;"),
    "traffic_padded_rows": ("int64_t rows = padded ? tm : m1 - m0;", "int64_t rows = tm;"),
    "traffic_b_uses_rows": ("b += depth * colsn;", "b += depth * rows;"),
    "footprint_acc_in_bytes": ("out[2] = tm * tn * s_acc;", "out[2] = tm * tn * s_in;"),
    "tile_range_unclamped": ("*hi = b < D ? b : D;", "*hi = b;"),
}

# cheap pins first; the child stops at the first failure
ORDER = ["check_counts", "check_worked_example", "check_encode_special", "check_special_cases", "check_sampled_and_strided",
         "check_against_numpy_matmul", "check_encode_f32", "check_encode_f16", "check_encode_bf16",
         "check_decode_exhaustive", "check_bruteforce_int", "check_bruteforce_float"]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_pin_is_listed():
    from tests import oracle_pins

    assert sorted(ORDER) == sorted(f.__name__ for f in oracle_pins.ALL_CHECKS)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %s" % name
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mut.so")
    oracle.compile_source(str(mutated), lib)
    script = textwrap.dedent(
        """
        import sys
        sys.path.insert(0, %r)
        import oracle
        from tests import oracle_pins
        o = oracle.Oracle(%r)
        checks = {f.__name__: f for f in oracle_pins.ALL_CHECKS}
        for name in %r:
            try:
                checks[name](o)
            except AssertionError:
                print("CAUGHT", name)
                sys.exit(0)
        print("MISSED")
        sys.exit(3)
        """
        % (ROOT, lib, ORDER)
    )
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    # a child that crashes (planted out-of-bounds access) also counts as caught
    assert "MISSED" not in out, "planted mistake %s passed every pin" % name
    assert r.returncode == 0 or r.returncode < 0 or "Error" in out, out[-2000:]
