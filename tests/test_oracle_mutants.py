"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a one-line textual change to a copy of ``oracle/ref_hgemm.c``,
compiled with gcc into a temporary directory (the real oracle is untouched).
This shows the pins in ``oracle_pins.py`` catch the plausible errors: a dropped
term, a wrong sign, a transposed operand or output, a wrong leading dimension,
a narrower accumulator, and off-by-one errors in the binary16 codec; for the
int8 variant a dropped term, an unsigned operand, a wrapped int32 sum, a
transposed output and ignored leading dimensions.
"""
import os

import pytest

import oracle as oracle_pkg
import oracle_pins

MUTANTS = {
    "drop_first_term": ("for (int64_t k = 0; k < K; ++k) s += g_dec",
                        "for (int64_t k = 1; k < K; ++k) s += g_dec"),
    "decode_drops_sign": ("return sign ? -v : v;", "return v;"),
    "ties_away_from_zero": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;",
                            "return fl + 1.0;"),
    "flush_subnormal_inputs": ("v = ldexp((double)frac, -24);", "v = 0.0;"),
    "overflow_threshold_low": ("if (a >= 65520.0)", "if (a >= 65504.0)"),
    "binary32_accumulator": ("double s = 0.0;", "float s = 0.0f;"),
    "ldc_ignored": ("C[i * ldc + j] = ref_f64_to_f16", "C[i * N + j] = ref_f64_to_f16"),
    "transposed_output": ("dot_in_order(A + i * lda, B + j * ldb, K)",
                          "dot_in_order(A + (j % M) * lda, B + (i % N) * ldb, K)"),
    "lda_ignored": ("dot_in_order(A + i * lda, B + j * ldb, K)",
                    "dot_in_order(A + i * K, B + j * ldb, K)"),
    "exponent_bias": ("(uint16_t)((e + 15) << 10)", "(uint16_t)((e + 14) << 10)"),
    "subnormal_boundary": ("if (e < -14) {", "if (e < -15) {"),
    "decode_exponent_offset": ("ldexp((double)(1024 + frac), expo - 25)",
                               "ldexp((double)(1024 + frac), expo - 24)"),
    # int8 variant
    "i8_drop_last_term": ("for (int64_t k = 0; k < K; ++k) s += (int64_t)a[k]",
                          "for (int64_t k = 0; k + 1 < K; ++k) s += (int64_t)a[k]"),
    "i8_unsigned_operand": ("s += (int64_t)a[k] * (int64_t)b[k];",
                            "s += (int64_t)(uint8_t)a[k] * (int64_t)b[k];"),
    "i8_int32_wraps": ("if (fits_int32(s)) C[i * ldc + j] = (int32_t)s;\n            else bad = 1;",
                       "C[i * ldc + j] = (int32_t)s;"),
    "i8_ldc_ignored": ("if (fits_int32(s)) C[i * ldc + j]", "if (fits_int32(s)) C[i * N + j]"),
    "i8_transposed": ("const int64_t s = idot(A + i * lda, B + j * ldb, K);",
                      "const int64_t s = idot(A + (j % M) * lda, B + (i % N) * ldb, K);"),
    # overlap micro-benchmark arithmetic
    "fma_unfused": ("y = fmaf(y, alpha, beta);", "y = (float)(y * alpha) + beta;"),
    "fma_one_step_short": ("for (int32_t it = 0; it < fma_iters; ++it)",
                           "for (int32_t it = 1; it < fma_iters; ++it)"),
    "fma_operands_swapped": ("y = fmaf(y, alpha, beta);", "y = fmaf(y, beta, alpha);"),
    "i8_ldb_ignored": ("const int64_t s = idot(A + rows[t] * lda, B + cols[t] * ldb, K);",
                       "const int64_t s = idot(A + rows[t] * lda, B + cols[t] * K, K);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    src = open(oracle_pkg.SOURCE, encoding="utf-8").read()
    assert src.count(find) == 1, f"mutation site for {name} not found exactly once"
    mpath = os.path.join(str(tmp_path), f"mut_{name}.c")
    with open(mpath, "w", encoding="utf-8") as f:
        f.write(src.replace(find, repl))
    lib = oracle_pkg.compile_source(mpath, os.path.join(str(tmp_path), f"libmut_{name}.so"))
    orc = oracle_pkg.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
