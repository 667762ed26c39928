"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant is a copy of the oracle's C source with one plausible mistake
substituted in (a dropped term, a wrong sign, index or exponent, a transposed
operand, an ignored stride), compiled into a scratch directory.  A pin set that
let any of them through would not be pinning the oracle.
"""

import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "dropped_first_k_term": ("for (int64_t k = 0; k < K; ++k) {\n                    double p",
                             "for (int64_t k = 1; k < K; ++k) {\n                    double p"),
    "dropped_last_k_term_points": ("for (int64_t k = 0; k < K; ++k) {\n            double p",
                                   "for (int64_t k = 0; k < K - 1; ++k) {\n            double p"),
    "s_without_abs": ("s += fabs(p);\n                }", "s += p;\n                }"),
    "transposed_layout": ("return col_major ? X[c * ld + r] : X[r * ld + c];",
                          "return col_major ? X[r * ld + c] : X[c * ld + r];"),
    "points_transposed_b": ("decode(element(Bz, k, ji[t], ldb, b_col), fmt)",
                            "decode(element(Bz, ji[t], k, ldb, b_col), fmt)"),
    "f16_exponent_off_by_one": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_exponent_off_by_one": ("ldexp((double)(128 + f), e - 134)", "ldexp((double)(128 + f), e - 133)"),
    "bf16_sign_bit": ("int sign = (h >> 15) & 1;\n    int e = (h >> 7)", "int sign = (h >> 14) & 1;\n    int e = (h >> 7)"),
    "batch_stride_b_ignored": ("const uint16_t *Bz = B + z * strideB;\n        /* step 1",
                               "const uint16_t *Bz = B;\n        /* step 1"),
    "row_window_offset_ignored": ("element(Az, row_begin + r, k, lda, a_col)", "element(Az, r, k, lda, a_col)"),
    "negated_sum": ("c += p;\n                    s += fabs(p);", "c -= p;\n                    s += fabs(p);"),
    "rowsum_dropped_last_column": ("for (int64_t c = 0; c < C; ++c) {\n            const int64_t at",
                                   "for (int64_t c = 0; c < C - 1; ++c) {\n            const int64_t at"),
    "rowsum_col_stride_ignored": ("r * row_stride + c * col_stride;", "r * row_stride + c;"),
    "rowsum_f32_read_as_f16": ("fmt == 2 ? widen_f32", "fmt == 3 ? widen_f32"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(source=str(path), out=str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"


def test_unmutated_copy_passes(tmp_path):
    path = tmp_path / "copy.c"
    path.write_text(open(oracle.SOURCE).read())
    orc = oracle.Oracle(oracle.build(source=str(path), out=str(tmp_path / "libcopy.so")))
    for pin in oracle_pins.ALL_PINS:
        pin(orc)
    assert os.path.exists(orc.path)
