"""Plant one plausible mistake at a time in a copy of oracle.c (on the CPU)
and check that at least one pin catches it.  This is how the pins show they
are strong enough: a dropped term, a wrong sign, a transposed operand, a
wrong index, a leading dimension ignored, a missing absolute value, an
unfused or reordered step, a wrong checksum weight, or a transpose that
drops a column, ignores a leading dimension or mirrors its output must each
fail something."""

import os
import shutil

import pytest

import oracle
from oracle import build as obuild

import pins

SRC = obuild.SOURCE

MUTANTS = {
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float",
                          "for (int64_t k = 0; k < K - 1; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float"),
    "wrong_sign": ("p[c] += t;", "p[c] -= t;"),
    "transposed_A": ("const double a = (double)A[i * lda + k];\n            const float *brow",
                     "const double a = (double)A[k * lda + i];\n            const float *brow"),
    "window_offset_lost": ("const float *brow = B + k * ldb + j0;", "const float *brow = B + k * ldb;"),
    "abs_missing": ("if (s) s[c] += fabs(t);", "if (s) s[c] += t;"),
    "int_path_transposed_B": ("(int64_t)B[k * ldb + j];", "(int64_t)B[j * ldb + k];"),
    "fma_unfused": ("acc = fmaf(A[i * lda + k], B[k * ldb + j], acc);",
                    "acc = A[i * lda + k] * B[k * ldb + j] + acc;"),
    "checksum_weight": ("r += a * bsum[k];", "r += a * babs[k];"),
    "transpose_last_column_dropped": ("for (int64_t j = 0; j < N; ++j) B[j * ldb + i]",
                                      "for (int64_t j = 0; j < N - (N > 1); ++j) B[j * ldb + i]"),
    "transpose_ignores_lda": ("B[j * ldb + i] = A[i * lda + j];", "B[j * ldb + i] = A[i * N + j];"),
    "transpose_ignores_ldb": ("B[j * ldb + i] = A[i * lda + j];", "B[j * M + i] = A[i * lda + j];"),
    "transpose_mirrored": ("B[j * ldb + i] = A[i * lda + j];", "B[j * ldb + (M - 1 - i)] = A[i * lda + j];"),
    "first_row_skipped": ("for (int64_t i = i0; i < i1; ++i) {", "for (int64_t i = i0 + (i1 > i0 + 1); i < i1; ++i) {"),
    "a_ignores_lda": ("const double a = (double)A[i * lda + k];\n            const float *brow",
                      "const double a = (double)A[i * K + k];\n            const float *brow"),
    "b_ignores_ldb": ("const float *brow = B + k * ldb + j0;", "const float *brow = B + k * N + j0;"),
    "k_starts_at_one": ("for (int64_t k = 0; k < K; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float *brow",
                        "for (int64_t k = (K > 1); k < K; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float *brow"),
    "int_path_dropped_term": ("for (int64_t k = 0; k < K; ++k)\n                acc += (int64_t)",
                              "for (int64_t k = 0; k < K - 1; ++k)\n                acc += (int64_t)"),
    "checksums_ignore_lda": ("s += (double)A[i * lda + k];\n            sa += fabs((double)A[i * lda + k]);",
                             "s += (double)A[i * K + k];\n            sa += fabs((double)A[i * K + k]);"),
    "fma_descending_k": ("for (int64_t k = 0; k < K; ++k)\n                acc = fmaf(",
                         "for (int64_t k = K - 1; k >= 0; --k)\n                acc = fmaf("),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(before, after))
    lib_path = str(tmp_path / "liboracle_mutant.so")
    # -Wno-error: a mutant may leave a now-unused variable behind
    obuild.build(str(path), lib_path, extra=["-Wno-error"])
    lib = oracle.open_library(lib_path)
    failures = {k: v for k, v in pins.run_all(lib).items() if v}
    assert failures, f"no pin caught the planted mistake {name}"
