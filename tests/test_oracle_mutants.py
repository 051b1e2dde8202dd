"""The oracle's pins must catch plausible mistakes.

Each case copies oracle_gemm.c to a temporary directory, plants one mistake (a
transposed operand, a dropped term, a wrong sign, an index that ignores the
leading dimension, a wrong exponent bias, ...), compiles it, and runs every pin
against that build. At least one pin must fail. The real oracle is untouched.
"""
from __future__ import annotations

import os

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle_gemm.c")

MUTANTS = {
    "B_transposed": ("opB == 0 ? k * ldb + j : j * ldb + k", "opB == 0 ? j * ldb + k : k * ldb + j"),
    "A_ignores_lda": ("opA == 0 ? i * lda + k", "opA == 0 ? i * K + k"),
    "A_transposed": ("opA == 0 ? i * lda + k : k * lda + i", "opA == 0 ? k * lda + i : i * lda + k"),
    "dropped_last_k": ("for (int64_t k = 0; k < K; ++k) {\n            double a",
                       "for (int64_t k = 0; k < K - 1; ++k) {\n            double a"),
    "sign": ("c[j] += a * b[j];", "c[j] += fabs(a) * b[j];"),
    "D_signed": ("d[j] += aa * fabs(b[j]);", "d[j] += aa * b[j];"),
    "f16_bias": ("e - 25", "e - 24"),
    "f16_subnormal": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_shift": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "row_select": ("int64_t i = rows ? rows[r] : r;", "int64_t i = r;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = oracle.open_library(oracle.compile_source(str(mut), str(tmp_path / "liboracle_mut.so")))

    def ref(ops, rows=None):
        return oracle.gemm_ref(ops, rows=rows, lib=lib)

    failures = []
    for pin in pins.PINS + [pins.pin_decoders]:
        try:
            pin(ref)
        except AssertionError:
            failures.append(pin.__name__)
        except ValueError:
            failures.append(pin.__name__)
    assert failures, f"mutant {name} passed every pin"
