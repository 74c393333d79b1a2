"""Plant plausible mistakes in copies of the oracle and show the pins catch them.

Each mutant is a textual edit of ``oracle/path_oracle.c`` (a dropped term, a
wrong sign or index, a transposed operand), compiled with gcc into a temporary
directory.  The test passes when at least one pin of ``test_oracle_pins``
fails on every mutant.  This runs on the CPU only.
"""
from __future__ import annotations

import os

import pytest

import oracle
from tests.test_oracle_pins import ALL_PINS

MUTANTS = {
    "householder_sign": ("z[t] -= a * w[t];", "z[t] += a * w[t];"),
    "beta_dropped": ("double a = beta * dot(w, z, d);", "double a = dot(w, z, d);"),
    "factor_index_shift": (
        "apply_householder(z, w + (size_t)j * d, beta[j], d);",
        "apply_householder(z, w + (size_t)(j - 1) * d, beta[j - 1], d);"),
    "gate_index_shift": ("if (logf) g += logf[j];", "if (logf) g += logf[j - 1];"),
    "gate_scaled": ("s[j] = scale * dot(k + (size_t)j * d, z, d) + g;",
                    "s[j] = scale * (dot(k + (size_t)j * d, z, d) + g);"),
    "query_for_key": ("s[j] = scale * dot(k + (size_t)j * d, z, d) + g;",
                      "s[j] = scale * dot(q + (size_t)j * d, z, d) + g;"),
    "walk_starts_at_previous_query": (
        "memcpy(z, q + (size_t)i * d, sizeof(double) * (size_t)d);\n    double g",
        "memcpy(z, q + (size_t)(i > 0 ? i - 1 : 0) * d, sizeof(double) * (size_t)d);\n    double g"),
    "lse_without_max": ("lse[r] = m + log(Z);", "lse[r] = log(Z);"),
    "unnormalised_weights": ("const double a = s[j] / Z;", "const double a = s[j];"),
    "keys_as_values": ("const double *vj = vh + (size_t)j * d;",
                       "const double *vj = kh + (size_t)j * d;"),
    "diagonal_skips_query": ("for (int j = i; j >= 0; --j) {\n        s[j]",
                             "for (int j = i; j >= 0; --j) {\n        if (j < i) apply_householder(z, w + (size_t)(j + 1) * d, beta[j + 1], d);\n        s[j]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(oracle.SOURCE).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(str(mutated), lib_path)
    lib = oracle.load(lib_path)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
