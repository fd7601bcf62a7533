"""Every plausible single mistake planted in the oracle must fail a pin.

Each mutant is a copy of ``oracle/oracle.c`` with one textual change (a
dropped term, a wrong sign, an off-by-one mask, a transposed operand, ...),
compiled on the CPU into a temporary library and run through all pins.  All
mutated index expressions stay inside the arrays, so a mutant can give wrong
numbers but never read out of bounds.
"""
import os

import pytest

import oracle
from oracle import oracle as oracle_mod
from tests import pins

MUTANTS = {
    "dot_wrong_index": ("dot += q_row[t] * k_row[t];", "dot += q_row[t] * k_row[(t + 1) % d];"),
    "k_transposed": ("dot += q_row[t] * k_row[t];", "dot += q_row[t] * k_head[t * N + j];"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "scale_squared": ("s[j] = scale * dot;", "s[j] = scale * scale * dot;"),
    "mask_off_by_one": ("if (causal && j > i) {", "if (causal && j >= i && j > 0) {"),
    "mask_reversed": ("if (causal && j > i) {", "if (causal && j < i) {"),
    "mask_ignored": ("if (causal && j > i) {", "if (causal && j > N) {"),
    "max_reversed": ("if (x[j] > m)\n            m = x[j];", "if (x[j] < m && x[j] != -INFINITY)\n            m = x[j];"),
    "max_not_subtracted": ("exp(x[j] - m);", "exp(x[j]);"),
    "shift_sign": ("exp(x[j] - m);", "exp(m - x[j]);"),
    "sum_drops_first": ("        l += p[j];", "        if (j) l += p[j];"),
    "no_normalise": ("p[j] = p[j] / l;", "p[j] = p[j] / (l > 1.0 ? 1.0 : 1.0);"),
    "lse_missing_max": ("return m + log(l);", "return log(l);"),
    "lse_log2": ("return m + log(l);", "return m + log2(l);"),
    "v_rows_reversed": ("const double *v_row = v_head + j * d;", "const double *v_row = v_head + (N - 1 - j) * d;"),
    "v_transposed": ("o_row[t] += p[j] * v_row[t];", "o_row[t] += p[j] * v_head[t * N + j];"),
    "q_row_shifted": ("score_row(qh + i * d, kh, i, N, d, scale, causal, s);",
                      "score_row(qh + (i ? i - 1 : 0) * d, kh, i, N, d, scale, causal, s);"),
    "q_row_shifted_full": ("score_row(qh + i * d, kh, i, N, d, scale, causal, S + i * N);",
                           "score_row(qh + (i ? i - 1 : 0) * d, kh, i, N, d, scale, causal, S + i * N);"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle_mod.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(mutated)
    lib = tmp_path / f"lib{name}.so"
    oracle.build(str(path), str(lib), extra_flags=("-w",))
    return oracle.Oracle(str(lib))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    o = _build_mutant(tmp_path, name, old, new)
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, FloatingPointError) as e:
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name!r} passed every pin"
