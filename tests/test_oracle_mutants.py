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
from tests import pins, pins_bwd, pins_decode

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

# Planted mistakes in the backward pass; each must fail a backward pin.
BWD_MUTANTS = {
    "bwd_drops_rowsum": ("ds[j] = p[j] * (ds[j] - dsum);", "ds[j] = p[j] * ds[j];"),
    "bwd_rowsum_sign": ("ds[j] = p[j] * (ds[j] - dsum);", "ds[j] = p[j] * (dsum - ds[j]);"),
    "bwd_rowsum_unweighted": ("dsum += p[j] * dp;", "dsum += dp;"),
    "bwd_do_row_shifted": ("grad_score_row(P + i * N, doh + i * d, vh, N, d, dS + i * N);",
                           "grad_score_row(P + i * N, doh + ((i + 1) % N) * d, vh, N, d, dS + i * N);"),
    "bwd_dp_wrong_index": ("dp += do_row[t] * v_row[t];", "dp += do_row[t] * v_row[(t + 1) % d];"),
    "bwd_dq_no_scale": ("dqh[i * d + t] = scale * acc;", "dqh[i * d + t] = acc;"),
    "bwd_dq_uses_q": ("acc += dS[i * N + j] * kh[j * d + t];", "acc += dS[i * N + j] * qh[j * d + t];"),
    "bwd_dq_transposed_ds": ("acc += dS[i * N + j] * kh[j * d + t];", "acc += dS[j * N + i] * kh[j * d + t];"),
    "bwd_dk_uses_p": ("ak += dS[i * N + j] * qh[i * d + t];", "ak += P[i * N + j] * qh[i * d + t];"),
    "bwd_dk_transposed_ds": ("ak += dS[i * N + j] * qh[i * d + t];", "ak += dS[j * N + i] * qh[i * d + t];"),
    "bwd_dk_no_scale": ("dkh[j * d + t] = scale * ak;", "dkh[j * d + t] = ak;"),
    "bwd_dv_uses_ds": ("av += P[i * N + j] * doh[i * d + t];", "av += dS[i * N + j] * doh[i * d + t];"),
    "bwd_dv_transposed_p": ("av += P[i * N + j] * doh[i * d + t];", "av += P[j * N + i] * doh[i * d + t];"),
    "bwd_dv_uses_v": ("av += P[i * N + j] * doh[i * d + t];", "av += P[i * N + j] * vh[i * d + t];"),
    "bwd_rows_wrong_index": ("acc += s[j] * kh[j * d + t];", "acc += s[j] * kh[j * d + (t + 1) % d];"),
    "bwd_keys_first_row_skipped": ("for (long i = i0; i < N; ++i) {\n                ak +=",
                                   "for (long i = i0 + 1; i < N; ++i) {\n                ak +="),
    "bwd_keys_dv_uses_ds": ("av += P[(i - i0) * N + j] * dout[i * d + t];",
                            "av += dS[(i - i0) * N + j] * dout[i * d + t];"),
}


# Planted mistakes in the Nq x Nk (decode) entry point; each must fail a decode pin.
DECODE_MUTANTS = {
    "qk_top_left_mask": ("score_row(q + r * d, k + bh * Nk * d, Nk - Nq + i, Nk, d, scale, causal, s);",
                         "score_row(q + r * d, k + bh * Nk * d, i, Nk, d, scale, causal, s);"),
    "qk_mask_one_late": ("score_row(q + r * d, k + bh * Nk * d, Nk - Nq + i, Nk, d, scale, causal, s);",
                         "score_row(q + r * d, k + bh * Nk * d, Nk - Nq + i + 1, Nk, d, scale, causal, s);"),
    "qk_v_wrong_head": ("weighted_sum(p, v + bh * Nk * d, Nk, d, o + r * d);",
                        "weighted_sum(p, v + (bh ? bh - 1 : 0) * Nk * d, Nk, d, o + r * d);"),
    "qk_query_index": ("const long bh = r / Nq, i = r % Nq;", "const long bh = r / Nq, i = (r + 1) % Nq;"),
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
        except (AssertionError, ValueError, FloatingPointError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name!r} passed every pin"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    o = _build_mutant(tmp_path, name, old, new)
    failures = []
    for pin in pins_bwd.BWD_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, FloatingPointError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name!r} passed every backward pin"


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_mutant_is_caught(name, tmp_path):
    old, new = DECODE_MUTANTS[name]
    o = _build_mutant(tmp_path, name, old, new)
    failures = []
    for pin in pins_decode.DECODE_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, FloatingPointError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name!r} passed every decode pin"
