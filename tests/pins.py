"""Checks that pin the fp64 oracle to facts that do not come from the oracle.

Each ``pin_*`` function takes a loaded ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with what the pages or mathematics
fix.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on builds of the oracle with one planted
mistake each and requires every such build to fail at least one of them.
"""
from __future__ import annotations

import decimal
import json
import math
import os

import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# P-1: the worked example of the unit-12 online-softmax lesson
# ---------------------------------------------------------------------------
def pin_worked_example(o):
    g = json.load(open(os.path.join(GOLDEN, "safe_softmax_worked_example.json")))
    x = np.array(g["x"], dtype=np.float64)
    assert max(g["x"]) == g["global_max"]
    assert [a - g["global_max"] for a in g["x"]] == g["shifted"]
    p, lse = o.softmax(x)
    # After the shift the largest exponential is e^0 = 1 (page 1, section 2.1)
    # and every other lies in (0, 1]: p_j / p_max = e^(shifted_j).
    shifted = np.array(g["shifted"], dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):  # a broken p fails below
        ratios = p / p[int(np.argmax(x))]
    _close(ratios, np.exp(shifted), 1e-15, "worked example ratios")
    assert np.all((p > 0) & (p <= 1)), "worked example: p outside (0, 1]"
    # LSE = global max + ln(sum of shifted exponentials)
    ref_lse = g["global_max"] + math.log(math.fsum(math.exp(s) for s in g["shifted"]))
    assert abs(lse - ref_lse) <= 1e-14, f"worked example LSE {lse} vs {ref_lse}"
    # The same numbers as one attention row: N = d = 4, scale 1, q_0 = e_1,
    # k_j = x_j e_1 gives s_0j = x_j; V = I_4 makes O[0] the softmax row itself.
    # Rows 1..3 have q = 0: uniform weights, O = 1/4, LSE = ln 4.
    Q = np.zeros((4, 4)); Q[0, 0] = 1.0
    K = np.zeros((4, 4)); K[:, 0] = x
    V = np.eye(4)
    O, L = o.attention(Q, K, V, 1.0, False)
    _close(O[0], p, 1e-16, "worked example as attention row 0")
    _close(O[1:], np.full((3, 4), 0.25), 1e-16, "q = 0 rows")
    _close(L, [ref_lse, math.log(4), math.log(4), math.log(4)], 1e-14, "worked example LSE rows")


# ---------------------------------------------------------------------------
# P-10 / library: softmax against scipy, shift invariance, masked entries
# ---------------------------------------------------------------------------
def pin_softmax_library(o):
    r = _rng(10)
    for n in (1, 2, 7, 64, 1000):
        x = r.normal(0, 3, n)
        p, lse = o.softmax(x)
        _close(p, scipy.special.softmax(x), 1e-15, f"softmax n={n}")
        assert abs(lse - scipy.special.logsumexp(x)) <= 1e-12, f"lse n={n}"
        # shift invariance: softmax(x + c) = softmax(x), LSE moves by c
        # x + c rounds x to the grid of numbers near 128 (spacing 2^-45), so
        # each logit moves by up to 2^-46; p moves by at most ~2 * 2^-46.
        p2, lse2 = o.softmax(x + 123.25)
        _close(p2, p, 1e-13, "shift invariance")
        assert abs(lse2 - (lse + 123.25)) <= 1e-11, "LSE shift"
    # masked (-inf) entries get probability exactly 0
    x = r.normal(0, 1, 9)
    x[[0, 4, 8]] = -np.inf
    p, lse = o.softmax(x)
    assert np.all(p[[0, 4, 8]] == 0.0), "masked entries must be exactly 0"
    keep = np.isfinite(x)
    _close(p[keep], scipy.special.softmax(x[keep]), 1e-15, "softmax with mask")
    assert abs(lse - scipy.special.logsumexp(x[keep])) <= 1e-13


def pin_softmax_overflow(o):
    """Logits far beyond exp's range (e^710 overflows fp64): the safe form of
    eq. (2) must still give the exact two-way split, sigma(a - b)."""
    for a, b in ((1000.0, 998.0), (-2000.0, -2003.5), (800.0, 800.0)):
        p, lse = o.softmax([a, b])
        _close(p, [scipy.special.expit(a - b), scipy.special.expit(b - a)], 1e-15,
               f"overflow regime {a},{b}")
        assert abs(lse - scipy.special.logsumexp([a, b])) <= 1e-12
    # same regime through the attention entry point (N = 2, d = 1, scale 1)
    Q = np.array([[100.0], [-100.0]])
    K = np.array([[10.0], [9.9]])
    V = np.array([[1.0], [-1.0]])
    O, L = o.attention(Q, K, V, 1.0, False)
    s = Q @ K.T
    ref = scipy.special.softmax(s, axis=1) @ V
    _close(O, ref, 1e-14, "attention with logits ~1e3")
    _close(L, scipy.special.logsumexp(s, axis=1), 1e-12, "LSE with logits ~1e3")


# ---------------------------------------------------------------------------
# P-3 + library: with V = I the output rows are the probability rows
# ---------------------------------------------------------------------------
def pin_identity_values(o):
    r = _rng(3)
    for causal in (False, True):
        N = d = 8
        Q = r.normal(0, 1, (N, d)); K = r.normal(0, 1, (N, d))
        scale = 0.37
        S = scale * (Q @ K.T)
        if causal:
            S = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, S)
        P_ref = scipy.special.softmax(S, axis=1)
        O, L = o.attention(Q, K, np.eye(N), scale, causal)
        _close(O, P_ref, 1e-15, f"V = I gives P (causal={causal})")
        _close(L, scipy.special.logsumexp(S, axis=1), 1e-14, "LSE vs logsumexp")
        _close(O.sum(axis=1), np.ones(N), 1e-15, "rows of P sum to 1")
        if causal:
            assert np.all(O[np.triu(np.ones((N, N), bool), 1)] == 0.0), \
                "masked probabilities must be exactly 0"
            assert np.all(O[np.tril(np.ones((N, N), bool))] > 0.0)
        assert np.all(O <= 1.0)


# ---------------------------------------------------------------------------
# P-7: Q = 0 closed forms (mean, causal prefix mean), including a ragged N
# ---------------------------------------------------------------------------
def pin_zero_query(o):
    r = _rng(7)
    N, d = 1000, 16
    Q = np.zeros((N, d)); K = r.normal(0, 1, (N, d)); V = r.normal(0, 1, (N, d))
    O, L = o.attention(Q, K, V, 0.125, False)
    _close(O, np.broadcast_to(V.mean(axis=0), (N, d)), 1e-13, "Q=0 mean")
    _close(L, np.full(N, math.log(N)), 1e-13, "Q=0 LSE = ln N")
    O, L = o.attention(Q, K, V, 0.125, True)
    prefix = np.cumsum(V, axis=0) / np.arange(1, N + 1)[:, None]
    _close(O, prefix, 1e-13, "Q=0 causal prefix mean")
    _close(L, np.log(np.arange(1, N + 1)), 1e-13, "Q=0 causal LSE = ln(i+1)")
    assert abs(L[999] - 6.907755278982137) <= 1e-13


# ---------------------------------------------------------------------------
# P-4: causal row 0 sees only key 0
# ---------------------------------------------------------------------------
def pin_causal_row0(o):
    r = _rng(4)
    B, H, N, d = 2, 3, 33, 8
    Q = r.normal(0, 2, (B, H, N, d)); K = r.normal(0, 2, (B, H, N, d))
    V = r.normal(0, 1, (B, H, N, d))
    O, L = o.attention(Q, K, V, 0.3, True)
    assert np.array_equal(O[:, :, 0], V[:, :, 0]), "causal O[0] must equal V[0] exactly"
    ref = 0.3 * np.einsum("bhd,bhd->bh", Q[:, :, 0], K[:, :, 0])
    _close(L[:, :, 0], ref, 1e-13, "causal LSE[0] = scale q0.k0")


# ---------------------------------------------------------------------------
# P-9, P-12, P-13: convex hull, linearity in V, joint permutation of K and V
# ---------------------------------------------------------------------------
def pin_invariants(o):
    r = _rng(12)
    B, H, N, d = 1, 2, 40, 6
    Q = r.normal(0, 1, (B, H, N, d)); K = r.normal(0, 1, (B, H, N, d))
    V1 = r.normal(0, 1, (B, H, N, d)); V2 = r.normal(0, 1, (B, H, N, d))
    for causal in (False, True):
        O1, L1 = o.attention(Q, K, V1, 0.5, causal)
        O2, L2 = o.attention(Q, K, V2, 0.5, causal)
        O3, L3 = o.attention(Q, K, 2.0 * V1 - 3.0 * V2, 0.5, causal)
        _close(O3, 2.0 * O1 - 3.0 * O2, 1e-13, "linearity in V")
        _close(L1, L2, 0.0, "LSE does not depend on V")
        for i in range(N):   # convex hull of the visible values
            vis = V1[:, :, : i + 1] if causal else V1
            assert np.all(O1[:, :, i] <= vis.max(axis=2) + 1e-14)
            assert np.all(O1[:, :, i] >= vis.min(axis=2) - 1e-14)
    perm = r.permutation(N)
    O1, L1 = o.attention(Q, K, V1, 0.5, False)
    Op, Lp = o.attention(Q, K[:, :, perm], V1[:, :, perm], 0.5, False)
    _close(Op, O1, 1e-14, "joint K/V row permutation")
    _close(Lp, L1, 1e-13, "joint K/V row permutation (LSE)")
    # permuting queries permutes output rows (non-causal)
    Oq, Lq = o.attention(Q[:, :, perm], K, V1, 0.5, False)
    _close(Oq, O1[:, :, perm], 1e-15, "query permutation")


# ---------------------------------------------------------------------------
# P-8: the large-logit regime of the N(0, 4^2) workload
# ---------------------------------------------------------------------------
def pin_large_logits(o):
    r = _rng(8)
    N, d = 256, 64
    Q = 4 * r.normal(0, 1, (N, d)); K = 4 * r.normal(0, 1, (N, d))
    V = r.normal(0, 1, (N, d))
    scale = 0.125
    O, L = o.attention(Q, K, V, scale, True)
    S = scale * (Q @ K.T)
    S = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, S)
    vmax = np.abs(V).max()
    checked = 0
    for i in range(N):
        row = np.sort(S[i][np.isfinite(S[i])])[::-1]
        if row.size < 2:
            continue
        gap = row[0] - row[1]
        if gap < 20:
            continue
        j = int(np.argmax(S[i]))
        # all other weights are at most e^-gap each
        bound = 2 * (row.size - 1) * math.exp(-gap) * vmax
        assert np.max(np.abs(O[i] - V[j])) <= bound + 1e-15, f"row {i} not near one-hot"
        checked += 1
    assert checked >= 5, "too few separated rows to check"
    assert np.all(np.isfinite(L))


# ---------------------------------------------------------------------------
# P-11: PyTorch's SDPA in float64 on the CPU (library routine)
# ---------------------------------------------------------------------------
def pin_torch_sdpa(o):
    import torch
    import torch.nn.functional as F

    g = torch.Generator().manual_seed(11)
    for (B, H, N, d, causal) in ((1, 1, 256, 64, False), (2, 3, 100, 64, True),
                                 (1, 2, 130, 128, True), (2, 2, 97, 64, False)):
        q = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
        k = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
        v = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
        scale = float(np.float32(1 / math.sqrt(d)))
        ref = F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
        s = scale * (q @ k.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        ref_lse = torch.logsumexp(s, dim=-1)
        O, L = o.attention(q.numpy(), k.numpy(), v.numpy(), scale, causal)
        _close(O, ref.numpy(), 1e-12, f"SDPA {B},{H},{N},{d},{causal}")
        _close(L, ref_lse.numpy(), 1e-12, "SDPA LSE")


# ---------------------------------------------------------------------------
# P-6: brute force in 40-digit decimal arithmetic on tiny inputs
# ---------------------------------------------------------------------------
def _dec_attention(Q, K, V, scale, causal):
    ctx = decimal.Context(prec=40)
    Dq = [[decimal.Decimal(float(x)) for x in row] for row in Q]
    Dk = [[decimal.Decimal(float(x)) for x in row] for row in K]
    Dv = [[decimal.Decimal(float(x)) for x in row] for row in V]
    sc = decimal.Decimal(float(scale))
    N, d = len(Dq), len(Dq[0])
    O, L = [], []
    for i in range(N):
        js = [j for j in range(N) if not (causal and j > i)]
        w = [ctx.exp(ctx.multiply(sc, sum((Dq[i][t] * Dk[j][t] for t in range(d)),
                                          decimal.Decimal(0)))) for j in js]
        z = sum(w, decimal.Decimal(0))
        O.append([float(ctx.divide(sum((w[a] * Dv[j][t] for a, j in enumerate(js)),
                                       decimal.Decimal(0)), z)) for t in range(d)])
        L.append(float(ctx.ln(z)))
    return np.array(O), np.array(L)


def pin_decimal_brute_force(o):
    r = _rng(6)
    for N, d in ((1, 1), (3, 2), (5, 4), (8, 3), (8, 4)):
        Q = r.normal(0, 1.5, (N, d)); K = r.normal(0, 1.5, (N, d))
        V = r.normal(0, 1, (N, d))
        for causal in (False, True):
            O, L = o.attention(Q, K, V, 0.7, causal)
            Ob, Lb = _dec_attention(Q, K, V, 0.7, causal)
            _close(O, Ob, 1e-13, f"decimal brute force N={N} d={d} causal={causal}")
            _close(L, Lb, 1e-13, "decimal brute force LSE")


# ---------------------------------------------------------------------------
# rows entry point agrees with the full entry point
# ---------------------------------------------------------------------------
def pin_rows_match_full(o):
    r = _rng(21)
    B, H, N, d = 2, 3, 77, 16
    Q = r.normal(0, 1, (B, H, N, d)); K = r.normal(0, 1, (B, H, N, d))
    V = r.normal(0, 1, (B, H, N, d))
    rows = np.array([(0, 0, 0), (1, 2, 76), (0, 1, 40), (1, 0, 13), (1, 2, 0)])
    for causal in (False, True):
        O, L = o.attention(Q, K, V, 0.25, causal)
        Or, Lr = o.attention_rows(Q, K, V, 0.25, causal, rows)
        _close(Or, O[rows[:, 0], rows[:, 1], rows[:, 2]], 0.0, "rows vs full O")
        _close(Lr, L[rows[:, 0], rows[:, 1], rows[:, 2]], 0.0, "rows vs full LSE")


ALL_PINS = [
    pin_worked_example,
    pin_softmax_library,
    pin_softmax_overflow,
    pin_identity_values,
    pin_zero_query,
    pin_causal_row0,
    pin_invariants,
    pin_large_logits,
    pin_torch_sdpa,
    pin_decimal_brute_force,
    pin_rows_match_full,
]
