"""Checks that pin the oracle's attention of Nq queries over Nk keys
(``attention_qk``, the decode case) to facts that do not come from that entry
point: the square oracle (pinned by ``pins.py``), the unit-12 causal lesson's
statement that a single decode query may attend to every existing key, closed
forms, and the two-block merge of the FA-v1 page (eq. (17), (20); the same
identity is what a split of the key axis relies on).
"""
from __future__ import annotations

import math

import numpy as np

from tests.pins import _close, _rng


def pin_qk_square_equals_attention(o):
    r = _rng(201)
    q, k, v = (r.normal(0, 1, (2, 2, 13, 8)) for _ in range(3))
    for causal in (False, True):
        a = o.attention(q, k, v, 0.4, causal)
        b = o.attention_qk(q, k, v, 0.4, causal)
        _close(b[0], a[0], 0.0, f"Nq = Nk output causal={causal}")
        _close(b[1], a[1], 0.0, f"Nq = Nk LSE causal={causal}")


def pin_qk_last_rows(o):
    """Nq < Nk: the queries are the last Nq positions, so the result equals
    the last Nq rows of the square problem whose last query rows are q."""
    r = _rng(202)
    B, H, Nk, d = 2, 3, 29, 6
    k, v = (r.normal(0, 1, (B, H, Nk, d)) for _ in range(2))
    for Nq in (1, 2, 7, Nk):
        qfull = r.normal(0, 1, (B, H, Nk, d))
        q = qfull[:, :, Nk - Nq:]
        for causal in (False, True):
            of, lf = o.attention(qfull, k, v, 0.5, causal)
            oq, lq = o.attention_qk(np.ascontiguousarray(q), k, v, 0.5, causal)
            _close(oq, of[:, :, Nk - Nq:], 0.0, f"last rows Nq={Nq} causal={causal}")
            _close(lq, lf[:, :, Nk - Nq:], 0.0, f"last rows LSE Nq={Nq} causal={causal}")


def pin_qk_single_query_sees_all(o):
    """Unit-12 causal lesson: a single-token decode step has no future key, so
    the causal mask changes nothing."""
    r = _rng(203)
    q = r.normal(0, 1, (3, 2, 1, 16))
    k, v = (r.normal(0, 1, (3, 2, 100, 16)) for _ in range(2))
    a = o.attention_qk(q, k, v, 0.25, True)
    b = o.attention_qk(q, k, v, 0.25, False)
    _close(a[0], b[0], 0.0, "single query causal = non-causal")
    _close(a[1], b[1], 0.0, "single query LSE")


def pin_qk_zero_query(o):
    """Q = 0: uniform weights over the visible keys.  Without the mask
    O = mean_j V_j and LSE = ln Nk; with it query i sees Nk - Nq + i + 1 keys."""
    r = _rng(204)
    Nq, Nk, d = 5, 37, 4
    v = r.normal(0, 1, (1, 1, Nk, d))
    k = r.normal(0, 1, (1, 1, Nk, d))
    q = np.zeros((1, 1, Nq, d))
    oo, ll = o.attention_qk(q, k, v, 0.7, False)
    _close(oo[0, 0], np.tile(v[0, 0].mean(axis=0), (Nq, 1)), 1e-15, "Q=0 mean")
    _close(ll[0, 0], np.full(Nq, math.log(Nk)), 1e-14, "Q=0 LSE")
    oo, ll = o.attention_qk(q, k, v, 0.7, True)
    for i in range(Nq):
        n = Nk - Nq + i + 1
        _close(oo[0, 0, i], v[0, 0, :n].mean(axis=0), 1e-15, f"Q=0 causal prefix mean {i}")
        assert abs(ll[0, 0, i] - math.log(n)) <= 1e-14, f"Q=0 causal LSE {i}"


def pin_qk_key_split_merge(o):
    """Split the keys into blocks, attend to each block on its own, merge:
    LSE = ln sum_s e^(LSE_s), O = sum_s e^(LSE_s - LSE) O_s (FA-v1 page,
    eq. (17) and (20) for the statistics, (37) for the output)."""
    r = _rng(205)
    B, H, Nq, Nk, d = 2, 2, 3, 50, 8
    q = r.normal(0, 2, (B, H, Nq, d))
    k, v = (r.normal(0, 1, (B, H, Nk, d)) for _ in range(2))
    full_o, full_l = o.attention_qk(q, k, v, 0.6, False)
    for cuts in ([0, 50], [0, 7, 50], [0, 3, 20, 21, 50], list(range(0, 51, 10))):
        parts = [o.attention_qk(q, np.ascontiguousarray(k[:, :, a:b]), np.ascontiguousarray(v[:, :, a:b]), 0.6, False)
                 for a, b in zip(cuts[:-1], cuts[1:]) if b - a >= Nq]
        if len(parts) != len(cuts) - 1:
            continue
        ls = np.stack([p[1] for p in parts])
        m = ls.max(axis=0)
        lse = m + np.log(np.exp(ls - m).sum(axis=0))
        out = sum(np.exp(p[1] - lse)[..., None] * p[0] for p in parts)
        _close(lse, full_l, 1e-13, f"merged LSE cuts={cuts}")
        _close(out, full_o, 1e-13, f"merged O cuts={cuts}")


DECODE_PINS = [
    pin_qk_square_equals_attention,
    pin_qk_last_rows,
    pin_qk_single_query_sees_all,
    pin_qk_zero_query,
    pin_qk_key_split_merge,
]
