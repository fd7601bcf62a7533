"""Tile-by-tile restatements of the pages' algorithms, in numpy fp64.

TEST INFRASTRUCTURE ONLY.  These functions follow the pages' steps in the
pages' notation so that the tests can pin two claims the pages make:

* tiling the score matrix and merging per-tile softmax statistics gives the
  same O as the untiled definition (page "解析 FlashAttention（2）", sections
  2.2-2.7 and 3.3-3.12; lesson "在线 Softmax 与 FlashAttention", QK^T tiling
  and online-softmax parts);
* the loop order (key/value blocks outside, as in the first page's
  Algorithm 1, or query blocks outside, as in the FlashAttention-2 loop of the
  unit-12 loop-order lesson and the pseudo-code of the Triton page section 2.2)
  does not change the result;
* skipping key tiles that lie wholly in the causal future is an exact
  elimination (unit-12 causal-mask lesson).

They are checked against ``oracle.c`` (the plain definition) in the tests; the
HIP library never sees them.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# Softmax statistics (page 1, section 2)
# ---------------------------------------------------------------------------
def local_stats(x: np.ndarray):
    """Local statistics of one block x^(b) (eq. (7)-(9) / (13)-(15)):
    m = max_j x_j, f = e^(x - m), l = sum f.  A block whose entries are all
    -inf (fully masked) has m = -inf, f = 0, l = 0."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x) if x.size else NEG_INF
    if m == NEG_INF:
        return NEG_INF, np.zeros_like(x), 0.0
    f = np.exp(x - m)
    return m, f, float(np.sum(f))


def rebase(m_from: float, m_to: float) -> float:
    """The factor e^(m_from - m_to) that moves an exponential sum from base
    m_from to base m_to (eq. (18)-(19)).  A state that has seen nothing
    (m_from = -inf) contributes nothing: factor 0."""
    if m_from == NEG_INF:
        return 0.0
    return math.exp(m_from - m_to)


def merge(m1: float, l1: float, m2: float, l2: float):
    """Two-block merge, eq. (17) and (20):
    m_new = max(m1, m2); l_new = e^(m1 - m_new) l1 + e^(m2 - m_new) l2."""
    m_new = max(m1, m2)
    if m_new == NEG_INF:
        return NEG_INF, 0.0
    return m_new, rebase(m1, m_new) * l1 + rebase(m2, m_new) * l2


def softmax_by_blocks(x: np.ndarray, block: int):
    """Softmax of one vector processed block by block: keep each block's local
    softmax and (m, l), update the global (m_max, l_all) after every block
    (eq. (17), (20), (28), (29)), then globalise every local softmax with
    eq. (26)/(27).  Returns (softmax, m_max, l_all)."""
    x = np.asarray(x, dtype=np.float64)
    blocks = [x[s:s + block] for s in range(0, x.size, block)]
    m_max, l_all = NEG_INF, 0.0
    local = []
    for xb in blocks:
        mb, fb, lb = local_stats(xb)
        local.append((mb, fb, lb))
        m_max, l_all = merge(m_max, l_all, mb, lb)
    out = []
    for mb, fb, lb in local:
        if lb == 0.0:
            out.append(np.zeros_like(fb))
            continue
        sm_local = fb / lb                          # eq. (10) / (16)
        out.append(sm_local * lb * rebase(mb, m_max) / l_all)  # eq. (26)/(27)
    return np.concatenate(out) if out else x.copy(), m_max, l_all


def streaming_stats(x: np.ndarray):
    """Element-by-element online statistics (unit-12 online-softmax lesson):
    m_t = max(m_{t-1}, x_t), l_t = l_{t-1} e^(m_{t-1} - m_t) + e^(x_t - m_t).
    Returns (m_n, l_n)."""
    m, l = NEG_INF, 0.0
    for xt in np.asarray(x, dtype=np.float64):
        m, l = merge(m, l, float(xt), 1.0 if xt != NEG_INF else 0.0)
    return m, l


# ---------------------------------------------------------------------------
# Causal tile classes (unit-12 causal-mask lesson)
# ---------------------------------------------------------------------------
def causal_tile_class(r0: int, r1: int, c0: int, c1: int) -> str:
    """Query rows [r0, r1) against key columns [c0, c1) under the mask j <= i:
    'skip' when even the smallest key is beyond the largest query (c0 >= r1,
    i.e. c0 > r1 - 1), 'past' when even the largest key is visible to the
    smallest query (c1 - 1 <= r0), otherwise 'diag' (the tile straddles the
    diagonal and needs an element-wise mask)."""
    if c0 >= r1:
        return "skip"
    if c1 - 1 <= r0:
        return "past"
    return "diag"


def _scores(Qi, Kj, rows, cols, scale, causal):
    S = scale * (Qi @ Kj.T)
    if causal:
        S = np.where(cols[None, :] > rows[:, None], NEG_INF, S)
    return S


# ---------------------------------------------------------------------------
# Page 1, section 4: Algorithm 1 (key/value blocks outside, query blocks
# inside, O / l / m kept in "HBM" and updated with eq. (37) every step)
# ---------------------------------------------------------------------------
def algorithm1(Q, K, V, Br: int, Bc: int, scale: float, causal: bool,
               skip_future: bool = True):
    """Q, K, V: [N, d] float64.  Returns (O, LSE).  Fully masked rows inside a
    tile contribute nothing (their local l is 0)."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    N, d = Q.shape
    O = np.zeros((N, d))                 # Algorithm 1, initialisation step
    l = np.zeros(N)
    m = np.full(N, NEG_INF)
    Tr, Tc = -(-N // Br), -(-N // Bc)
    for j in range(Tc):                  # outer loop over K_j, V_j
        c0, c1 = j * Bc, min(N, (j + 1) * Bc)
        Kj, Vj = K[c0:c1], V[c0:c1]
        cols = np.arange(c0, c1)
        for i in range(Tr):              # inner loop over Q_i, O_i, l_i, m_i
            r0, r1 = i * Br, min(N, (i + 1) * Br)
            if causal and skip_future and causal_tile_class(r0, r1, c0, c1) == "skip":
                continue
            rows = np.arange(r0, r1)
            Sij = _scores(Q[r0:r1], Kj, rows, cols, scale, causal)
            for r in range(r1 - r0):     # rows are independent (section 3.9)
                mt, Pt, lt = local_stats(Sij[r])       # m~, P~, l~
                g = r0 + r
                m_new, l_new = merge(m[g], l[g], mt, lt)
                if l_new == 0.0:
                    continue
                # eq. (37): O_i <- diag(l_new)^-1 (diag(l) e^(m - m_new) O_i
                #                                  + e^(m~ - m_new) P~ V_j)
                O[g] = (l[g] * rebase(m[g], m_new) * O[g]
                        + rebase(mt, m_new) * (Pt @ Vj)) / l_new
                m[g], l[g] = m_new, l_new
    lse = m + np.log(l)
    return O, lse


# ---------------------------------------------------------------------------
# Query blocks outside, key/value blocks inside, unnormalised accumulator and
# one final division (unit-12 loop-order lesson; Triton page section 2.2)
# ---------------------------------------------------------------------------
def q_outer(Q, K, V, Br: int, Bc: int, scale: float, causal: bool,
            skip_future: bool = True):
    """Q, K, V: [N, d] float64.  Returns (O, LSE)."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    N, d = Q.shape
    O = np.empty((N, d))
    lse = np.empty(N)
    for r0 in range(0, N, Br):
        r1 = min(N, r0 + Br)
        rows = np.arange(r0, r1)
        Qi = Q[r0:r1]
        acc = np.zeros((r1 - r0, d))    # O~: not yet divided by l
        l = np.zeros(r1 - r0)
        m = np.full(r1 - r0, NEG_INF)
        for c0 in range(0, N, Bc):
            c1 = min(N, c0 + Bc)
            if causal and skip_future and causal_tile_class(r0, r1, c0, c1) == "skip":
                continue
            cols = np.arange(c0, c1)
            S = _scores(Qi, K[c0:c1], rows, cols, scale, causal)
            m_new = np.maximum(m, S.max(axis=1))       # new running maximum
            # alpha from the OLD m, before m is replaced
            alpha = np.array([rebase(a, b) for a, b in zip(m, m_new)])
            with np.errstate(invalid="ignore"):
                P = np.where(S == NEG_INF, 0.0, np.exp(S - m_new[:, None]))
            l = alpha * l + P.sum(axis=1)
            acc = alpha[:, None] * acc + P @ V[c0:c1]  # rescale, then add
            m = m_new
        O[r0:r1] = acc / l[:, None]
        lse[r0:r1] = m + np.log(l)
    return O, lse
