"""Checks that pin the oracle's backward pass (dQ, dK, dV) to facts that do not
come from its backward code.

The pages state only that the backward pass recomputes S and P from Q, K and
the saved row statistics ("解析 FlashAttention（2）", section 1.2 (3); Triton
page, section 5.1) and print no gradient formulas.  The oracle's gradients are
the chain-rule derivative of its forward definition, so they are pinned here
against:
  * central finite differences of the forward oracle (itself pinned by
    ``pins.py``) on tiny inputs: the derivative by its definition;
  * float64 autograd through plain PyTorch CPU ops of the same definition;
  * closed forms (a single key, Q = 0, equal value rows, causal row 0 and the
    last key);
  * invariants of any softmax-attention gradient: the key gradients sum to 0
    (adding one vector to every key changes nothing), the value gradients sum
    to the summed output gradient (rows of P sum to 1), the identity
    sum_i <Q_i, dQ_i> = sum_j <K_j, dK_j>, linearity in dO, and equivariance
    under a joint permutation of keys and values;
  * the entry points for chosen rows (dQ) and chosen keys (dK, dV) against
    the full one.
Each ``pin_bwd_*`` takes a loaded ``oracle.Oracle`` and raises AssertionError
on disagreement.
"""
from __future__ import annotations

import numpy as np

from tests.pins import _close, _rng


def _loss(o, q, k, v, dout, scale, causal):
    """L = sum(dO * O) through the forward oracle; its gradient is the
    backward pass for output gradient dO."""
    out, _ = o.attention(q, k, v, scale, causal)
    return float(np.sum(dout * out))


def _fd_grad(o, which, q, k, v, dout, scale, causal, h=1e-6):
    args = [q.copy(), k.copy(), v.copy()]
    x = args[which]
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        x0 = x[idx]
        x[idx] = x0 + h
        lp = _loss(o, *args, dout, scale, causal)
        x[idx] = x0 - h
        lm = _loss(o, *args, dout, scale, causal)
        x[idx] = x0
        g[idx] = (lp - lm) / (2 * h)
    return g


def pin_bwd_finite_differences(o):
    r = _rng(101)
    for N, d, causal, scale in ((1, 3, False, 0.7), (4, 3, False, 0.7), (5, 2, True, 1.3),
                                (7, 4, True, 0.5), (6, 5, False, 0.35)):
        q, k, v, dout = (r.normal(0, 1, (1, 1, N, d)) for _ in range(4))
        dq, dk, dv = o.attention_backward(q, k, v, dout, scale, causal)
        for which, g in enumerate((dq, dk, dv)):
            fd = _fd_grad(o, which, q, k, v, dout, scale, causal)
            _close(g, fd, 2e-7, f"finite differences of {'QKV'[which]} N={N} d={d} causal={causal}")


def pin_bwd_torch_autograd(o):
    import torch

    r = _rng(102)
    for B, H, N, d, causal in ((1, 2, 9, 4, False), (2, 1, 13, 8, True), (1, 1, 33, 16, True)):
        scale = 1.0 / np.sqrt(d)
        q, k, v, dout = (r.normal(0, 1, (B, H, N, d)) for _ in range(4))
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        out = torch.softmax(s, dim=-1) @ tv
        out.backward(torch.tensor(dout))
        dq, dk, dv = o.attention_backward(q, k, v, dout, scale, causal)
        for name, a, b in (("dQ", dq, tq.grad), ("dK", dk, tk.grad), ("dV", dv, tv.grad)):
            _close(a, b.numpy(), 1e-12, f"autograd {name} N={N} causal={causal}")


def pin_bwd_closed_forms(o):
    r = _rng(103)
    # A single key: P = [1], so O = V and dV = dO, dQ = dK = 0.
    q, k, v, dout = (r.normal(0, 1, (1, 1, 1, 4)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = o.attention_backward(q, k, v, dout, 0.9, causal)
        _close(dv, dout, 0.0, "single key dV")
        _close(dq, np.zeros_like(dq), 0.0, "single key dQ")
        _close(dk, np.zeros_like(dk), 0.0, "single key dK")
    N, d = 11, 5
    k, v, dout = (r.normal(0, 1, (1, 1, N, d)) for _ in range(3))
    q0 = np.zeros((1, 1, N, d))
    # Q = 0: uniform weights.  Non-causal: dV_j = mean_i dO_i for every j, and
    # dK = scale * dS^T Q = 0.  Causal: P_ij = 1/(i+1) for j <= i, so
    # dV_j = sum_{i >= j} dO_i / (i+1).
    dq, dk, dv = o.attention_backward(q0, k, v, dout, 0.6, False)
    _close(dv[0, 0], np.tile(dout[0, 0].mean(axis=0), (N, 1)), 1e-14, "Q=0 dV (mean)")
    _close(dk, np.zeros_like(dk), 0.0, "Q=0 dK")
    # dQ_i = scale * sum_j P_ij (dP_ij - sum_k P_ik dP_ik) K_j with P_ij = 1/N:
    # dQ_i = (scale / N) sum_j (dO_i . (v_j - mean v)) K_j
    vbar = v[0, 0].mean(axis=0)
    ref = np.array([0.6 / N * sum((dout[0, 0, i] @ (v[0, 0, j] - vbar)) * k[0, 0, j] for j in range(N))
                    for i in range(N)])
    _close(dq[0, 0], ref, 1e-14, "Q=0 dQ")
    dq, dk, dv = o.attention_backward(q0, k, v, dout, 0.6, True)
    ref = np.array([sum(dout[0, 0, i] / (i + 1) for i in range(j, N)) for j in range(N)])
    _close(dv[0, 0], ref, 1e-14, "Q=0 causal dV (suffix sum)")
    # All value rows equal: O does not depend on the weights, so dQ = dK = 0
    # (up to rounding) and dV_j = sum_i P_ij dO_i still sums to sum_i dO_i.
    q = r.normal(0, 1, (1, 1, N, d))
    vc = np.tile(r.normal(0, 1, (1, 1, 1, d)), (1, 1, N, 1))
    for causal in (False, True):
        dq, dk, dv = o.attention_backward(q, k, vc, dout, 0.6, causal)
        _close(dq, np.zeros_like(dq), 1e-14, "equal V rows dQ")
        _close(dk, np.zeros_like(dk), 1e-14, "equal V rows dK")
    # Causal: query 0 sees only key 0, so dQ[0] = 0; the last key is seen only
    # by the last query, so dV[N-1] = P[N-1, N-1] dO[N-1] and
    # dK[N-1] = scale * dS[N-1, N-1] Q[N-1].
    dq, dk, dv = o.attention_backward(q, k, v, dout, 0.6, True)
    _close(dq[0, 0, 0], np.zeros(d), 0.0, "causal dQ[0]")
    s = 0.6 * q[0, 0, N - 1] @ k[0, 0].T
    p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    dp = dout[0, 0, N - 1] @ v[0, 0].T
    ds_last = p[-1] * (dp[-1] - p @ dp)
    _close(dv[0, 0, N - 1], p[-1] * dout[0, 0, N - 1], 1e-14, "causal last-key dV")
    _close(dk[0, 0, N - 1], 0.6 * ds_last * q[0, 0, N - 1], 1e-14, "causal last-key dK")


def pin_bwd_invariants(o):
    r = _rng(104)
    B, H, N, d = 2, 2, 10, 6
    q, k, v, d1, d2 = (r.normal(0, 1, (B, H, N, d)) for _ in range(5))
    for causal in (False, True):
        dq, dk, dv = o.attention_backward(q, k, v, d1, 0.45, causal)
        # sum over keys of dK is 0; sum over keys of dV is sum over queries of dO
        _close(dk.sum(axis=2), np.zeros((B, H, d)), 1e-13, "sum_j dK_j = 0")
        _close(dv.sum(axis=2), d1.sum(axis=2), 1e-13, "sum_j dV_j = sum_i dO_i")
        # sum_i <Q_i, dQ_i> = sum_j <K_j, dK_j> (both are scale * sum_ij dS_ij q_i.k_j)
        lhs = np.einsum("bhnd,bhnd->bh", q, dq)
        rhs = np.einsum("bhnd,bhnd->bh", k, dk)
        _close(lhs, rhs, 1e-12, "sum <Q, dQ> = sum <K, dK>")
        # linear in dO
        a, b = 0.75, -1.5
        g1 = o.attention_backward(q, k, v, d1, 0.45, causal)
        g2 = o.attention_backward(q, k, v, d2, 0.45, causal)
        g12 = o.attention_backward(q, k, v, a * d1 + b * d2, 0.45, causal)
        for x1, x2, x12, name in zip(g1, g2, g12, ("dQ", "dK", "dV")):
            _close(x12, a * x1 + b * x2, 1e-12, f"linearity in dO ({name})")
    # non-causal: permuting keys and values jointly permutes dK, dV the same
    # way and leaves dQ unchanged
    perm = r.permutation(N)
    dq, dk, dv = o.attention_backward(q, k, v, d1, 0.45, False)
    pq, pk, pv = o.attention_backward(q, k[:, :, perm], v[:, :, perm], d1, 0.45, False)
    _close(pq, dq, 1e-13, "key permutation dQ")
    _close(pk, dk[:, :, perm], 1e-13, "key permutation dK")
    _close(pv, dv[:, :, perm], 1e-13, "key permutation dV")


def pin_bwd_rows_match_full(o):
    r = _rng(105)
    B, H, N, d = 2, 3, 17, 8
    q, k, v, dout = (r.normal(0, 1, (B, H, N, d)) for _ in range(4))
    rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in (0, 5, N - 1)])
    for causal in (False, True):
        dq = o.attention_backward(q, k, v, dout, 0.3, causal)[0]
        got = o.attention_backward_dq_rows(q, k, v, dout, 0.3, causal, rows)
        _close(got, dq[rows[:, 0], rows[:, 1], rows[:, 2]], 0.0, f"dQ rows causal={causal}")


def pin_bwd_kv_keys_match_full(o):
    r = _rng(106)
    N, d = 23, 8
    q, k, v, dout = (r.normal(0, 1, (1, 1, N, d)) for _ in range(4))
    for causal in (False, True):
        _, dk, dv = o.attention_backward(q, k, v, dout, 0.3, causal)
        for keys in ([0, 7, N - 1], [N - 1], [5, 3, 5]):
            gk, gv = o.attention_backward_kv_keys(q[0, 0], k[0, 0], v[0, 0], dout[0, 0], 0.3,
                                                  causal, keys)
            _close(gk, dk[0, 0, keys], 1e-14, f"dK keys {keys} causal={causal}")
            _close(gv, dv[0, 0, keys], 1e-14, f"dV keys {keys} causal={causal}")


BWD_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_torch_autograd,
    pin_bwd_closed_forms,
    pin_bwd_invariants,
    pin_bwd_rows_match_full,
    pin_bwd_kv_keys_match_full,
]
