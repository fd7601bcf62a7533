"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph on
ROCm): every replay, with new inputs copied into the captured tensors and
eager work and synchronisations between replays, gives the eager result bit
for bit.  The kernels allocate nothing, keep no state between calls and
enqueue no memset, so a captured call is the same work as an eager one.
"""
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

pytestmark = pytest.mark.gpu


def _draws(w, n):
    out = []
    for i in range(n):
        wi = inputs.Workload(w.name, w.B, w.H, w.N, w.d, w.dtype, w.dist, w.causal,
                             seed=w.seed + 100 * i)
        out.append(tuple(t.cuda() for t in inputs.make_qkv(wi)))
    return out


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # warm-up outside the graph (allocations, library load)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    return g, res


@pytest.mark.parametrize("d,causal", [(128, True), (64, False), (80, True)])
def test_forward_graph_replays(d, causal):
    w = inputs.Workload(f"graph_fwd_d{d}", 2, 4, 1000, d, "bf16", "normal", causal, seed=31000 + d)
    draws = _draws(w, 3)
    q, k, v = (t.clone() for t in draws[0])
    g, (o, lse) = _capture(lambda: fa.forward(q, k, v, causal=causal, scale=w.scale))
    for i, (qi, ki, vi) in enumerate(draws):
        q.copy_(qi); k.copy_(ki); v.copy_(vi)
        g.replay()
        torch.cuda.synchronize()
        o_e, l_e = fa.forward(qi, ki, vi, causal=causal, scale=w.scale)   # eager, between replays
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, l_e), f"replay {i}"


def test_backward_graph_replays():
    w = inputs.Workload("graph_bwd", 1, 3, 700, 128, "bf16", "normal", True, seed=32000)
    draws = _draws(w, 3)
    dout0 = inputs.make_dout(w).cuda()
    q, k, v = (t.clone() for t in draws[0])
    dout = dout0.clone()

    def step():
        o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
        return fa.backward(q, k, v, o, lse, dout, causal=True, scale=w.scale)[:3]

    g, grads = _capture(step)
    for i, (qi, ki, vi) in enumerate(draws):
        q.copy_(qi); k.copy_(ki); v.copy_(vi); dout.copy_(dout0 * (i + 1))
        g.replay()
        torch.cuda.synchronize()
        o_e, l_e = fa.forward(qi, ki, vi, causal=True, scale=w.scale)
        ref = fa.backward(qi, ki, vi, o_e, l_e, dout0 * (i + 1), causal=True, scale=w.scale)[:3]
        torch.cuda.synchronize()
        for a, b in zip(grads, ref):
            assert torch.equal(a, b), f"replay {i}"


# (1, 3000) and (4, 3000): split and merge kernels; (1, 600) and (2, 400):
# few chunks, split and merge in one kernel
@pytest.mark.parametrize("nq,nk", [(1, 3000), (4, 3000), (1, 600), (2, 400)])
def test_decode_graph_replays(nq, nk):
    dw = inputs.DecodeWorkload(f"graph_dec{nq}_{nk}", 2, 4, nq, nk, 128, "normal", True,
                               seed=33000 + nq)
    q0, k0, v0 = (t.cuda() for t in inputs.make_decode_qkv(dw))
    q, k, v = q0.clone(), k0.clone(), v0.clone()
    g, (o, lse) = _capture(lambda: fa.decode(q, k, v, causal=True, scale=dw.scale))
    for i in range(3):
        qi, ki, vi = q0 * (1 + i), k0.roll(i, dims=2), v0 * (1 - 0.25 * i)
        q.copy_(qi); k.copy_(ki); v.copy_(vi)
        g.replay()
        torch.cuda.synchronize()
        o_e, l_e = fa.decode(qi, ki, vi, causal=True, scale=dw.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, l_e), f"replay {i}"
