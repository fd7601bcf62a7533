"""Rows past N are never read: every entry point, run on tensors that are
followed in memory by NaN, gives finite results identical bit for bit to a
run on plain allocations.

The sequence lengths are ragged (not multiples of the 64-row tiles), so the
last tile of the last (batch, head) reaches past the end of the tensor,
into the NaN.  The MFMA kernels copy tiles with buffer loads whose
descriptors end at the last valid row, and the hardware turns reads past it
into zeros; the fp32 kernel and the vector-ALU decode kernels test each row
index before loading.  A load whose range check missed those rows would
pull NaN into the result (a masked probability of 0 times NaN is NaN).
"""
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

pytestmark = pytest.mark.gpu

PAD = 1 << 16  # elements of NaN after each tensor


def _nan_backed(t):
    """A copy of contiguous device tensor t at the start of a larger
    allocation whose tail is NaN."""
    buf = torch.full((t.numel() + PAD,), float("nan"), dtype=t.dtype, device="cuda")
    view = buf[: t.numel()].view(t.shape)
    view.copy_(t)
    return view, buf


def _equal(a, b):
    return torch.equal(a, b) and bool(torch.isfinite(a.float()).all())


@pytest.mark.parametrize("d,causal", [(64, True), (64, False), (128, True), (128, False),
                                      (32, True), (96, False)])
def test_forward(d, causal):
    w = inputs.Workload("guard", 1, 2, 1000, d, "bf16", "normal", causal, seed=31 + d)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o1, l1 = fa.forward(q, k, v, causal=causal, scale=w.scale)
    (qn, _bq), (kn, _bk), (vn, _bv) = (_nan_backed(t) for t in (q, k, v))
    o2, l2 = fa.forward(qn, kn, vn, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    print(f"forward d={d} causal={causal}", flush=True)
    assert _equal(o1, o2) and _equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_fp16(d):
    w = inputs.Workload("guard16", 1, 2, 777, d, "f16", "normal", True, seed=41 + d)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o1, l1 = fa.forward(q, k, v, causal=True, scale=w.scale)
    (qn, _bq), (kn, _bk), (vn, _bv) = (_nan_backed(t) for t in (q, k, v))
    o2, l2 = fa.forward(qn, kn, vn, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert _equal(o1, o2) and _equal(l1, l2)


# fp32: grids below one workgroup per compute unit take the 4-row, 64-way
# split shape, larger ones the 16-row (8 above d = 64) 16-way one
@pytest.mark.parametrize("B,H,N,d,causal", [(1, 2, 1000, 64, True), (2, 8, 1000, 64, False),
                                            (1, 2, 333, 128, True), (4, 8, 300, 128, False)])
def test_forward_fp32(B, H, N, d, causal):
    w = inputs.Workload("guard32", B, H, N, d, "f32", "normal", causal, seed=45 + d + N)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o1, l1 = fa.forward(q, k, v, causal=causal, scale=w.scale)
    (qn, _bq), (kn, _bk), (vn, _bv) = (_nan_backed(t) for t in (q, k, v))
    o2, l2 = fa.forward(qn, kn, vn, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    print(f"forward fp32 B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    assert _equal(o1, o2) and _equal(l1, l2)


@pytest.mark.parametrize("d,causal", [(64, True), (128, True), (128, False)])
def test_backward(d, causal):
    w = inputs.Workload("guardb", 1, 2, 1000, d, "bf16", "normal", causal, seed=51 + d)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    g = torch.Generator().manual_seed(52 + d)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).cuda()
    o, lse = fa.forward(q, k, v, causal=causal, scale=w.scale)
    r1 = fa.backward(q, k, v, o, lse, dout, causal=causal, scale=w.scale)
    views = [_nan_backed(t) for t in (q, k, v, o, lse, dout)]
    qn, kn, vn, on, ln, dn = (x[0] for x in views)
    r2 = fa.backward(qn, kn, vn, on, ln, dn, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    print(f"backward d={d} causal={causal}", flush=True)
    for a, b in zip(r1, r2):
        assert _equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
def test_kv_outer(d):
    w = inputs.Workload("guardk", 1, 2, 1000, d, "bf16", "normal", True, seed=61 + d)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o1, l1 = fa.forward_kv_outer(q, k, v, causal=True, scale=w.scale)
    (qn, _bq), (kn, _bk), (vn, _bv) = (_nan_backed(t) for t in (q, k, v))
    o2, l2 = fa.forward_kv_outer(qn, kn, vn, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert _equal(o1, o2) and _equal(l1, l2)


# (1, 1000) and (2, 500): split and merge in one kernel; (1, 3000): the
# vector-ALU split kernel and the merge; 5 and 16 queries: the MFMA kernel
@pytest.mark.parametrize("nq,nk", [(1, 1000), (2, 500), (1, 3000), (5, 1000), (16, 1000)])
def test_decode(nq, nk):
    g = torch.Generator().manual_seed(70 + nq)
    q = torch.randn(1, 2, nq, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, 2, nk, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, nk, 128, generator=g).to(torch.bfloat16).cuda()
    o1, l1 = fa.decode(q, k, v, causal=True)
    (qn, _bq), (kn, _bk), (vn, _bv) = (_nan_backed(t) for t in (q, k, v))
    o2, l2 = fa.decode(qn, kn, vn, causal=True)
    torch.cuda.synchronize()
    assert _equal(o1, o2) and _equal(l1, l2)
