"""The decode pass on fp16 tensors and on strided views (fa_decode_ex,
through the C ABI), against the fp64 oracle and against the dense bf16 path.

Gates: fp16 inputs take the decode (forward) bf16 gates divided by 8, the
ratio of the two formats' unit roundoffs: max |O - O_ref| <= 2.5e-3,
relative L2 <= 6.25e-4; LSE <= 1e-3.  Strided views of either type
(a key/value cache kept as [B, Nk, H, d], queries and output as
[B, Nq, H, d]) must reproduce the dense result of the same type bit for bit.
"""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

pytestmark = pytest.mark.gpu


def _check16(o, lse, o_ref, lse_ref, what):
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    max_abs = float(np.abs(o - o_ref).max())
    rel = float(np.linalg.norm((o - o_ref).ravel()) / np.linalg.norm(o_ref.ravel()))
    lse_err = float(np.abs(lse - lse_ref).max())
    print(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} lse={lse_err:.3e}", flush=True)
    assert max_abs <= 2.5e-3 and rel <= 6.25e-4 and lse_err <= 1e-3, what


@pytest.mark.parametrize("nq,nk,d,causal,dist", [
    (1, 1000, 128, False, "normal"), (2, 777, 64, True, "normal4"), (5, 4097, 128, True, "normal"),
    (16, 333, 64, False, "uniform"), (3, 500, 80, True, "normal"), (16, 2000, 112, True, "normal4")])
def test_fp16_parity(nq, nk, d, causal, dist, oracle_lib):
    w = inputs.DecodeWorkload(f"dec16_nq{nq}_nk{nk}_d{d}", 2, 2, nq, nk, d, dist, causal,
                              seed=27000 + nq + d, dtype="f16")
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_decode_qkv(w)
    for splits in (0, 3):
        o, lse = fa.decode(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=w.scale,
                           num_splits=splits)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle_lib.attention_qk(q, k, v, w.scale, causal)
        _check16(o, lse, o_ref, lse_ref, f"{w.name} splits={splits}")


def _bnhd(t):
    """The same values as a [B, H, rows, d] view of a [B, rows, H, d] tensor."""
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("nq,d,nk", [(1, 128, 1500), (2, 64, 1500), (5, 128, 1500),
                                     (16, 80, 1500), (1, 96, 300), (2, 128, 500)])
def test_strided_matches_dense(dtype, nq, d, nk):
    w = inputs.DecodeWorkload(f"decst_{dtype}_{nq}_{d}_{nk}", 2, 3, nq, nk, d, "normal", True,
                              seed=28000 + nq + d, dtype=dtype)
    q, k, v = (t.cuda() for t in inputs.make_decode_qkv(w))
    o, lse = fa.decode(q, k, v, causal=True, scale=w.scale)
    qs, ks, vs = _bnhd(q), _bnhd(k), _bnhd(v)
    out = _bnhd(torch.empty_like(q))
    assert not ks.is_contiguous()   # (with one query, q and o are contiguous anyway)
    o2, l2 = fa.decode(qs, ks, vs, causal=True, scale=w.scale, out=out)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_shared_kv_heads():
    """k and v shared by every head (head stride 0) equal the dense call on
    them repeated per head."""
    w = inputs.DecodeWorkload("dec_shared", 2, 3, 4, 900, 128, "normal", True, seed=29)
    q, k, v = (t.cuda() for t in inputs.make_decode_qkv(w))
    ke, ve = k[:, :1].expand(-1, 3, -1, -1), v[:, :1].expand(-1, 3, -1, -1)
    assert ke.stride(1) == 0
    o1, l1 = fa.decode(q, ke.contiguous(), ve.contiguous(), causal=True, scale=w.scale)
    o2, l2 = fa.decode(q, ke, ve, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
