"""The backward pass on fp16 tensors and on strided views (fa_bwd_ex,
through the C ABI), against the fp64 oracle's gradients and against the dense
bf16 path.

Gates: fp16 inputs take test_gpu_backward's gates divided by 8, the ratio of
the two formats' unit roundoffs (every error term there is a multiple of the
rounding of P, dS, O inside delta or the stored result): relative L2
<= 1.25e-3 and max error <= 2.5e-3 of the largest magnitude per gradient.
Strided views of either type must reproduce the dense result of the same
type bit for bit (the same kernels with other offsets).
"""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

pytestmark = pytest.mark.gpu

TOL_REL_F16 = 1e-2 / 8
TOL_MAX_F16 = 2e-2 / 8


def _grads(q, k, v, dout, causal, scale):
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv, delta = fa.backward(q, k, v, o, lse, dout, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv, delta, o, lse


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 77, 64, True), (1, 2, 300, 128, False), (2, 1, 1000, 128, True),
    (1, 3, 333, 64, False), (1, 2, 300, 48, True), (1, 2, 257, 96, True)])
def test_fp16_parity(B, H, N, d, causal, oracle_lib):
    w = inputs.Workload(f"bwd16_{B}x{H}x{N}_d{d}_{int(causal)}", B, H, N, d, "f16", "normal",
                        causal, seed=23000 + N + d)
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_dout(w)
    dq, dk, dv, _, _, _ = _grads(q.cuda(), k.cuda(), v.cuda(), dout.cuda(), causal, w.scale)
    refs = oracle_lib.attention_backward(q, k, v, dout, w.scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        g = g.float().cpu().double().numpy()
        assert np.all(np.isfinite(g)), name
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        mx = float(np.abs(g - r).max() / np.abs(r).max())
        print(f"  {name}: rel_l2={rel:.3e} max_err/max_ref={mx:.3e}", flush=True)
        assert rel <= TOL_REL_F16 and mx <= TOL_MAX_F16, name


def _bnhd(t):
    """The same values as a [B, H, N, d] view of a [B, N, H, d] tensor."""
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d,causal", [(64, True), (128, False), (80, True)])
def test_strided_matches_dense(dtype, d, causal):
    """q, k, v, o, dout and the three gradients all as [B, N, H, d]-ordered
    views: bit-equal to the dense call."""
    w = inputs.Workload(f"bwdst_{dtype}_d{d}", 2, 3, 333, d, dtype, "normal", causal,
                        seed=24000 + d)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    dout = inputs.make_dout(w).cuda()
    dq, dk, dv, delta, o, lse = _grads(q, k, v, dout, causal, w.scale)
    qs, ks, vs, os_, ds = (_bnhd(t) for t in (q, k, v, o, dout))
    outs = tuple(_bnhd(torch.empty_like(q)) for _ in range(3))
    assert not qs.is_contiguous() and not outs[0].is_contiguous()
    dq2, dk2, dv2, delta2 = fa.backward(qs, ks, vs, os_, lse, ds, causal=causal, scale=w.scale,
                                        out=outs)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv, delta), (dq2, dk2, dv2, delta2)):
        assert torch.equal(a, b)


def test_shared_kv_heads():
    """k and v shared by every head (head stride 0): the gradients equal
    those of the dense call on k and v repeated per head."""
    w = inputs.Workload("bwd_shared", 2, 3, 200, 64, "bf16", "normal", True, seed=25)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    dout = inputs.make_dout(w).cuda()
    k1, v1 = k[:, :1].contiguous(), v[:, :1].contiguous()
    ke, ve = k1.expand(-1, 3, -1, -1), v1.expand(-1, 3, -1, -1)
    assert ke.stride(1) == 0
    kd, vd = ke.contiguous(), ve.contiguous()
    dq, dk, dv, _, o, lse = _grads(q, kd, vd, dout, True, w.scale)
    dq2, dk2, dv2, _ = fa.backward(q, ke, ve, o, lse, dout, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), (dq2, dk2, dv2)):
        assert torch.equal(a, b)


def test_fp16_matches_bf16_structure(oracle_lib):
    """The fp16 and bf16 results of the same fp32 draw both pass their gates
    and the fp16 one is the closer to the oracle (its roundings are finer)."""
    errs = {}
    for dt in ("bf16", "f16"):
        w = inputs.Workload(f"bwd_cmp_{dt}", 1, 2, 500, 128, dt, "normal", True, seed=26)
        q, k, v = inputs.make_qkv(w)
        dout = inputs.make_dout(w)
        dq, _, _, _, _, _ = _grads(q.cuda(), k.cuda(), v.cuda(), dout.cuda(), True, w.scale)
        r = oracle_lib.attention_backward(q, k, v, dout, w.scale, True)[0]
        g = dq.float().cpu().double().numpy()
        errs[dt] = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    print(f"  dQ rel-L2: bf16 {errs['bf16']:.3e}, fp16 {errs['f16']:.3e}", flush=True)
    assert errs["f16"] < errs["bf16"]


def test_bwd_ex_error_codes_on_device():
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float16, device="cuda")
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        fa.backward(q, q, q, q, lse, q.to(torch.bfloat16))
    with pytest.raises(fa.FAError) as e:
        fa.backward(q, q.clone(), q.clone(), q.clone(), lse, q.clone(), scale=0.0)
    assert e.value.code == fa.FA_ERR_SCALE
