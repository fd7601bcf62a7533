"""Parity of the key/value-outer forward pass (fa_fwd_kv_outer: Algorithm 1's
loop order, O, l, m round-tripping through device memory) with the fp64
oracle, through the C ABI.  Same gates as fa_fwd for bf16 inputs: max-abs
<= 2e-2, relative L2 <= 5e-3 over the whole tensor, LSE <= 1e-3."""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run(q, k, v, causal, scale):
    dev = torch.device("cuda:0")
    o, lse = fa.forward_kv_outer(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def check(o, lse, o_ref, lse_ref, what):
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{what}: non-finite"
    max_abs = float(np.abs(o - o_ref).max())
    rel = float(np.linalg.norm((o - o_ref).ravel()) / np.linalg.norm(o_ref.ravel()))
    lse_err = float(np.abs(lse - lse_ref).max())
    _say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} lse={lse_err:.3e}")
    assert max_abs <= 2e-2 and rel <= 5e-3 and lse_err <= 1e-3, what


SMALL = [
    (1, 1, 1, 64, "normal", False),
    (1, 1, 1, 128, "normal", True),
    (1, 2, 63, 64, "normal", True),
    (1, 2, 64, 128, "normal", False),
    (2, 1, 65, 64, "uniform", True),
    (1, 3, 127, 128, "normal", True),
    (1, 2, 129, 64, "normal4", True),
    (2, 2, 300, 128, "normal", False),
    (1, 2, 1000, 128, "normal4", True),
    (1, 2, 777, 64, "uniform", False),
]


@pytest.mark.parametrize("B,H,N,d,dist,causal", SMALL)
def test_kvouter_small(B, H, N, d, dist, causal, oracle_lib):
    w = inputs.Workload(f"kvo_{B}x{H}x{N}x{d}_{dist}_{int(causal)}", B, H, N, d, "bf16", dist,
                        causal, seed=4000 + N + d)
    _say(f"case {w.name}")
    q, k, v = inputs.make_qkv(w)
    o, lse = run(q, k, v, causal, w.scale)
    o_ref, lse_ref = oracle_lib.attention(q, k, v, w.scale, causal)
    check(o, lse, o_ref, lse_ref, w.name)


@pytest.mark.parametrize("name", ["w2_bf16_b4h16_n2048_d64", "w5a_bf16_b16h12_n1000_d64",
                                  "w5b_bf16_b16h12_n1000_d64_causal",
                                  "w3_bf16_b2h32_n8192_d128_causal"])
def test_kvouter_workloads(name, oracle_lib):
    w = inputs.WORKLOADS[name]
    _say(f"case {w.name} (key/value-outer)")
    q, k, v = inputs.make_qkv(w)
    o, lse = run(q, k, v, w.causal, w.scale)
    rows = inputs.sample_rows(w, 256)
    o_ref, lse_ref = oracle_lib.attention_rows(q, k, v, w.scale, w.causal, rows)
    check(o[rows[:, 0], rows[:, 1], rows[:, 2]], lse[rows[:, 0], rows[:, 1], rows[:, 2]],
          o_ref, lse_ref, w.name + " sampled")


def test_kvouter_matches_fused_forward():
    """Both loop orders give the same O within rounding (unit-12 loop-order
    lesson)."""
    w = inputs.Workload("orders", 2, 3, 700, 128, "bf16", "normal", True, seed=12)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o1, l1 = fa.forward(q, k, v, causal=True, scale=w.scale)
    o2, l2 = fa.forward_kv_outer(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.allclose(o1.float(), o2.float(), atol=2e-2, rtol=0)
    assert torch.allclose(l1, l2, atol=1e-3, rtol=0)


def test_kvouter_workspace_errors():
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    k, v, o = torch.zeros_like(q), torch.zeros_like(q), torch.empty_like(q)
    lse = torch.empty(1, 1, 64, device="cuda")
    need = fa.fa_fwd_kv_outer_workspace_size(1, 1, 64, 64)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert fa.fa_fwd_kv_outer(q, k, v, o, lse, 1, 1, 64, 64, 0.125, 0, ws, need - 4,
                              None) == fa.FA_ERR_WORKSPACE
    assert fa.fa_fwd_kv_outer(q, k, v, o, lse, 1, 1, 64, 64, 0.125, 0, k, need,
                              None) == fa.FA_ERR_ALIAS
