"""Parity of the HIP decode path (fa_decode, through the C ABI) with the fp64
oracle's attention of Nq queries over Nk keys (the queries being the last Nq
positions; bottom-right mask).

Gates are the forward pass's for bf16 inputs: max |O_gpu - O_ref| <= 2e-2,
relative L2 <= 5e-3 over the whole tensor, |LSE_gpu - LSE_ref| <= 1e-3.
"""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_decode(q, k, v, causal, scale, splits=0):
    dev = torch.device("cuda:0")
    o, lse = fa.decode(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                       num_splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def check(o, lse, o_ref, lse_ref, what):
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{what}: non-finite"
    max_abs = float(np.abs(o - o_ref).max())
    rel = float(np.linalg.norm((o - o_ref).ravel()) / np.linalg.norm(o_ref.ravel()))
    lse_err = float(np.abs(lse - lse_ref).max())
    _say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} lse={lse_err:.3e}")
    assert max_abs <= 2e-2 and rel <= 5e-3 and lse_err <= 1e-3, what


CASES = [
    # (B, H, Nq, Nk, d, causal, dist, splits)
    (1, 1, 1, 1, 64, False, "normal", 0),
    (1, 1, 1, 1, 128, True, "normal", 0),
    (1, 2, 1, 63, 64, False, "normal", 0),
    (2, 1, 1, 64, 128, True, "normal", 1),
    (1, 3, 1, 65, 64, False, "uniform", 2),
    (2, 2, 2, 100, 128, True, "normal", 0),
    (1, 2, 3, 257, 64, True, "normal4", 3),
    (1, 2, 5, 1000, 128, False, "normal", 0),
    (1, 1, 8, 8, 64, True, "normal", 0),
    (2, 3, 8, 4097, 128, True, "normal", 0),
    (1, 2, 13, 777, 64, True, "uniform", 5),
    (1, 1, 16, 16, 128, True, "normal", 0),
    (1, 2, 16, 2000, 64, False, "normal4", 0),
    (1, 2, 16, 3000, 128, True, "normal", 1000),
    # more than four queries run on the MFMA split kernel: chunks of one to
    # several 32-key tiles in rounds of three, and causal tail chunks that
    # the first queries cannot see
    (1, 2, 6, 130, 128, True, "normal", 3),
    (1, 1, 16, 33, 64, True, "normal4", 0),
    (2, 2, 12, 511, 128, False, "uniform", 2),
    (1, 3, 7, 4096, 64, True, "normal", 0),
    (1, 2, 9, 200, 64, True, "normal", 4),
    # one or two queries and at most eight chunks run split and merge in one
    # workgroup per head (one wave per chunk); more chunks take the split and
    # merge kernels
    (2, 3, 2, 449, 128, True, "normal4", 8),   # last chunk: one key, hidden from query 0
    (1, 2, 2, 300, 80, True, "uniform", 0),
    (3, 5, 1, 511, 48, False, "normal", 0),
    (1, 2, 2, 1500, 128, True, "normal", 0),   # 24 chunks: split and merge kernels
    (1, 1, 1, 700, 64, False, "normal4", 9),   # 9 requested: 11 keys over 64 each -> 9 chunks
    # more chunks than the merge kernel stages at once (1024): its weights
    # go through LDS in several passes
    (1, 1, 1, 131072, 64, False, "normal", 2048),
    (1, 2, 3, 120000, 128, True, "normal4", 1300),   # MFMA kernel: 1250 chunks of 96 keys
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,dist,splits", CASES)
def test_decode_shapes(B, H, Nq, Nk, d, causal, dist, splits, oracle_lib):
    w = inputs.DecodeWorkload(f"dec_{B}x{H}_{Nq}x{Nk}_d{d}_{int(causal)}_{dist}_s{splits}",
                              B, H, Nq, Nk, d, dist, causal, seed=3000 + Nq + Nk + d)
    _say(f"case {w.name}")
    q, k, v = inputs.make_decode_qkv(w)
    o, lse = run_decode(q, k, v, causal, w.scale, splits)
    o_ref, lse_ref = oracle_lib.attention_qk(q, k, v, w.scale, causal)
    check(o, lse, o_ref, lse_ref, w.name)


@pytest.mark.parametrize("name", sorted(inputs.DECODE_WORKLOADS))
def test_decode_workloads(name, oracle_lib):
    w = inputs.DECODE_WORKLOADS[name]
    _say(f"case {w.name}")
    q, k, v = inputs.make_decode_qkv(w)
    o, lse = run_decode(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle_lib.attention_qk(q, k, v, w.scale, w.causal)
    check(o, lse, o_ref, lse_ref, w.name)


@pytest.mark.parametrize("nq", [1, 2, 4])
def test_decode_split_counts_agree(nq, oracle_lib):
    """Any split of the key axis gives the same result within rounding (with
    one or two queries, up to eight chunks merge inside one workgroup and
    more in the merge kernel)."""
    w = inputs.DecodeWorkload("splits", 1, 4, nq, 5000, 128, "normal", True, seed=44 + nq)
    q, k, v = inputs.make_decode_qkv(w)
    o_ref, lse_ref = oracle_lib.attention_qk(q, k, v, w.scale, True)
    for splits in (1, 2, 7, 8, 9, 40, 79, 0):
        o, lse = run_decode(q, k, v, True, w.scale, splits)
        check(o, lse, o_ref, lse_ref, f"nq={nq} splits={splits}")


def test_decode_equals_forward_rows():
    """Nq = Nk decode with the mask equals fa_fwd (top-left mask) within
    rounding; a single decode query equals the last row of a causal fa_fwd."""
    w = inputs.Workload("eq", 1, 2, 16, 128, "bf16", "normal", True, seed=8)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    of, lf = fa.forward(q, k, v, causal=True, scale=w.scale)
    od, ld = fa.decode(q, k, v, causal=True, scale=w.scale)
    assert torch.allclose(od.float(), of.float(), atol=2e-2, rtol=0)
    assert torch.allclose(ld, lf, atol=1e-3, rtol=0)
    o1, l1 = fa.decode(q[:, :, -1:].contiguous(), k, v, causal=True, scale=w.scale)
    assert torch.allclose(o1.float(), of[:, :, -1:].float(), atol=2e-2, rtol=0)
    assert torch.allclose(l1, lf[:, :, -1:], atol=1e-3, rtol=0)


def test_decode_deterministic():
    w = inputs.DECODE_WORKLOADS["d5_bf16_b16h12_nq1_nk1000_d64"]
    q, k, v = (t.cuda() for t in inputs.make_decode_qkv(w))
    a = fa.decode(q, k, v, scale=w.scale)
    b = fa.decode(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_error_codes_on_device():
    q = torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 100, 64, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 1, device="cuda")
    need = fa.fa_decode_workspace_size(1, 1, 1, 100, 64, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = fa.fa_decode(q, k, v, o, lse, 1, 1, 1, 100, 64, 0.125, 0, 0, ws, need - 1, None)
    assert rc == fa.FA_ERR_WORKSPACE
    rc = fa.fa_decode(q, k, v, o, lse, 1, 1, 1, 100, 64, 0.125, 0, 0, k, need, None)
    assert rc == fa.FA_ERR_ALIAS
    q17 = torch.zeros(1, 1, 17, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.decode(q17, k, v)
    assert e.value.code == fa.FA_ERR_SHAPE
