"""The largest shapes a test can afford, against the fp64 oracle.

* Tensors past 2^31 elements: B = 1280, H = 64, N = 256, d = 128 puts
  1.25 * 2^31 elements (5 GiB of bf16) in each of Q, K, V, O.  Heads from
  batch entry 1024 on start past element 2^31 (and past byte 2^32), so an
  offset held in 32 bits anywhere in the forward, backward or decode path
  would read or write the wrong head.  Inputs are drawn on the device
  (make_qkv_device); the oracle gets a few whole heads, including the last
  one, copied back.
* Long rows: one head of N = 2^20 keys at d = 64 (causal, the pipelined
  4-wave kernel) and N = 2^19 at d = 128 (causal, the 8-wave kernel); the
  oracle computes sampled rows one by one, the last row over all N keys.
Gates are those of the parity and backward tests.
"""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

from .test_gpu_parity import check

pytestmark = pytest.mark.gpu

BIG = inputs.Workload("big_b1280h64n256d128", 1280, 64, 256, 128, "bf16", "normal", False, seed=901)
# (b, h) heads handed to the oracle: first, past byte 2^31, past element 2^31, last
HEADS = [(0, 0), (700, 5), (1100, 33), (1279, 63)]


@pytest.fixture(scope="module")
def big_inputs():
    print(f"generating {BIG.name} on the device", flush=True)
    q, k, v = inputs.make_qkv_device(BIG, "cuda")
    assert q.numel() == 5 << 29
    yield q, k, v
    del q, k, v
    torch.cuda.empty_cache()


def _heads(t):
    """The HEADS of a [B, H, N, d] (or [B, H, N]) device tensor as one
    [1, len(HEADS), ...] CPU tensor."""
    return torch.stack([t[b, h].cpu() for b, h in HEADS]).unsqueeze(0)


def test_forward_beyond_4gib(big_inputs, oracle_lib):
    q, k, v = big_inputs
    for causal in (False, True):
        o, lse = fa.forward(q, k, v, causal=causal, scale=BIG.scale)
        torch.cuda.synchronize()
        print(f"forward causal={causal} done", flush=True)
        assert all(bool(torch.isfinite(o[b]).all()) for b in range(BIG.B))
        qh, kh, vh = _heads(q), _heads(k), _heads(v)
        o_ref, lse_ref = oracle_lib.attention(qh, kh, vh, BIG.scale, causal)
        got = _heads(o).float().double().numpy()
        got_lse = _heads(lse).double().numpy()
        check(got, got_lse, o_ref, lse_ref, "bf16", f"{BIG.name} causal={causal} heads")
        del o, lse


def test_backward_beyond_4gib(big_inputs, oracle_lib):
    q, k, v = big_inputs
    g = torch.Generator("cuda").manual_seed(BIG.seed + 10000)
    dout = torch.empty_like(q)
    for b in range(BIG.B):
        dout[b].copy_(torch.randn(q.shape[1:], generator=g, device="cuda"))
    o, lse = fa.forward(q, k, v, causal=True, scale=BIG.scale)
    dq, dk, dv, _ = fa.backward(q, k, v, o, lse, dout, causal=True, scale=BIG.scale)
    torch.cuda.synchronize()
    print("backward done", flush=True)
    refs = oracle_lib.attention_backward(_heads(q), _heads(k), _heads(v), _heads(dout), BIG.scale,
                                         True)
    for name, gt, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        got = _heads(gt).float().double().numpy()
        rel = float(np.linalg.norm(got - r) / np.linalg.norm(r))
        mx = float(np.abs(got - r).max() / np.abs(r).max())
        print(f"  {name}: rel={rel:.2e} max/maxref={mx:.2e}", flush=True)
        assert np.all(np.isfinite(got)) and rel <= 1e-2 and mx <= 2e-2


def test_decode_beyond_4gib(big_inputs, oracle_lib):
    q, k, v = big_inputs
    qd = q[:, :, -3:].contiguous()   # the three newest positions of every sequence
    o, lse = fa.decode(qd, k, v, causal=True, scale=BIG.scale)
    torch.cuda.synchronize()
    print("decode done", flush=True)
    o_ref, lse_ref = oracle_lib.attention_qk(_heads(qd), _heads(k), _heads(v), BIG.scale, True)
    check(_heads(o).float().double().numpy(), _heads(lse).double().numpy(), o_ref, lse_ref, "bf16",
          "decode heads")


@pytest.mark.parametrize("N,d", [(1 << 20, 64), (1 << 19, 128)])
def test_long_rows(N, d, oracle_lib):
    w = inputs.Workload(f"long_n{N}_d{d}", 1, 1, N, d, "bf16", "normal", True, seed=902 + d)
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_qkv(w)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rows = inputs.sample_rows(w, 12)
    o_ref, lse_ref = oracle_lib.attention_rows(q, k, v, w.scale, True, rows)
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    got_lse = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    check(got, got_lse, o_ref, lse_ref, "bf16", w.name + " sampled")
