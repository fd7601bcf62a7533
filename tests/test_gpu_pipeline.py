"""Parity of the head-dim-128 forward kernel at the shapes that exercise its
structure, against the fp64 oracle (same gates as test_gpu_parity).

At d = 128 the forward pass runs 256 query rows per workgroup (8 waves of 32
rows), walks the keys in 32-key half tiles with the P V^T of half tile h-1,
the K Q^T of half tile h+1 and the softmax of half tile h in one step, keeps
three 64-key LDS buffers per operand in rotation, and lets a wave whose rows
have seen all their keys leave the loop early.  The sequence lengths below
sit on and around the boundaries of those pieces: half tiles (32), tiles
(64), the three-buffer cycle (192), workgroups (256), and waves lying wholly
past N in the last workgroup.  Causal head dim 64 with N >= 8192 runs the
same kernel with 4-wave workgroups (test_d64_long_causal).
"""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

from .test_gpu_parity import check, run_gpu

pytestmark = pytest.mark.gpu

LENGTHS = [2, 33, 95, 192, 255, 256, 257, 449, 513, 769]


def _case(B, H, N, dist, causal, dtype, oracle_lib, seed):
    w = inputs.Workload(f"d128_{B}x{H}x{N}_{dtype}_{dist}_{int(causal)}", B, H, N, 128, dtype, dist,
                        causal, seed=seed)
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_qkv(w)
    o, lse = run_gpu(q, k, v, causal, w.scale)
    o_ref, lse_ref = oracle_lib.attention(q, k, v, w.scale, causal)
    check(o, lse, o_ref, lse_ref, dtype, w.name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", LENGTHS)
def test_d128_lengths(N, causal, oracle_lib):
    _case(1, 2, N, "normal", causal, "bf16", oracle_lib, seed=5000 + N)


@pytest.mark.parametrize("N,causal", [(257, True), (513, False), (769, True)])
def test_d128_large_logits(N, causal, oracle_lib):
    """Q, K ~ N(0, 4^2): row maxima move across tiles, so the exponent base
    is moved (and the accumulator rescaled) inside the pipelined steps."""
    _case(1, 2, N, "normal4", causal, "bf16", oracle_lib, seed=6000 + N)


@pytest.mark.parametrize("N,causal", [(255, True), (513, False)])
def test_d128_fp16(N, causal, oracle_lib):
    _case(1, 2, N, "normal", causal, "f16", oracle_lib, seed=7000 + N)


@pytest.mark.parametrize("B,H,N", [(1, 3, 300), (2, 2, 512), (3, 5, 129)])
def test_d128_grid_shapes(B, H, N, oracle_lib):
    """Workgroup counts that are (2 x 2 x 2 = 8) and are not (3, 15) a
    multiple of the XCD count, which changes the workgroup -> tile order."""
    _case(B, H, N, "uniform", True, "bf16", oracle_lib, seed=8000 + B * H * N)


@pytest.mark.parametrize("N,dist,dtype", [(8200, "normal4", "bf16"), (8192, "normal", "f16"),
                                          (9001, "uniform", "bf16")])
def test_d64_long_causal(N, dist, dtype, oracle_lib):
    """Causal head dim 64 with N >= 8192 runs the same pipelined kernel with
    4-wave workgroups (128 rows); whole-tensor parity for one head, ragged
    N included."""
    w = inputs.Workload(f"d64_long_{N}_{dtype}_{dist}", 1, 1, N, 64, dtype, dist, True,
                        seed=9000 + N)
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_qkv(w)
    o, lse = run_gpu(q, k, v, True, w.scale)
    o_ref, lse_ref = oracle_lib.attention(q, k, v, w.scale, True)
    check(o, lse, o_ref, lse_ref, dtype, w.name)


def test_d128_strided_matches_dense():
    """[B, N, H, d]-ordered views give the dense result bit for bit."""
    w = inputs.Workload("d128_strided", 2, 3, 449, 128, "bf16", "normal", True, seed=91)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    qs, ks, vs = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
    assert not qs.is_contiguous()
    o2, l2 = fa.forward(qs, ks, vs, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_d128_deterministic():
    """Repeated calls give bit-identical results."""
    w = inputs.Workload("d128_det", 2, 4, 1500, 128, "bf16", "normal", True, seed=92)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o1, l1 = fa.forward(q, k, v, causal=True, scale=w.scale)
    o2, l2 = fa.forward(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.isfinite(o1.float().cpu().numpy()).all()
