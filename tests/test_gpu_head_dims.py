"""Every entry point at the head dims other than 64 and 128, against the
fp64 oracle.  Forward: the odd multiples of 16 (16, 48, 80, 112; 32 and 96
have layouts of their own and are in test_gpu_forward_ex), gates of
test_gpu_parity.  Backward, decode and the Algorithm 1 order: 16, 32, 48,
80, 96, 112 (further down).

These run the 128-row kernel in the layout of the next multiple of 32: S
takes d/16 k-steps, the LDS tiles and the output blocks are 32 columns wider
than d at most, the tile copies fill the columns at and past d with zeros,
and the output rows store only the first d columns.  The cases cover both
masks, ragged and one-row sequences, fp16, fp32 (the vector-ALU kernel),
[B, N, H, d] views, reads past the last row, and writes: nothing outside O
changes.
"""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

from .test_gpu_parity import check, run_gpu

pytestmark = pytest.mark.gpu

DIMS = [16, 48, 80, 112]


def _case(B, H, N, d, dtype, dist, causal, oracle_lib, seed):
    w = inputs.Workload(f"d{d}_{B}x{H}x{N}_{dtype}_{dist}_{int(causal)}", B, H, N, d, dtype, dist,
                        causal, seed=seed)
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_qkv(w)
    o, lse = run_gpu(q, k, v, causal, w.scale)
    o_ref, lse_ref = oracle_lib.attention(q, k, v, w.scale, causal)
    check(o, lse, o_ref, lse_ref, dtype, w.name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 77, 300])
@pytest.mark.parametrize("d", DIMS)
def test_bf16(d, N, causal, oracle_lib):
    _case(1, 2, N, d, "bf16", "normal", causal, oracle_lib, seed=11000 + 10 * d + N)


@pytest.mark.parametrize("d", DIMS)
def test_bf16_large_logits(d, oracle_lib):
    _case(2, 1, 257, d, "bf16", "normal4", True, oracle_lib, seed=12000 + d)


@pytest.mark.parametrize("d", DIMS)
def test_fp16(d, oracle_lib):
    _case(1, 2, 200, d, "f16", "normal", True, oracle_lib, seed=13000 + d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", DIMS)
def test_fp32(d, causal, oracle_lib):
    _case(1, 2, 150, d, "f32", "normal", causal, oracle_lib, seed=14000 + d)


@pytest.mark.parametrize("d", DIMS)
def test_strided_matches_dense(d):
    """[B, N, H, d]-ordered views give the dense result bit for bit."""
    w = inputs.Workload(f"d{d}_strided", 2, 3, 333, d, "bf16", "uniform", True, seed=15000 + d)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    qs, ks, vs = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
    assert not qs.is_contiguous()
    o2, l2 = fa.forward(qs, ks, vs, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("d", DIMS)
def test_guard_rows_and_output_bounds(d):
    """Inputs followed in memory by NaN give results identical bit for bit to
    plain allocations (no read past the last row, no read of a column at or
    past d), and O written into the middle of a NaN-filled buffer leaves the
    NaN around it untouched (no store past d or past the last row)."""
    w = inputs.Workload(f"d{d}_guard", 1, 2, 1000, d, "bf16", "normal", False, seed=16000 + d)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    o1, l1 = fa.forward(q, k, v, causal=False, scale=w.scale)
    pad = 1 << 14
    views, bufs = [], []
    for t in (q, k, v):
        buf = torch.full((t.numel() + pad,), float("nan"), dtype=t.dtype, device="cuda")
        buf[: t.numel()].copy_(t.reshape(-1))
        views.append(buf[: t.numel()].view(t.shape))
        bufs.append(buf)
    obuf = torch.full((o1.numel() + 2 * pad,), float("nan"), dtype=o1.dtype, device="cuda")
    out = obuf[pad: pad + o1.numel()].view(o1.shape)
    o2, l2 = fa.forward(*views, causal=False, scale=w.scale, out=out)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert bool(torch.isfinite(o2.float()).all())
    assert bool(torch.isnan(obuf[:pad].float()).all()) and bool(torch.isnan(obuf[pad + o1.numel():].float()).all())
    print(f"guard d={d} ok", flush=True)


def test_head_dim_rejected():
    """d must be a multiple of 16 from 16 to 128: 72 and 144 are refused
    before any launch."""
    for d in (72, 144):
        q = torch.zeros(1, 1, 64, d, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(fa.FAError) as e:
            fa.forward(q, q.clone(), q.clone())
        assert e.value.code == fa.FA_ERR_HEADDIM


# --- backward at the head dims other than 64 and 128 --------------------------
# The backward kernels run DH < 64 in the 64-column layout and 64 < DH < 128
# in the 128-column one (S and dP over DH/16 k-steps; dQ, dK, dV stored for
# the first DH columns only).  Gates and delta check of test_gpu_backward,
# whose derivation assumes rows of many keys: with two keys, dP - delta is
# P1 (dP0 - dP1) and cancels, so the 2^-9 rounding of O inside delta alone
# moves dQ and dK by up to 1e-2 relative at any head dim (measured at N = 2
# for d = 32, 64, 128: 1.7e-3 .. 1.1e-2).  N = 33 is the shortest ragged
# length here; one key has its own test.
BWD_DIMS = [16, 32, 48, 80, 96, 112]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [33, 77, 300])
@pytest.mark.parametrize("d", BWD_DIMS)
def test_backward(d, N, causal, oracle_lib):
    from .test_gpu_backward import check_delta, check_grad, run_bwd

    w = inputs.Workload(f"bwd_d{d}_{N}_{int(causal)}", 1, 2, N, d, "bf16", "normal", causal,
                        seed=17000 + 10 * d + N)
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_dout(w)
    dq, dk, dv, o, delta = run_bwd(q, k, v, dout, causal, w.scale)
    refs = oracle_lib.attention_backward(q, k, v, dout, w.scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        check_grad(g, r, f"{w.name} {name}")
    check_delta(delta, dout, o, w.name)


@pytest.mark.parametrize("d", BWD_DIMS)
def test_backward_single_key(d):
    """N = 1: the one probability is 1, so dV = dO exactly and dQ = dK = 0 up
    to the rounding of dP - delta (two fp32 dot products of the same terms,
    summed in different orders); the relative gates of the other cases have
    no scale here (the exact gradients are 0)."""
    from .test_gpu_backward import run_bwd

    w = inputs.Workload(f"bwd_d{d}_n1", 2, 3, 1, d, "bf16", "normal", False, seed=17500 + d)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_dout(w)
    dq, dk, dv, _, _ = run_bwd(q, k, v, dout, False, w.scale)
    assert np.array_equal(dv, dout.float().double().numpy())
    bound = 1e-5 * float(np.abs(dout.float().numpy()).max() * np.abs(v.float().numpy()).max()) * d
    assert float(np.abs(dq).max()) <= bound and float(np.abs(dk).max()) <= bound


@pytest.mark.parametrize("d", [48, 112])
def test_backward_large_logits(d, oracle_lib):
    from .test_gpu_backward import check_grad, run_bwd

    w = inputs.Workload(f"bwd_d{d}_big", 2, 1, 257, d, "bf16", "normal4", True, seed=18000 + d)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_dout(w)
    dq, dk, dv, _, _ = run_bwd(q, k, v, dout, True, w.scale)
    refs = oracle_lib.attention_backward(q, k, v, dout, w.scale, True)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        check_grad(g, r, f"{w.name} {name}", big_logits=True)


@pytest.mark.parametrize("d", BWD_DIMS)
def test_backward_guard_and_bounds(d):
    """NaN after every input and around each gradient: the gradients are
    bit-equal to those of plain allocations and nothing outside them is
    written (no store past d or past the last row)."""
    w = inputs.Workload(f"bwd_d{d}_guard", 1, 2, 1000, d, "bf16", "normal", True, seed=19000 + d)
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    dout = inputs.make_dout(w).cuda()
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    r1 = fa.backward(q, k, v, o, lse, dout, causal=True, scale=w.scale)
    pad = 1 << 14

    def nan_backed(t):
        buf = torch.full((t.numel() + pad,), float("nan"), dtype=t.dtype, device="cuda")
        buf[: t.numel()].copy_(t.reshape(-1))
        return buf[: t.numel()].view(t.shape), buf

    qn, kn, vn, on, ln, dn = (nan_backed(t)[0] for t in (q, k, v, o, lse, dout))
    outs = []
    for t in r1[:3]:
        buf = torch.full((t.numel() + 2 * pad,), float("nan"), dtype=t.dtype, device="cuda")
        outs.append((buf[pad: pad + t.numel()].view(t.shape), buf))
    delta = torch.empty_like(lse)
    rc = fa.fa_bwd(qn, kn, vn, on, dn, ln, outs[0][0], outs[1][0], outs[2][0], delta, 1, 2, 1000,
                   d, w.scale, True, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert rc == fa.FA_OK
    for a, (b, buf) in zip(r1[:3], outs):
        n = a.numel()
        assert torch.equal(a, b) and bool(torch.isfinite(b.float()).all())
        assert bool(torch.isnan(buf[:pad].float()).all()) and bool(torch.isnan(buf[pad + n:].float()).all())
    print(f"backward guard d={d} ok", flush=True)


# --- decode and the Algorithm 1 order at the head dims other than 64 and 128
# Both run DH in the layout of the next of 64 and 128 (decode: lanes of the
# columns at and past DH hold zeros in the vector-ALU kernel; the MFMA kernel
# and the Algorithm 1 kernel as the backward's tiles).  Gates of
# test_gpu_decode and test_gpu_kvouter (the forward's bf16 gates).
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq", [1, 2, 5, 16])
@pytest.mark.parametrize("d", BWD_DIMS)
def test_decode(d, nq, causal, oracle_lib):
    from .test_gpu_decode import check as dcheck, run_decode

    w = inputs.DecodeWorkload(f"dec_d{d}_nq{nq}_{int(causal)}", 2, 2, nq, 333, d, "normal", causal,
                              seed=20000 + 10 * d + nq)
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_decode_qkv(w)
    for splits in (0, 3):
        o, lse = run_decode(q, k, v, causal, w.scale, splits)
        o_ref, lse_ref = oracle_lib.attention_qk(q, k, v, w.scale, causal)
        dcheck(o, lse, o_ref, lse_ref, f"{w.name} splits={splits}")


@pytest.mark.parametrize("nq", [1, 5])
@pytest.mark.parametrize("d", [48, 112])
def test_decode_guard_and_bounds(d, nq):
    """NaN after K and V and around O: results bit-equal to plain
    allocations, nothing outside O written."""
    g = torch.Generator().manual_seed(21000 + d + nq)
    q = torch.randn(1, 2, nq, d, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, 2, 1000, d, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, 1000, d, generator=g).to(torch.bfloat16).cuda()
    o1, l1 = fa.decode(q, k, v, causal=True)
    pad = 1 << 14

    def nan_backed(t):
        buf = torch.full((t.numel() + pad,), float("nan"), dtype=t.dtype, device="cuda")
        buf[: t.numel()].copy_(t.reshape(-1))
        return buf[: t.numel()].view(t.shape)

    kn, vn = nan_backed(k), nan_backed(v)
    need = fa.fa_decode_workspace_size(1, 2, nq, 1000, d, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    obuf = torch.full((o1.numel() + 2 * pad,), float("nan"), dtype=o1.dtype, device="cuda")
    o2 = obuf[pad: pad + o1.numel()].view(o1.shape)
    l2 = torch.empty_like(l1)
    rc = fa.fa_decode(q, kn, vn, o2, l2, 1, 2, nq, 1000, d, 1.0 / d ** 0.5, 1, 0, ws, need,
                      torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert rc == fa.FA_OK
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and bool(torch.isfinite(o2.float()).all())
    assert bool(torch.isnan(obuf[:pad].float()).all()) and bool(torch.isnan(obuf[pad + o1.numel():].float()).all())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", BWD_DIMS)
def test_kv_outer(d, causal, oracle_lib):
    from .test_gpu_kvouter import check as kcheck, run as krun

    w = inputs.Workload(f"kvo_d{d}_{int(causal)}", 1, 2, 300, d, "bf16", "normal", causal,
                        seed=22000 + d)
    print(f"case {w.name}", flush=True)
    q, k, v = inputs.make_qkv(w)
    o, lse = krun(q, k, v, causal, w.scale)
    o_ref, lse_ref = oracle_lib.attention(q, k, v, w.scale, causal)
    kcheck(o, lse, o_ref, lse_ref, w.name)
