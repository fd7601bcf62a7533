"""Forward pass at the head dims that are odd multiples of 16 (16, 48, 80,
112), against the fp64 oracle with the gates of test_gpu_parity.

These run the 128-row kernel in the layout of the next multiple of 32: S
takes d/16 k-steps, the LDS tiles and the output blocks are 32 columns wider
than d at most, the tile copies fill the columns at and past d with zeros,
and the output rows store only the first d columns.  The cases cover both
masks, ragged and one-row sequences, fp16, fp32 (the vector-ALU kernel),
[B, N, H, d] views, reads past the last row, and writes: nothing outside O
changes.
"""
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
