"""The checking build of the library (libfa_safesync.so, compiled with
FA_SAFE_SYNC=1: every copy into an LDS tile buffer completes and is made
visible at a workgroup barrier before any compute, and every buffer's reads
complete at a barrier before it is refilled) must give the regular build's
results bit for bit.  The arithmetic of the two builds is the same; only the
overlap of copies with compute differs, so any difference would expose a
missing wait or barrier in the regular pipelines (a race on an LDS buffer).
Covered: the forward pass at the B2 H32 N8192 d128 causal shape and at ragged
sequence lengths (both head dims' kernels, the 4-wave causal d64 pipeline at
N >= 8192, fp16 and strided views), the backward pass and decode."""
import ctypes

import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import _lib, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    return fa.load_library(), _lib.open_library(_lib.SAFE_SYNC_LIB_PATH)


def _say(msg):
    print(msg, flush=True)


def _fwd(lib, q, k, v, causal, scale, strided=False):
    B, H, N, d = q.shape
    o = torch.empty_like(q) if not strided else \
        torch.empty(B, N, H, d, dtype=q.dtype, device=q.device).permute(0, 2, 1, 3)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    s = torch.cuda.current_stream().cuda_stream
    if q.dtype == torch.bfloat16 and not strided:
        rc = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, H, N, d, scale, int(causal), s)
    else:
        st = (ctypes.c_int64 * 12)(*[x for t in (q, k, v, o) for x in t.stride()[:3]])
        dt = fa.FA_DTYPE_FP16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
        rc = lib.fa_fwd_ex(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                           lse.data_ptr(), B, H, N, d, scale, int(causal), st, s)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return o, lse


FWD = [
    # (B, H, N, d, dtype, dist, causal, strided)
    (2, 32, 8192, 128, "bf16", "normal", True, False),
    (2, 3, 1000, 128, "bf16", "normal", True, False),
    (1, 4, 777, 128, "bf16", "normal4", False, False),
    (1, 3, 8300, 64, "bf16", "normal4", True, False),
    (4, 5, 1000, 64, "bf16", "uniform", True, False),
    (2, 3, 777, 64, "bf16", "normal", False, False),
    (1, 3, 1111, 96, "bf16", "normal", True, False),
    (2, 2, 999, 128, "f16", "normal", True, True),
]


@pytest.mark.parametrize("B,H,N,d,dtype,dist,causal,strided", FWD)
def test_forward_checking_build_identical(B, H, N, d, dtype, dist, causal, strided, libs):
    reg, safe = libs
    w = inputs.Workload(f"sync_{B}x{H}x{N}x{d}", B, H, N, d, dtype, dist, causal, seed=700 + N + d)
    _say(f"case {w.name} {dtype} causal={causal} strided={strided}")
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    if strided:
        q, k, v = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
    o1, l1 = _fwd(reg, q, k, v, causal, w.scale, strided)
    o2, l2 = _fwd(safe, q, k, v, causal, w.scale, strided)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "checking build differs"


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 3, 1000, 128, True), (2, 2, 777, 64, False),
                                             (1, 2, 4100, 128, True)])
def test_backward_checking_build_identical(B, H, N, d, causal, libs):
    reg, safe = libs
    w = inputs.Workload(f"syncb_{B}x{H}x{N}x{d}", B, H, N, d, "bf16", "normal", causal, seed=800 + N)
    _say(f"case {w.name} backward causal={causal}")
    q, k, v = (t.cuda() for t in inputs.make_qkv(w))
    dout = inputs.make_dout(w).cuda()
    o, lse = _fwd(reg, q, k, v, causal, w.scale)
    s = torch.cuda.current_stream().cuda_stream
    outs = []
    for lib in (reg, safe):
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        delta = torch.empty_like(lse)
        rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                        delta.data_ptr(), B, H, N, d, w.scale, int(causal), s)
        assert rc == 0, rc
        torch.cuda.synchronize()
        outs.append((dq, dk, dv, delta))
    for a, b in zip(*outs):
        assert torch.equal(a, b), "checking build differs"


@pytest.mark.parametrize("Nq,Nk,d,causal", [(1, 5000, 128, False), (8, 3000, 64, True),
                                             (16, 4097, 128, True), (2, 500, 64, True)])
def test_decode_checking_build_identical(Nq, Nk, d, causal, libs):
    reg, safe = libs
    w = inputs.DecodeWorkload(f"syncd_{Nq}x{Nk}x{d}", 2, 3, Nq, Nk, d, "normal", causal, 900 + Nk)
    _say(f"case {w.name} decode")
    q, k, v = (t.cuda() for t in inputs.make_decode_qkv(w))
    need = fa.fa_decode_workspace_size(w.B, w.H, Nq, Nk, d, 0)
    s = torch.cuda.current_stream().cuda_stream
    outs = []
    for lib in (reg, safe):
        o = torch.empty_like(q)
        lse = torch.empty(w.B, w.H, Nq, dtype=torch.float32, device="cuda")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        rc = lib.fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           w.B, w.H, Nq, Nk, d, w.scale, int(causal), 0, ws.data_ptr(), need, s)
        assert rc == 0, rc
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
