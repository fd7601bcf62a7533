"""fa_decode_noalloc (the allocation-free decode: partials in the library's
fixed device scratch instead of a caller workspace) against fa_decode, the
entry point it is a variant of: on calls in a row, each with a smaller
input than the one before (so the scratch still holds older partials), the
outputs must equal fa_decode's with the same num_splits bit for bit (same
kernels, same split), and both must meet the fp64 oracle's bf16 gates."""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, Nq, Nk, d, causal, splits, seed), each call smaller than the one
    # before: MFMA split kernel and merge, vector-ALU split kernel and merge
    # (partials in the scratch again), then split and merge in one kernel
    # (no partials at all)
    (2, 8, 4, 6000, 128, True, 0, 61),
    (1, 2, 1, 3000, 128, True, 0, 63),
    (1, 4, 1, 1000, 64, False, 0, 62),
]


def _run(fn_name, w, q, k, v, splits):
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device="cuda")
    if fn_name == "noalloc":
        rc = fa.fa_decode_noalloc(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, w.causal,
                                  splits, torch.cuda.current_stream())
    else:
        need = fa.fa_decode_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, splits)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        rc = fa.fa_decode(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, w.causal, splits,
                          ws, need, torch.cuda.current_stream())
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_matches_fa_decode_on_calls_in_a_row(oracle_lib):
    for B, H, Nq, Nk, d, causal, splits, seed in CASES:
        w = inputs.DecodeWorkload(f"noalloc_{B}x{H}x{Nq}x{Nk}x{d}", B, H, Nq, Nk, d, "normal",
                                  causal, seed)
        print(f"case {w.name} causal={causal}", flush=True)
        need = fa.fa_decode_workspace_size(B, H, Nq, Nk, d, splits)
        assert 0 < need <= fa.FA_DECODE_SCRATCH_BYTES
        q, k, v = inputs.make_decode_qkv(w)
        qd, kd, vd = (t.cuda() for t in (q, k, v))
        o1, l1 = _run("noalloc", w, qd, kd, vd, splits)
        o2, l2 = _run("ws", w, qd, kd, vd, splits)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "noalloc differs from fa_decode"
        o_ref, lse_ref = oracle_lib.attention_qk(q, k, v, w.scale, causal)
        o = o1.float().cpu().double().numpy()
        max_abs = float(np.abs(o - o_ref).max())
        rel = float(np.linalg.norm((o - o_ref).ravel()) / np.linalg.norm(o_ref.ravel()))
        lse_err = float(np.abs(l1.cpu().double().numpy() - lse_ref).max())
        print(f"  max_abs={max_abs:.3e} rel_l2={rel:.3e} lse={lse_err:.3e}", flush=True)
        assert max_abs <= 2e-2 and rel <= 5e-3 and lse_err <= 1e-3


def test_noalloc_rejects_oversized_call():
    """Partials of B64 H64 Nq16 d128 (one chunk per head: 33.5 MB) exceed the
    17 MiB scratch: FA_ERR_SCRATCH, nothing enqueued (the tensors are real
    and in bounds for the shapes passed)."""
    q = torch.zeros(64, 64, 16, 128, dtype=torch.bfloat16, device="cuda")
    k, v, o = torch.zeros_like(q), torch.zeros_like(q), torch.empty_like(q)
    lse = torch.empty(64, 64, 16, dtype=torch.float32, device="cuda")
    assert fa.fa_decode_workspace_size(64, 64, 16, 16, 128, 0) > fa.FA_DECODE_SCRATCH_BYTES
    rc = fa.fa_decode_noalloc(q, k, v, o, lse, 64, 64, 16, 16, 128, 0.088, 1, 0, None)
    assert rc == fa.FA_ERR_SCRATCH
