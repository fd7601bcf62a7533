"""The C ABI of libfa on the CPU: the library loads, exports every function
include/fa.h declares, and rejects bad arguments with the documented codes
before anything reaches the GPU (every call here fails validation, so no HIP
runtime call is made)."""
import os
import re

import pytest

import exact_attention_32_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared == sorted(fa.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), f"{name} missing from {fa.LIB_PATH}"


def test_checking_build_exports_every_declared_symbol():
    """The checking build (FA_SAFE_SYNC=1) is the same library: same ABI."""
    from exact_attention_32_amd import _lib

    safe = _lib.open_library(_lib.SAFE_SYNC_LIB_PATH)
    for name in _declared_functions():
        assert hasattr(safe, name), f"{name} missing from {_lib.SAFE_SYNC_LIB_PATH}"


def test_status_codes_match_header():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    codes = dict((n, int(v)) for n, v in re.findall(r"\b(FA_\w+)\s*=\s*(\d+)", text))
    for name, value in codes.items():
        assert getattr(fa, name) == value, name


def test_strerror(lib):
    for code in range(12):
        s = fa.fa_strerror(code)
        assert s.startswith(["FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_HEADDIM",
                             "FA_ERR_SCALE", "FA_ERR_ALIGN", "FA_ERR_HIP",
                             "FA_ERR_ALIAS", "FA_ERR_WORKSPACE", "FA_ERR_DTYPE",
                             "FA_ERR_STRIDE", "FA_ERR_SCRATCH"][code])
    assert "unknown" in fa.fa_strerror(99)
    assert "unknown" in fa.fa_strerror(-1)


# Fake, well separated, 16-byte aligned addresses: validation rejects every
# call below before any of them could be dereferenced.
BASE = 1 << 40
GAP = 1 << 36
Q, K, V, O, L = (BASE + i * GAP for i in range(5))
GOOD = dict(B=2, H=3, N=100, d=64, scale=0.125, causal=1)


def _call(fn, q=Q, k=K, v=V, o=O, lse=L, **kw):
    args = dict(GOOD)
    args.update(kw)
    return fn(q, k, v, o, lse, args["B"], args["H"], args["N"], args["d"],
              args["scale"], args["causal"], None)


@pytest.mark.parametrize("fn", [fa.fa_fwd, fa.fa_fwd_f32])
def test_validation_codes(fn, lib):
    assert _call(fn, q=0) == fa.FA_ERR_NULL
    assert _call(fn, lse=0) == fa.FA_ERR_NULL
    assert _call(fn, o=0, B=0) == fa.FA_ERR_NULL          # NULL is checked first
    assert _call(fn, B=0) == fa.FA_ERR_SHAPE
    assert _call(fn, H=-1) == fa.FA_ERR_SHAPE
    assert _call(fn, N=0) == fa.FA_ERR_SHAPE
    assert _call(fn, N=(1 << 30) + 1) == fa.FA_ERR_SHAPE
    assert _call(fn, B=1 << 16, H=1 << 10, N=1 << 10) == fa.FA_ERR_SHAPE  # 2^42 elements
    for d in (0, 8, 24, 72, 127, 144, 256):
        assert _call(fn, d=d) == fa.FA_ERR_HEADDIM
    for d in (16, 32, 48, 80, 96, 112):   # every multiple of 16 up to 128: fails later, on the scale
        assert _call(fn, d=d, scale=0.0) == fa.FA_ERR_SCALE
    for s in (0.0, -0.125, float("inf"), float("nan")):
        assert _call(fn, scale=s) == fa.FA_ERR_SCALE
    assert _call(fn, q=Q + 8) == fa.FA_ERR_ALIGN
    assert _call(fn, lse=L + 4) == fa.FA_ERR_ALIGN
    assert _call(fn, o=Q) == fa.FA_ERR_ALIAS
    assert _call(fn, o=K + 16) == fa.FA_ERR_ALIAS
    assert _call(fn, lse=V + 1024) == fa.FA_ERR_ALIAS
    esize = 2 if fn is fa.fa_fwd else 4
    nbytes = 2 * 3 * 100 * 64 * esize
    assert _call(fn, lse=O + nbytes - 16) == fa.FA_ERR_ALIAS
    # adjacent but not overlapping is fine as far as aliasing goes; make the
    # call fail on the shape instead so that nothing is launched
    assert _call(fn, o=Q + nbytes, B=0) == fa.FA_ERR_SHAPE


def test_launch_size_limit(lib):
    """B*H*ceil(N/128) <= 2^22: no kernel launches 2^31 or more work-items.
    At the limit the shape passes (the call then fails on the scale, before
    any launch); one (batch*head, 128-row block) pair more is FA_ERR_SHAPE."""
    for fn in (fa.fa_fwd, fa.fa_fwd_f32):
        assert _call(fn, B=1 << 12, H=1 << 10, N=1, d=16, scale=0.0) == fa.FA_ERR_SCALE
        assert _call(fn, B=1 << 12, H=(1 << 10) + 1, N=1, d=16) == fa.FA_ERR_SHAPE
        assert _call(fn, B=1 << 11, H=1 << 10, N=256, d=16, scale=0.0) == fa.FA_ERR_SCALE
        assert _call(fn, B=1 << 11, H=1 << 10, N=257, d=16) == fa.FA_ERR_SHAPE
    assert _bwd(B=1 << 12, H=1 << 10, N=128, d=16, scale=0.0) == fa.FA_ERR_SCALE
    assert _bwd(B=1 << 12, H=1 << 10, N=129, d=16) == fa.FA_ERR_SHAPE
    ws = fa.fa_decode_workspace_size
    assert ws(1 << 18, 1, 16, 16, 16, 1) > 0                     # B*H*Nq = 2^22
    assert ws((1 << 18) + 1, 1, 16, 16, 16, 1) == 0              # one merge row too many
    assert ws(1 << 22, 1, 1, 128, 16, 1) > 0                     # B*H*ceil(Nk/128) = 2^22
    assert ws(1 << 22, 1, 1, 129, 16, 1) == 0
    assert fa.fa_fwd_kv_outer_workspace_size(1 << 12, 1 << 10, 129, 16) == 0
    rc = fa.fa_decode(Q, K, V, O, L, (1 << 18) + 1, 1, 16, 16, 16, 0.25, 0, 1, BASE + 7 * GAP,
                      1 << 40, None)
    assert rc == fa.FA_ERR_SHAPE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from exact_attention_32_amd import _lib

    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load_library(str(tmp_path / "missing.so"))


# fa_bwd: q, k, v, o, dout, lse, dq, dk, dv, delta
BQ, BK, BV, BO, BD, BL, BDQ, BDK, BDV, BDL = (BASE + i * GAP for i in range(10))


def _bwd(**kw):
    p = dict(q=BQ, k=BK, v=BV, o=BO, dout=BD, lse=BL, dq=BDQ, dk=BDK, dv=BDV, delta=BDL)
    args = dict(GOOD)
    for key, val in kw.items():
        (p if key in p else args)[key] = val
    return fa.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["dout"], p["lse"], p["dq"], p["dk"],
                     p["dv"], p["delta"], args["B"], args["H"], args["N"], args["d"],
                     args["scale"], args["causal"], None)


def test_bwd_validation_codes(lib):
    for name in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta"):
        assert _bwd(**{name: 0}) == fa.FA_ERR_NULL, name
    assert _bwd(B=0) == fa.FA_ERR_SHAPE
    assert _bwd(N=(1 << 30) + 1) == fa.FA_ERR_SHAPE
    for d in (0, 8, 72, 144):                    # multiples of 16 up to 128 only
        assert _bwd(d=d) == fa.FA_ERR_HEADDIM
    for d in (16, 32, 96, 112):                  # accepted: fails later, on the scale
        assert _bwd(d=d, scale=0.0) == fa.FA_ERR_SCALE
    assert _bwd(scale=float("nan")) == fa.FA_ERR_SCALE
    assert _bwd(scale=0.0) == fa.FA_ERR_SCALE
    assert _bwd(dk=BDK + 8) == fa.FA_ERR_ALIGN
    assert _bwd(delta=BDL + 4) == fa.FA_ERR_ALIGN
    # every output against every input, and the outputs against each other
    for out in ("dq", "dk", "dv", "delta"):
        for src in (BQ, BK, BV, BO, BD, BL):
            assert _bwd(**{out: src}) == fa.FA_ERR_ALIAS, out
    assert _bwd(dk=BDQ) == fa.FA_ERR_ALIAS
    assert _bwd(delta=BDV + 64) == fa.FA_ERR_ALIAS


def test_decode_workspace_size(lib):
    ws = fa.fa_decode_workspace_size
    assert ws(1, 1, 1, 100, 64, 0) > 0
    assert ws(2, 32, 1, 8192, 128, 0) >= 2 * 32 * 1 * 129 * 4   # at least one chunk
    assert ws(1, 1, 1, 100, 64, 1) < ws(1, 1, 1, 100, 64, 2)
    assert ws(1, 1, 1, 4096, 128, 10 ** 6) == ws(1, 1, 1, 4096, 128, 64)   # capped at Nk/64
    for bad in ((0, 1, 1, 100, 64, 0), (1, 1, 0, 100, 64, 0), (1, 1, 17, 100, 64, 0),
                (1, 1, 8, 7, 64, 0), (1, 1, 1, 100, 72, 0), (1, 1, 1, 100, 144, 0)):
        assert ws(*bad) == 0, bad
    assert ws(1, 1, 1, 100, 96, 1) >= 96 * 4 + 4   # every multiple of 16 up to 128
    # automatic split count: about 2048 single-wave workgroups for one or two
    # queries (vector-ALU kernels), 768 for more (MFMA kernel), at least 64
    # keys per chunk
    for B, H, Nq, Nk, d, S in ((2, 32, 1, 8192, 128, 32), (2, 32, 2, 8192, 64, 32),
                               (2, 32, 3, 8192, 128, 12), (2, 32, 16, 8192, 128, 12),
                               (1, 16, 1, 16384, 64, 128), (1, 8, 16, 32768, 128, 96),
                               (16, 12, 1, 1000, 64, 11), (16, 12, 4, 1000, 64, 4),
                               (1, 1, 16, 300, 128, 5), (64, 64, 8, 8192, 128, 1)):
        assert ws(B, H, Nq, Nk, d, 0) == ws(B, H, Nq, Nk, d, S), (B, H, Nq, Nk, d, S)
        assert ws(B, H, Nq, Nk, d, 0) < ws(B, H, Nq, Nk, d, S + 1) or S * 64 >= Nk


def test_decode_validation_codes(lib):
    DQ, DK, DV, DO, DL, DW = (BASE + i * GAP for i in range(6))

    def call(q=DQ, k=DK, v=DV, o=DO, lse=DL, ws=DW, B=2, H=3, Nq=1, Nk=500, d=128,
             scale=0.125, causal=0, splits=0, wsb=1 << 30):
        return fa.fa_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, splits, ws, wsb,
                            None)
    assert call(q=0) == fa.FA_ERR_NULL
    assert call(lse=0) == fa.FA_ERR_NULL
    assert call(Nq=0) == fa.FA_ERR_SHAPE
    assert call(Nq=17) == fa.FA_ERR_SHAPE
    assert call(Nq=8, Nk=7) == fa.FA_ERR_SHAPE
    assert call(d=72) == fa.FA_ERR_HEADDIM
    assert call(d=80, scale=-1.0) == fa.FA_ERR_SCALE   # 80 is accepted
    assert call(scale=-1.0) == fa.FA_ERR_SCALE
    assert call(ws=0) == fa.FA_ERR_WORKSPACE
    assert call(wsb=16) == fa.FA_ERR_WORKSPACE
    assert call(o=DO + 8) == fa.FA_ERR_ALIGN
    assert call(ws=DK) == fa.FA_ERR_ALIAS
    assert call(o=DQ) == fa.FA_ERR_ALIAS
    assert call(lse=DW + 64) == fa.FA_ERR_ALIAS


def test_decode_noalloc_validation_codes(lib):
    """The allocation-free decode rejects bad arguments like fa_decode, and
    calls whose partials exceed its fixed scratch with FA_ERR_SCRATCH, all
    before any HIP call (the scratch size check comes before the device
    address lookup)."""
    DQ, DK, DV, DO, DL = (BASE + i * GAP for i in range(5))

    def call(q=DQ, k=DK, v=DV, o=DO, lse=DL, B=2, H=3, Nq=1, Nk=500, d=128, scale=0.125,
             causal=0, splits=0):
        return fa.fa_decode_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, splits, None)
    assert call(q=0) == fa.FA_ERR_NULL
    assert call(lse=0) == fa.FA_ERR_NULL
    assert call(Nq=0) == fa.FA_ERR_SHAPE
    assert call(Nq=17) == fa.FA_ERR_SHAPE
    assert call(Nq=8, Nk=7) == fa.FA_ERR_SHAPE
    assert call(d=72) == fa.FA_ERR_HEADDIM
    assert call(scale=-1.0) == fa.FA_ERR_SCALE
    # partials of B64 H64 Nq16 d128 with the automatic split count: far past the scratch
    assert fa.fa_decode_workspace_size(64, 64, 16, 8192, 128, 0) > fa.FA_DECODE_SCRATCH_BYTES
    assert call(B=64, H=64, Nq=16, Nk=8192) == fa.FA_ERR_SCRATCH
    assert call(B=64, H=64, Nq=16, Nk=8192, splits=1) == fa.FA_ERR_SCRATCH
    # the largest automatic case it is sized for fits
    assert fa.fa_decode_workspace_size(2, 32, 16, 8192, 128, 0) <= fa.FA_DECODE_SCRATCH_BYTES
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    m = re.search(r"#define FA_DECODE_SCRATCH_BYTES \((\d+)ul << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_DECODE_SCRATCH_BYTES
    assert call(B=2, H=32, Nq=16, Nk=8192, o=DO + 8) == fa.FA_ERR_ALIGN
    assert call(o=DQ) == fa.FA_ERR_ALIAS
    assert call(lse=DO + 64) == fa.FA_ERR_ALIAS


def test_kv_outer_validation_and_size(lib):
    ws = fa.fa_fwd_kv_outer_workspace_size
    assert ws(1, 1, 100, 64) >= 100 * 64 * 4 + 2 * 100 * 4
    assert ws(2, 3, 100, 128) > ws(1, 3, 100, 128)
    assert ws(1, 1, 0, 64) == 0 and ws(1, 1, 10, 72) == 0
    assert ws(1, 1, 10, 80) >= 10 * 80 * 4 + 2 * 10 * 4
    W = BASE + 7 * GAP

    def call(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, ws=W, wsb=1 << 30)
        a.update(kw)
        return fa.fa_fwd_kv_outer(a["q"], a["k"], a["v"], a["o"], a["lse"], 2, 3, 100, 64, 0.125,
                                  1, a["ws"], a["wsb"], None)
    assert call(q=0) == fa.FA_ERR_NULL
    assert call(ws=0) == fa.FA_ERR_WORKSPACE
    assert call(wsb=1024) == fa.FA_ERR_WORKSPACE
    assert call(ws=W + 8) == fa.FA_ERR_ALIGN
    assert call(ws=K) == fa.FA_ERR_ALIAS
    assert call(ws=L - 64) == fa.FA_ERR_ALIAS


def test_fwd_ex_validation_codes(lib):
    B, H, N, d = 2, 3, 100, 64
    dense = [H * N * d, N * d, d] * 4
    bshd = [N * H * d, d, H * d] * 4           # [B, N, H, d] memory order

    def call(dtype=fa.FA_DTYPE_BF16, strides=dense, **kw):
        p = dict(q=Q, k=K, v=V, o=O, lse=L)
        p.update(kw)
        return fa.fa_fwd_ex(dtype, p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, N, d, 0.125,
                            1, strides, None)
    assert call(strides=None) == fa.FA_ERR_NULL
    assert call(q=0) == fa.FA_ERR_NULL
    assert call(dtype=2) == fa.FA_ERR_DTYPE
    assert call(dtype=-1) == fa.FA_ERR_DTYPE
    bad = list(dense); bad[2] = 32                 # q row stride < d
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    bad = list(dense); bad[5] = 1 << 25            # k row stride > 2^24
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    bad = list(dense); bad[0] = -8
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    bad = list(dense); bad[1] = N * d + 4          # not a multiple of 8 elements
    assert call(strides=bad) == fa.FA_ERR_ALIGN
    bad = list(dense); bad[9:12] = [H * N * d, 8 * d, d]   # o heads overlap (8 rows apart)
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    bad = list(dense); bad[9:12] = [0, N * d, d]           # o batches on top of each other
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    shared = list(dense); shared[3:5] = [N * d, 0]         # k shared by all heads: allowed
    shared[6:8] = [N * d, 0]
    assert call(strides=shared, o=Q) == fa.FA_ERR_ALIAS    # (fails on the alias only)
    assert call(strides=bshd, o=K + 64) == fa.FA_ERR_ALIAS
    assert call(strides=bshd, lse=V + 1024) == fa.FA_ERR_ALIAS
    assert call(strides=bshd, q=Q + 8) == fa.FA_ERR_ALIGN


def test_bwd_ex_validation_codes(lib):
    B, H, N, d = 2, 3, 100, 64
    dense = [H * N * d, N * d, d] * 8
    bshd = [N * H * d, d, H * d] * 8           # [B, N, H, d] memory order

    def call(dtype=fa.FA_DTYPE_BF16, strides=dense, **kw):
        p = dict(q=BQ, k=BK, v=BV, o=BO, dout=BD, lse=BL, dq=BDQ, dk=BDK, dv=BDV, delta=BDL)
        p.update(kw)
        return fa.fa_bwd_ex(dtype, p["q"], p["k"], p["v"], p["o"], p["dout"], p["lse"], p["dq"],
                            p["dk"], p["dv"], p["delta"], B, H, N, d, 0.125, 1, strides, None)
    assert call(strides=None) == fa.FA_ERR_NULL
    for name in ("q", "dout", "lse", "dv", "delta"):
        assert call(**{name: 0}) == fa.FA_ERR_NULL, name
    assert call(dtype=2) == fa.FA_ERR_DTYPE
    bad = list(dense); bad[2] = 32                 # q row stride < d
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    bad = list(dense); bad[14] = 1 << 25           # dout row stride > 2^24
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    bad = list(dense); bad[18] = -8                # dk batch stride < 0
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    bad = list(dense); bad[4] = N * d + 4          # k head stride not a multiple of 8
    assert call(strides=bad) == fa.FA_ERR_ALIGN
    assert call(dq=BDQ + 8) == fa.FA_ERR_ALIGN
    bad = list(dense); bad[21:24] = [H * N * d, 8 * d, d]   # dv heads overlap
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    shared = list(dense); shared[3:5] = [N * d, 0]           # k shared by all heads: allowed
    assert call(strides=shared, dq=BQ) == fa.FA_ERR_ALIAS    # (fails on the alias only)
    assert call(strides=bshd, dk=BV + 64) == fa.FA_ERR_ALIAS
    assert call(strides=bshd, delta=BL + 64) == fa.FA_ERR_ALIAS
    assert call(strides=bshd, dv=BDQ + 128) == fa.FA_ERR_ALIAS   # outputs overlap
    assert call(strides=bshd, q=BQ + 8) == fa.FA_ERR_ALIGN


def test_decode_ex_validation_codes(lib):
    B, H, Nq, Nk, d = 2, 3, 4, 500, 64
    dense = [H * Nq * d, Nq * d, d, H * Nk * d, Nk * d, d, H * Nk * d, Nk * d, d,
             H * Nq * d, Nq * d, d]
    DQ, DK, DV, DO, DL, DW = (BASE + i * GAP for i in range(6))

    def call(dtype=fa.FA_DTYPE_BF16, strides=dense, **kw):
        p = dict(q=DQ, k=DK, v=DV, o=DO, lse=DL, ws=DW, wsb=1 << 30)
        p.update(kw)
        return fa.fa_decode_ex(dtype, p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, Nq, Nk, d,
                               0.125, 1, 0, p["ws"], p["wsb"], strides, None)
    assert call(strides=None) == fa.FA_ERR_NULL
    assert call(o=0) == fa.FA_ERR_NULL
    assert call(dtype=5) == fa.FA_ERR_DTYPE
    bad = list(dense); bad[5] = 32                  # k row stride < d
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    bad = list(dense); bad[4] = Nk * d + 4          # k head stride not a multiple of 8
    assert call(strides=bad) == fa.FA_ERR_ALIGN
    bad = list(dense); bad[9:12] = [H * Nq * d, 2 * d, d]   # o heads overlap
    assert call(strides=bad) == fa.FA_ERR_STRIDE
    assert call(wsb=64) == fa.FA_ERR_WORKSPACE
    assert call(ws=DK) == fa.FA_ERR_ALIAS
    assert call(o=DV + 64) == fa.FA_ERR_ALIAS
    shared = list(dense); shared[3:5] = [Nk * d, 0]          # k shared by all heads: allowed
    assert call(strides=shared, o=DQ) == fa.FA_ERR_ALIAS     # (fails on the alias only)
