"""Seeded random configurations of every entry point against the fp64 oracle
(shapes, head dims, masks, value distributions and layouts drawn from one
generator), to cross the options that the fixed cases do not combine.
Gates as in the fixed tests of each entry point."""
import numpy as np
import pytest
import torch

import exact_attention_32_amd as fa
from exact_attention_32_amd import inputs

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(20260)
DISTS = ["normal", "normal4", "uniform"]


def _cfgs(n, dims, dtypes, rng=RNG, seed0=7000):
    out = []
    for i in range(n):
        out.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                        N=int(rng.integers(1, 700)), d=int(rng.choice(dims)),
                        dtype=str(rng.choice(dtypes)), dist=str(rng.choice(DISTS)),
                        causal=bool(rng.integers(0, 2)), layout=str(rng.choice(["dense", "bnhd"])),
                        seed=seed0 + i))
    return out


FWD = _cfgs(24, [32, 64, 96, 128], ["bf16", "f16", "bf16"])
BWD = _cfgs(10, [64, 128], ["bf16"])
DEC = [dict(B=int(RNG.integers(1, 3)), H=int(RNG.integers(1, 4)), Nq=int(RNG.integers(1, 17)),
            Nk=int(RNG.integers(16, 3000)), d=int(RNG.choice([64, 128])),
            causal=bool(RNG.integers(0, 2)), dist=str(RNG.choice(DISTS)),
            splits=int(RNG.choice([0, 1, 3, 17])), seed=8000 + i) for i in range(10)]
# Head dims that are odd multiples of 16, from a generator of their own (the
# draws above stay as they were).
FWD_ODD = _cfgs(8, [16, 48, 80, 112], ["bf16", "f16"], rng=np.random.default_rng(20261),
                seed0=7500)
BWD_ODD = _cfgs(6, [16, 32, 48, 80, 96, 112], ["bf16"], rng=np.random.default_rng(20262),
                seed0=7600)


def _err(o, ref):
    o = o.float().cpu().double().numpy() if hasattr(o, "cpu") else o
    return float(np.abs(o - ref).max()), float(np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-300))


@pytest.mark.parametrize("c", FWD + FWD_ODD, ids=lambda c: f"N{c['N']}d{c['d']}{c['dtype']}{c['layout']}c{int(c['causal'])}")
def test_random_forward(c, oracle_lib):
    w = inputs.Workload("rf", c["B"], c["H"], c["N"], c["d"], c["dtype"], c["dist"], c["causal"],
                        seed=c["seed"])
    q, k, v = inputs.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    if c["layout"] == "bnhd":
        qd, kd, vd = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (qd, kd, vd))
    o, lse = fa.forward(qd, kd, vd, causal=c["causal"], scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle_lib.attention(q, k, v, w.scale, c["causal"])
    ma, rel = _err(o, ro)
    le = float(np.abs(lse.cpu().double().numpy() - rl).max())
    ga, gr = (2e-2, 5e-3) if c["dtype"] == "bf16" else (2.5e-3, 6.25e-4)
    print(f"  {c}: max_abs={ma:.2e} rel={rel:.2e} lse={le:.2e}", flush=True)
    assert ma <= ga and rel <= gr and le <= 1e-3


@pytest.mark.parametrize("c", BWD + BWD_ODD, ids=lambda c: f"N{c['N']}d{c['d']}c{int(c['causal'])}")
def test_random_backward(c, oracle_lib):
    w = inputs.Workload("rb", c["B"], c["H"], c["N"], c["d"], "bf16", c["dist"], c["causal"],
                        seed=c["seed"])
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_dout(w)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=c["causal"], scale=w.scale)
    dq, dk, dv, _ = fa.backward(q.cuda(), k.cuda(), v.cuda(), o, lse, dout.cuda(),
                                causal=c["causal"], scale=w.scale)
    torch.cuda.synchronize()
    refs = oracle_lib.attention_backward(q, k, v, dout, w.scale, c["causal"])
    big = c["dist"] == "normal4"
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        ma, rel = _err(g, r)
        scale = float(np.abs(r).max())
        print(f"  {c} {name}: rel={rel:.2e} max/maxref={ma / max(scale, 1e-300):.2e}", flush=True)
        assert rel <= (2e-2 if big else 1e-2)
        assert ma <= (4e-2 if big else 2e-2) * scale


@pytest.mark.parametrize("c", DEC, ids=lambda c: f"Nq{c['Nq']}Nk{c['Nk']}d{c['d']}c{int(c['causal'])}s{c['splits']}")
def test_random_decode(c, oracle_lib):
    w = inputs.DecodeWorkload("rd", c["B"], c["H"], c["Nq"], max(c["Nk"], c["Nq"]), c["d"],
                              c["dist"], c["causal"], seed=c["seed"])
    q, k, v = inputs.make_decode_qkv(w)
    o, lse = fa.decode(q.cuda(), k.cuda(), v.cuda(), causal=c["causal"], scale=w.scale,
                       num_splits=c["splits"])
    torch.cuda.synchronize()
    ro, rl = oracle_lib.attention_qk(q, k, v, w.scale, c["causal"])
    ma, rel = _err(o, ro)
    le = float(np.abs(lse.cpu().double().numpy() - rl).max())
    print(f"  {c}: max_abs={ma:.2e} rel={rel:.2e} lse={le:.2e}", flush=True)
    assert ma <= 2e-2 and rel <= 5e-3 and le <= 1e-3
