"""Seeded synthetic inputs for the attention forward and backward passes.

This module is the only code shared by the tests, the benchmark and the
oracle side: it draws numbers and knows the workload shapes, and holds none of
the attention arithmetic.

Recipe (one ``torch.Generator('cpu')`` per workload, seeded with the workload's
seed; Q, then K, then V, each drawn as fp32 [B, H, N, d] and then rounded to
the storage dtype by round-to-nearest-even):

* ``normal``  -- i.i.d. N(0, 1) (``torch.randn``);
* ``normal4`` -- Q and K i.i.d. N(0, 4^2) (``4 * torch.randn``), V N(0, 1);
  large logits whose row maxima move from tile to tile;
* ``uniform`` -- i.i.d. U(-1, 1) (``2 * torch.rand - 1``).

The output gradient dO of the backward pass is drawn from its own generator
(seed + 10000), i.i.d. N(0, 1), rounded to bf16 (``make_dout``).

``scale`` is the fp32 value of 1/sqrt(d).  The pages measure on no public
dataset: every input is synthetic and shaped like the pages' workloads
(N = 2048, d = 64 in the Triton page's tuning table; N around 10^4 with
d = 128 in the unit-12 memory lesson).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32", "bf16" or "f16"
    dist: str           # "normal", "normal4" or "uniform"
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        """fp32(1/sqrt(d)) widened to a Python float."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Nominal matmul FLOPs 4*B*H*N^2*d, halved under the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads; the last one is run both without and with the mask,
# from the same tensors.
WORKLOADS = {
    "w1_f32_n256_d64": Workload("w1_f32_n256_d64", 1, 1, 256, 64, "f32", "normal", False, 1),
    "w2_bf16_b4h16_n2048_d64": Workload("w2_bf16_b4h16_n2048_d64", 4, 16, 2048, 64, "bf16", "normal", False, 2),
    "w3_bf16_b2h32_n8192_d128_causal": Workload("w3_bf16_b2h32_n8192_d128_causal", 2, 32, 8192, 128, "bf16", "normal", True, 3),
    "w4_bf16_b1h16_n16384_d64_causal_big_logits": Workload("w4_bf16_b1h16_n16384_d64_causal_big_logits", 1, 16, 16384, 64, "bf16", "normal4", True, 4),
    "w5a_bf16_b16h12_n1000_d64": Workload("w5a_bf16_b16h12_n1000_d64", 16, 12, 1000, 64, "bf16", "uniform", False, 5),
    "w5b_bf16_b16h12_n1000_d64_causal": Workload("w5b_bf16_b16h12_n1000_d64_causal", 16, 12, 1000, 64, "bf16", "uniform", True, 5),
}

HEADLINE = "w3_bf16_b2h32_n8192_d128_causal"


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def make_qkv(w: Workload, device="cpu"):
    """Returns (q, k, v) as torch tensors of the workload's storage dtype,
    contiguous [B, H, N, d], on ``device``."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)

    def draw(big: bool):
        if w.dist == "uniform":
            x = 2.0 * torch.rand(shape, generator=g, dtype=torch.float32) - 1.0
        else:
            x = torch.randn(shape, generator=g, dtype=torch.float32)
            if big:
                x = 4.0 * x
        return x

    big = w.dist == "normal4"
    q = draw(big)
    k = draw(big)
    v = draw(False)
    dt = torch_dtype(w.dtype)
    return tuple(t.to(dt).contiguous().to(device) for t in (q, k, v))


def make_qkv_device(w: Workload, device):
    """(q, k, v) with make_qkv's recipe (distribution; Q, then K, then V),
    drawn on ``device`` from a torch generator of that device seeded with the
    workload's seed, one batch entry at a time.  For tensors too large to
    draw on the host in reasonable time; the numbers differ from make_qkv's."""
    g = torch.Generator(device).manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    dt = torch_dtype(w.dtype)
    big = w.dist == "normal4"
    out = []
    for which in range(3):
        t = torch.empty(shape, dtype=dt, device=device)
        for b in range(w.B):
            if w.dist == "uniform":
                x = 2.0 * torch.rand(shape[1:], generator=g, device=device, dtype=torch.float32) - 1.0
            else:
                x = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
                if big and which < 2:
                    x = 4.0 * x
            t[b].copy_(x)
        out.append(t)
    return tuple(out)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Nq queries (the newest positions) over Nk keys of each (batch, head)."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dist: str
    causal: bool
    seed: int
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Matmul FLOPs 4*d per visible (query, key) pair."""
        if self.causal:
            pairs = sum(self.Nk - self.Nq + i + 1 for i in range(self.Nq))
        else:
            pairs = self.Nq * self.Nk
        return 4.0 * self.B * self.H * pairs * self.d

    @property
    def bytes(self) -> float:
        """Compulsory HBM bytes: read Q, K, V once, write O (bf16) and LSE."""
        bh = self.B * self.H
        return 2.0 * bh * (2 * self.Nk + 2 * self.Nq) * self.d + 4.0 * bh * self.Nq


# Decode steps over the key/value shapes of the workloads above: the newest
# query (or 16 of them, masked) of each sequence.
DECODE_WORKLOADS = {
    "d3_bf16_b2h32_nq1_nk8192_d128": DecodeWorkload("d3_bf16_b2h32_nq1_nk8192_d128", 2, 32, 1, 8192, 128, "normal", False, 13),
    "d3q16_bf16_b2h32_nq16_nk8192_d128_causal": DecodeWorkload("d3q16_bf16_b2h32_nq16_nk8192_d128_causal", 2, 32, 16, 8192, 128, "normal", True, 23),
    "d4_bf16_b1h16_nq1_nk16384_d64_big_logits": DecodeWorkload("d4_bf16_b1h16_nq1_nk16384_d64_big_logits", 1, 16, 1, 16384, 64, "normal4", False, 14),
    "d5_bf16_b16h12_nq1_nk1000_d64": DecodeWorkload("d5_bf16_b16h12_nq1_nk1000_d64", 16, 12, 1, 1000, 64, "uniform", False, 15),
}

DECODE_HEADLINE = "d3_bf16_b2h32_nq1_nk8192_d128"


def make_decode_qkv(w: DecodeWorkload, device="cpu"):
    """(q [B,H,Nq,d], k, v [B,H,Nk,d]) with the recipe of make_qkv (Q, then K,
    then V from one generator seeded with the workload's seed)."""
    g = torch.Generator("cpu").manual_seed(w.seed)

    def draw(shape, big):
        if w.dist == "uniform":
            return 2.0 * torch.rand(shape, generator=g, dtype=torch.float32) - 1.0
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        return 4.0 * x if big else x

    big = w.dist == "normal4"
    q = draw((w.B, w.H, w.Nq, w.d), big)
    k = draw((w.B, w.H, w.Nk, w.d), big)
    v = draw((w.B, w.H, w.Nk, w.d), False)
    dt = torch_dtype(w.dtype)
    return tuple(t.to(dt).contiguous().to(device) for t in (q, k, v))


def make_dout(w: Workload, device="cpu"):
    """The output gradient dO for the backward pass: i.i.d. N(0, 1) from a
    generator seeded with seed + 10000, as fp32 [B, H, N, d] rounded to the
    workload's storage dtype."""
    g = torch.Generator("cpu").manual_seed(w.seed + 10000)
    x = torch.randn((w.B, w.H, w.N, w.d), generator=g, dtype=torch.float32)
    return x.to(torch_dtype(w.dtype)).contiguous().to(device)


def sample_rows(w: Workload, count: int, seed: int = 1234):
    """A seeded sample of (b, h, i) output rows, always including the first
    and last query of the first and last head, plus uniform draws."""
    rng = np.random.default_rng(seed + w.seed)
    fixed = [(0, 0, 0), (0, 0, w.N - 1), (w.B - 1, w.H - 1, 0), (w.B - 1, w.H - 1, w.N - 1)]
    n = max(0, count - len(fixed))
    drawn = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.H, n),
                      rng.integers(0, w.N, n)], axis=1) if n else np.zeros((0, 3), np.int64)
    rows = np.concatenate([np.array(fixed, dtype=np.int64), drawn.astype(np.int64)])
    return rows
