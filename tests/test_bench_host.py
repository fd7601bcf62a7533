"""Host-side parts of bench.py (no GPU): the single-GPU refusal, the source
hash that ties the committed profile summaries to the kernels they were
taken on, and the unit counts its figures are built from."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_attention_32_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_source_hash_ignores_comments_only(tmp_path):
    src = os.path.join(ROOT, bench.KERNEL_SOURCES[0])
    text = open(src, encoding="utf-8").read()
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text(text)
    b.write_text("// a new comment\n" + text.replace("\n", "\n  ", 3) + "\n/* and another */\n")
    c.write_text(text.replace("kSumMax", "kSumMaxX", 1))
    h = bench.kernel_source_hash
    assert h([str(a)]) == h([str(b)])
    assert h([str(a)]) != h([str(c)])


def test_committed_traffic_summaries_match_the_sources():
    """Every forward traffic summary was taken on the kernel sources as they
    are, so the bench line's `traffic` field is filled for every forward
    workload (it is left null when a kernel changed after its counters)."""
    for name in inputs.WORKLOADS:
        got = bench.read_traffic(name)
        assert got is not None and got > 0, name
        w = inputs.WORKLOADS[name]
        el = 4 if w.dtype == "f32" else 2
        compulsory = 4 * w.B * w.H * w.N * w.d * el + 4 * w.B * w.H * w.N
        # a single head (w1) is spread over all 8 XCDs, and each XCD's L2
        # fetches its K and V once
        most = 8.0 if w.B * w.H == 1 else 2.0
        assert compulsory * 0.95 <= got <= compulsory * most, (name, got, compulsory)


def test_unit_counts():
    w3 = inputs.WORKLOADS["w3_bf16_b2h32_n8192_d128_causal"]
    assert w3.flops == 2 * 2 * 32 * 8192 * 8192 * 128  # 4 B H N^2 d, halved by the mask
    d3 = inputs.DECODE_WORKLOADS["d3_bf16_b2h32_nq1_nk8192_d128"]
    assert d3.bytes == 2 * 2 * 32 * (2 * 8192 + 2) * 128 + 4 * 2 * 32
    d3q16 = inputs.DECODE_WORKLOADS["d3q16_bf16_b2h32_nq16_nk8192_d128_causal"]
    pairs = sum(8192 - 16 + i + 1 for i in range(16))
    assert d3q16.flops == 4 * 2 * 32 * pairs * 128


@pytest.mark.parametrize("peak,expected", [(bench.PEAK_HBM_GBS, 8000.0)])
def test_published_peaks(peak, expected):
    assert peak == expected
