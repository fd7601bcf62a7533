#!/usr/bin/env python3
"""Benchmark of the fused attention forward pass on one MI355X.

One step = one call of the whole forward pass (one kernel launch of fa_fwd)
over one batch of seeded synthetic input that is already resident in HBM.
Default workload: B=2, H=32, N=8192, d=128, bf16, causal (the configuration
the MFMA-peak target is stated for).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--pass fwd|bwd]

--pass decode times fa_decode (one step = one call: the split and merge
kernels, or the single fused kernel for one or two queries over few chunks)
on a decode workload (default: the newest query over B=2, H=32,
Nk=8192, d=128): HBM-bound, so `value` and `roofline` are GB/s of compulsory
traffic (read Q, K, V once, write O and LSE) against 8 TB/s.

--pass kvouter times fa_fwd_kv_outer (the forward pass in Algorithm 1's
key/value-outer order, one launch per 64-key block, O, l, m round-tripping
through device memory) on a forward workload: same FLOPs and metric as the
forward pass; its roofline is HBM, with the algorithm's own traffic per call
(each step reads Q_i and the O_i, l_i, m_i state and writes the state back;
K_j, V_j once per step and head) counted from the block geometry.

--pass bwd times the backward pass instead (one step = one fa_bwd call: the
dq kernel and the dkdv kernel) with the nominal backward FLOPs
10*B*H*N^2*d (five N x N x d products), halved under the causal mask.

FLOPs are the nominal matmul count 4*B*H*N^2*d, halved under the causal
mask.  `roofline` reports the average launch duration, measured with one
pair of HIP events recorded on the launch stream around the K timed steps
(`kernel_ms`), against the bf16 dense MFMA peak; `traffic` comes from the committed rocprofv3 counter summary of the
same command when it still matches the kernel source.  `cpu_baseline` times
the fp64 oracle on a bounded sample of rows of the same workload.

`python bench.py --oracle-timings` times the oracle alone (no GPU) on the
small workloads (fp32 B1 H1 N256 d64; B4 H16 N2048 d64; B16 H12 N1000 d64
with and without the mask), whole workload, on one core and on every host
thread, and prints the host's CPU model.

Counter helpers (used to produce the summaries under profiles/):
  python bench.py --copy-calibration ...   also runs one plain device copy
                                           of 1 GiB (for counter scaling)
  python bench.py --summarize-trace DIR CMD [K [FLOPS [PEAK]]]
                                                  per-kernel summary of a
                                                  --kernel-trace --stats run
                                                  (mean of the last K dispatches)
  python bench.py --summarize-counters FDIR WDIR WORKLOAD CMD [KERNEL]
                                                  traffic summary of the
                                                  FETCH_SIZE / WRITE_SIZE runs
  python bench.py --summarize-pmc KERNEL_SUBSTRING TRACE_DIR CMD DIR [DIR ...]
                                                  per-dispatch SQ/GRBM counters
                                                  of one kernel, with the mean
                                                  duration from a kernel trace
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU * 2.4 GHz * 4096 FLOP/clk
# MI355X fp32 vector ALU: 256 CU * 4 SIMD * 16 lanes * 2 fp32 values (packed
# FMA) * 2 FLOP * 2.4 GHz.  The library emits no packed fp32 instructions, so
# its vector code can reach half of this; the fp32 kernel runs on the vector
# ALUs, not the matrix cores (used only for fp32 workloads)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = ["exact_attention_32_amd/csrc/fa_fwd_bf16.hip",
                  "exact_attention_32_amd/csrc/fa_fwd_f32.hip"]
BWD_KERNEL_SOURCES = ["exact_attention_32_amd/csrc/fa_bwd_bf16.hip"]
COPY_BYTES = 1 << 30


def run_timed(step, stream, dev, steps: int):
    """The timed region: `steps` steps back to back on `stream`, synchronised
    on both sides.  Returns (wall seconds, mean milliseconds per step between
    one pair of HIP events recorded on the launch stream around the steps).
    The mean includes the dispatch gap between consecutive launches.  An
    event pair around every step would lengthen every step instead: the
    extra markers between launches measured 26 us per step at B2 H32 N8192
    d128 (1010 vs 978 us) and 5-8 us on launches of 10-50 us."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(steps):
            step()
        end.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of the kernel sources' code: comments and whitespace are removed
    first, so that editing a comment does not disown the committed counter
    summaries."""
    import re

    h = hashlib.sha256()
    for p in sources:
        text = open(os.path.join(ROOT, p), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """Bytes per launch from the committed counter summary of this workload
    (profiles/*_traffic.txt), or None when there is none for the current
    kernel source."""
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt"))):
        fields = {}
        for line in open(path):
            if ":" in line and line.split(":", 1)[0].isupper():
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("WORKLOAD") != workload:
            continue
        if fields.get("KERNEL_SOURCE_SHA256_16") != kernel_source_hash():
            continue
        try:
            return int(fields["HBM_BYTES_PER_LAUNCH"])
        except (KeyError, ValueError):
            continue
    return None


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


ORACLE_TIMING_WORKLOADS = ["w1_f32_n256_d64", "w2_bf16_b4h16_n2048_d64",
                           "w5a_bf16_b16h12_n1000_d64", "w5b_bf16_b16h12_n1000_d64_causal"]


def oracle_timing_child(name: str, threads: int) -> None:
    """Time the oracle's full forward pass (every row, the plain definition)
    on one workload with `threads` OpenMP threads; print one JSON line."""
    import oracle
    from exact_attention_32_amd import inputs

    w = inputs.WORKLOADS[name]
    q, k, v = inputs.make_qkv(w)
    o = oracle.default()
    o.set_num_threads(threads)
    o.attention(q[:, :1, :8], k[:, :1, :8], v[:, :1, :8], w.scale, w.causal)  # warm-up
    t0 = time.perf_counter()
    o.attention(q, k, v, w.scale, w.causal)
    dt = time.perf_counter() - t0
    print(json.dumps({"workload": name, "threads": o.num_threads(), "seconds": round(dt, 3),
                      "gflops": round(w.flops / dt / 1e9, 3)}), flush=True)


def oracle_timings() -> int:
    """The oracle on the small workloads, on one core and on every host
    thread, each in a child process (the OpenMP thread count is fixed at
    start-up).  One JSON line per run, then a summary line."""
    import subprocess

    rows = []
    # every thread this job may use: OMP_NUM_THREADS where the host sets a
    # share, else every host thread
    share = os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count() or 1)
    for name in ORACLE_TIMING_WORKLOADS:
        for threads in ("1", share):
            env = dict(os.environ, OMP_NUM_THREADS=threads)
            r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-timing-child",
                                name, "--oracle-threads", threads], env=env,
                               capture_output=True, text=True, check=True)
            line = json.loads(r.stdout.strip().splitlines()[-1])
            print(json.dumps(line), flush=True)
            rows.append(line)
    print(json.dumps({"oracle_timings": rows, "cpu_model": cpu_model(),
                      "host_threads": os.cpu_count(), "threads_used": int(share)}), flush=True)
    return 0


def cpu_baseline_bwd(w, q, k, v, dout, target_s: float):
    """The oracle's backward pass timed on the host cores on a seeded sample
    of dQ rows of the same workload.  For each row the oracle forms the
    score row, the dP row and the dQ row: three of the five products of the
    backward pass, so FLOPs per row = 3/5 of the workload's backward FLOPs
    divided by its number of rows."""
    import numpy as np

    import oracle
    from exact_attention_32_amd import inputs

    o = oracle.default()
    qd, kd, vd, dd = (t.float().numpy().astype(np.float64) for t in (q, k, v, dout))
    per_row = 0.6 * 2.5 * w.flops / (w.B * w.H * w.N)
    rows = inputs.sample_rows(w, 64, seed=99)
    t0 = time.perf_counter()
    o.attention_backward_dq_rows(qd, kd, vd, dd, w.scale, w.causal, rows)
    dt = max(time.perf_counter() - t0, 1e-3)
    n = int(min(200000, max(64, 64 * target_s / dt)))
    rows = inputs.sample_rows(w, n, seed=100)
    t0 = time.perf_counter()
    o.attention_backward_dq_rows(qd, kd, vd, dd, w.scale, w.causal, rows)
    dt = time.perf_counter() - t0
    return {
        "value": n * per_row / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": o.num_threads(),
        "kind": "oracle",
        "sample": f"{n} seeded dQ rows of {w.name} (fp64 definition: score, dP and dQ row "
                  f"each), {dt:.1f} s; FLOPs per row = 3/5 of the workload's backward "
                  f"FLOPs / rows",
        "cpu_model": cpu_model(),
    }


def cpu_baseline(w, q, k, v, target_s: float):
    """The oracle as it stands, timed on the host cores on a seeded sample of
    output rows of the same workload; nominal FLOPs per row are the
    workload's FLOPs divided by its number of rows."""
    import numpy as np

    import oracle
    from exact_attention_32_amd import inputs

    o = oracle.default()
    qd, kd, vd = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    per_row = w.flops / (w.B * w.H * w.N)
    # calibrate on a few rows, then size the sample to about target_s seconds
    rows = inputs.sample_rows(w, 64, seed=99)
    t0 = time.perf_counter()
    o.attention_rows(qd, kd, vd, w.scale, w.causal, rows)
    dt = max(time.perf_counter() - t0, 1e-3)
    n = int(min(200000, max(64, 64 * target_s / dt)))
    rows = inputs.sample_rows(w, n, seed=100)
    t0 = time.perf_counter()
    o.attention_rows(qd, kd, vd, w.scale, w.causal, rows)
    dt = time.perf_counter() - t0
    return {
        "value": n * per_row / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": o.num_threads(),
        "kind": "oracle",
        "sample": f"{n} seeded output rows of {w.name} (fp64 definition, full score row "
                  f"each), {dt:.1f} s; FLOPs per row = workload FLOPs / rows",
        "cpu_model": cpu_model(),
    }


def _db_rows(directory: str, query: str):
    import sqlite3

    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*_results.db"), recursive=True)):
        con = sqlite3.connect(path)
        rows += list(con.execute(query))
        con.close()
    return rows


def summarize_trace(directory: str, command: str, timed: int = 0, flops: float = 0.0,
                    peak: float = PEAK_BF16_TFLOPS) -> None:
    """Print the per-kernel summary of a `rocprofv3 --kernel-trace --stats`
    run (SQLite output under `directory`).  With `timed` > 0, also the mean
    duration of the last `timed` dispatches of the most frequent kernel (the
    timed steps of the traced bench command, after its warm-up launches) and,
    with `flops`, the TFLOP/s and fraction of the bf16 peak it gives."""
    print(f"COMMAND: {command}")
    print("KERNEL_SOURCE_SHA256_16:", kernel_source_hash())
    print("BWD_KERNEL_SOURCE_SHA256_16:", kernel_source_hash(BWD_KERNEL_SOURCES))
    print("kernel | calls | total_ms | average_us | percent")
    top = _db_rows(directory, "select name, total_calls, total_duration, average, percentage "
                              "from top_kernels")
    for name, calls, total, avg, pct in top:
        # rocprofv3 reports these two columns in microseconds
        print(f"{name} | {calls} | {total / 1e3:.3f} | {avg:.2f} | {pct:.1f}")
    for name, vgpr, agpr, sgpr, lds, scratch in _db_rows(
            directory, "select distinct name, vgpr_count, accum_vgpr_count, sgpr_count, "
                       "lds_size, scratch_size from kernels"):
        print(f"resources {name}: vgpr={vgpr} agpr={agpr} sgpr={sgpr} lds={lds} scratch={scratch}")
    if timed and top:
        name = max(top, key=lambda r: r[1])[0]
        durs = [d for n, d in _db_rows(directory, "select name, duration from kernels "
                                                  "order by start") if n == name]
        last = durs[-timed:]
        us = sum(last) / len(last) / 1e3
        print("DISPATCH_US (in order): " + ", ".join(f"{d / 1e3:.1f}" for d in durs))
        print(f"TIMED_DISPATCHES: last {len(last)} of {len(durs)}")
        print(f"TIMED_MEAN_US: {us:.2f}")
        if flops:
            tf = flops / (us * 1e-6) / 1e12
            print(f"TIMED_TFLOPS: {tf:.3f}")
            print(f"TIMED_FRACTION_OF_PEAK ({peak} TFLOP/s): {tf / peak:.4f}")


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, command: str,
                       kernel: str = "fwd_") -> None:
    """Print the traffic summary of two `rocprofv3 --pmc` runs of
    `bench.py --copy-calibration` (FETCH_SIZE in `fetch_dir`, WRITE_SIZE in
    `write_dir`) for the kernels whose name contains `kernel`.  Each counter
    is scaled by COPY_BYTES / (its reading for the plain device copy of
    COPY_BYTES that the same run performs)."""
    q = "select kernel_name, value from counters_collection where counter_name = '%s'"
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _db_rows(d, q % counter)
        fa_kib = [v for k, v in rows if kernel in k]
        copy_kib = [v for k, v in rows if "copyBuffer" in k]
        if not fa_kib or len(copy_kib) != 1:
            raise SystemExit(f"{counter}: expected attention launches and one copy in {d}")
        factor = COPY_BYTES / (copy_kib[0] * 1024.0)
        mean = sum(fa_kib) / len(fa_kib)
        out[counter] = (mean, factor, fa_kib, copy_kib[0])
    print(f"COMMAND: {command}")
    print(f"WORKLOAD: {workload}")
    print(f"KERNEL: {kernel}")
    print(f"KERNEL_SOURCE_SHA256_16: {kernel_source_hash()}")
    total = 0
    for counter, (mean, factor, vals, copy) in out.items():
        scaled = mean * 1024.0 * factor
        total += scaled
        print(f"{counter}_KIB_PER_LAUNCH: {mean:.1f} (launches: {', '.join(f'{v:.1f}' for v in vals)})")
        print(f"{counter}_COPY_KIB: {copy:.1f} for a copy of {COPY_BYTES} bytes -> factor {factor:.4f}")
        print(f"{counter}_BYTES_PER_LAUNCH_SCALED: {scaled:.0f}")
    print(f"HBM_BYTES_PER_LAUNCH: {total:.0f}")


def kvouter_bytes(w) -> float:
    """HBM bytes the key/value-outer order moves per call, counted per
    (query block i, key block j) step as Algorithm 1 states them: read Q_i
    and (after the first step) O_i, l_i, m_i; write O_i, l_i, m_i (fp32), or
    at a row block's last step the bf16 O_i and its LSE; K_j and V_j once per
    key block and head."""
    Br, Bc = 128, 64
    nqb, nkb = -(-w.N // Br), -(-w.N // Bc)
    total = 0.0
    for j in range(nkb):
        rows_j = min(Bc, w.N - j * Bc)
        total += 2 * rows_j * w.d * 2
        i0 = (j * Bc) // Br if w.causal else 0
        for i in range(i0, nqb):
            rows = min(Br, w.N - i * Br)
            last_row = min(w.N, (i + 1) * Br) - 1
            j_last = last_row // Bc if w.causal else nkb - 1
            total += rows * w.d * 2                      # Q_i
            if j > 0:
                total += rows * (w.d * 4 + 8)            # O_i, l_i, m_i read
            if j == j_last:
                total += rows * (w.d * 2 + 4)            # bf16 O_i and LSE
            else:
                total += rows * (w.d * 4 + 8)            # O_i, l_i, m_i written
    return total * w.B * w.H


def bench_decode(args) -> int:
    import numpy as np
    import torch

    import exact_attention_32_amd as fa
    from exact_attention_32_amd import inputs

    w = inputs.DECODE_WORKLOADS[args.workload or inputs.DECODE_HEADLINE]
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_decode_qkv(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    need = fa.fa_decode_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step():
        rc = fa.fa_decode(qd, kd, vd, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, w.causal, 0,
                          ws, need, stream)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, fa.fa_strerror(rc))

    torch.cuda.synchronize(dev)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    wall, kernel_ms = run_timed(step, stream, dev, args.steps)
    ms_per_step = wall * 1e3 / args.steps
    gbs = w.bytes / (ms_per_step * 1e-3) / 1e9
    achieved = w.bytes / (kernel_ms * 1e-3) / 1e9
    line = {
        "metric": "attention decode GB/s on 1 MI355X (bf16, compulsory HBM bytes) + % HBM peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "inputs": w.dist, "pass": "decode",
                   "bytes_per_step": w.bytes, "flops_per_step": w.flops,
                   "tflops": round(w.flops / (kernel_ms * 1e-3) / 1e12, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None, "kernel_ms": round(kernel_ms, 4)},
    }
    if not args.no_cpu_baseline:
        import oracle

        orc = oracle.default()
        qn, kn, vn = (t.float().numpy().astype(np.float64) for t in (q, k, v))
        t0 = time.perf_counter()
        reps = 0
        while True:
            orc.attention_qk(qn, kn, vn, w.scale, w.causal)
            reps += 1
            if time.perf_counter() - t0 > min(args.cpu_seconds, 10.0):
                break
        dt = (time.perf_counter() - t0) / reps
        line["cpu_baseline"] = {
            "value": round(w.bytes / dt / 1e9, 3), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"the whole workload {reps} time(s), {dt:.2f} s each (fp64 definition "
                      f"on the same bf16 inputs); bytes = the compulsory bf16 bytes",
            "cpu_model": cpu_model()}
    print(json.dumps(line), flush=True)
    return 0


def summarize_pmc(kernel: str, trace_dir: str, command: str, dirs) -> None:
    """Per-dispatch averages of the counters collected in the `--pmc` runs
    under `dirs` for the kernels whose name contains `kernel`, and derived
    figures.  SQ_BUSY_CYCLES is the sum over the 32 shader engines (8 XCDs x
    4) of their busy cycles; SQ_VALU_MFMA_BUSY_CYCLES the sum over the 1024
    SIMDs of their matrix-core busy cycles (32 per 32x32x16 MFMA, 16 per
    16x16x32).  Each counter record carries its dispatch's start and end, so
    the shader clock of a dispatch is SQ_BUSY_CYCLES / 32 / its duration; the
    MFMA-busy fraction is SQ_VALU_MFMA_BUSY_CYCLES / (1024 * SQ_BUSY_CYCLES /
    32) of the kernel's cycles, and SQ_VALU_MFMA_BUSY_CYCLES / (1024 *
    duration * 2.4 GHz) of the nominal peak; the VALU issue fraction = 4 *
    SQ_ACTIVE_INST_VALU (quad-cycles, MFMA issue included) / (1024 *
    SQ_BUSY_CYCLES / 32).  (GRBM_GUI_ACTIVE / 8 counts each XCD's cycles over
    the whole counter window around the dispatch: close to the shader
    engines' busy cycles for millisecond kernels, up to twice them for
    kernels of tens of microseconds; it is printed but not used.)
    `trace_dir` (a kernel trace of the same command) is reported beside
    them."""
    vals, clocks, busy, peak_frac = {}, [], [], []
    per_dispatch = {}
    for d in dirs:
        for name, counter, value, start, end, disp in _db_rows(
                d, "select kernel_name, counter_name, value, start, end, dispatch_id "
                   "from counters_collection"):
            if kernel in name:
                vals.setdefault(counter, []).append(value)
                per_dispatch.setdefault((d, disp), {})[counter] = (value, start, end)
    for rec in per_dispatch.values():
        if "SQ_BUSY_CYCLES" in rec:
            v, start, end = rec["SQ_BUSY_CYCLES"]
            if end > start:
                clocks.append(v / 32.0 / (end - start))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in rec:
                m = rec["SQ_VALU_MFMA_BUSY_CYCLES"][0]
                busy.append(m / (1024.0 * v / 32.0))
                if end > start:
                    peak_frac.append(m / 1024.0 / ((end - start) * 2.4))
    durs = [avg for name, _, _, avg, _ in _db_rows(
        trace_dir, "select name, total_calls, total_duration, average, percentage from top_kernels")
        if kernel in name]
    print(f"COMMAND: {command}")
    print(f"KERNEL: {kernel}")
    print("counter | dispatches | mean per dispatch")
    mean = {}
    for c in sorted(vals):
        mean[c] = sum(vals[c]) / len(vals[c])
        print(f"{c} | {len(vals[c])} | {mean[c]:.6g}")
    se_cycles = mean.get("SQ_BUSY_CYCLES", 0.0) / 32.0
    if se_cycles:
        print(f"BUSY_CYCLES_PER_DISPATCH_PER_SHADER_ENGINE: {se_cycles:.4g}")
    if clocks:
        print("SHADER_CLOCK_GHZ_PER_DISPATCH: " + ", ".join(f"{c:.3f}" for c in clocks))
        print(f"SHADER_CLOCK_GHZ: {sum(clocks) / len(clocks):.3f}")
    if busy:
        print(f"MFMA_BUSY_FRACTION: {sum(busy) / len(busy):.3f}")
    if peak_frac:
        print(f"MFMA_BUSY_FRACTION_AT_2.4GHZ: {sum(peak_frac) / len(peak_frac):.3f}")
    if durs:
        print(f"MEAN_DURATION_US (kernel trace, every dispatch): {durs[0]:.2f}")
    if se_cycles and "SQ_ACTIVE_INST_VALU" in mean:
        # SQ_ACTIVE_INST_VALU counts issue quad-cycles (4 clocks) summed over waves
        print(f"VALU_ISSUE_FRACTION: {4 * mean['SQ_ACTIVE_INST_VALU'] / (1024 * se_cycles):.3f}")
    if se_cycles and "SQ_INSTS_MFMA" in mean:
        per_simd = {c: mean[c] / 1024 for c in mean if c.startswith("SQ_INSTS")}
        print("INSTRUCTIONS_PER_SIMD_PER_DISPATCH: " +
              ", ".join(f"{c[9:]}={v:.4g}" for c, v in sorted(per_simd.items())))
        m = mean["SQ_INSTS_MFMA"]
        if m:
            print("PER_MFMA: " + ", ".join(f"{c[9:]}={mean[c] / m:.2f}"
                                          for c in sorted(mean) if c.startswith("SQ_INSTS")
                                          and c != "SQ_INSTS_MFMA"))
    if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_ACTIVE_INST_LDS" in mean and mean["SQ_ACTIVE_INST_LDS"]:
        print(f"LDS_BANK_CONFLICT_PER_LDS_ACTIVE_CYCLE: "
              f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_ACTIVE_INST_LDS']:.4f}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--dtype", choices=("bf16", "f16"), default=None,
                    help="forward pass: run the workload's shape in this type (fa_fwd_ex)")
    ap.add_argument("--layout", choices=("bhnd", "bnhd"), default="bhnd",
                    help="forward pass: memory order of q, k, v, o ([B,N,H,d] goes through "
                         "fa_fwd_ex as strided views)")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "decode", "kvouter"),
                    default="fwd")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-trace", nargs="+", metavar="ARG",
                    help="DIR COMMAND [TIMED_STEPS [FLOPS]]")
    ap.add_argument("--summarize-counters", nargs="+",
                    metavar="ARG", help="FETCH_DIR WRITE_DIR WORKLOAD COMMAND [KERNEL_SUBSTRING]")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG")
    ap.add_argument("--oracle-timings", action="store_true",
                    help="time the oracle on the small workloads on one core and on all "
                         "host threads (no GPU)")
    ap.add_argument("--oracle-timing-child", metavar="WORKLOAD", help=argparse.SUPPRESS)
    ap.add_argument("--oracle-threads", type=int, default=1, help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.oracle_timings:
        return oracle_timings()
    if args.oracle_timing_child:
        oracle_timing_child(args.oracle_timing_child, args.oracle_threads)
        return 0

    if args.summarize_trace:
        a = args.summarize_trace
        summarize_trace(a[0], a[1], int(a[2]) if len(a) > 2 else 0,
                        float(a[3]) if len(a) > 3 else 0.0,
                        float(a[4]) if len(a) > 4 else PEAK_BF16_TFLOPS)
        return 0
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters[:5])
        return 0
    if args.summarize_pmc:
        a = args.summarize_pmc
        summarize_pmc(a[0], a[1], a[2], a[3:])
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py: the library runs on one GPU (single-GPU kernels, no "
                  "collectives); run it with --gpus 1.", flush=True)
        return 2

    import torch

    import exact_attention_32_amd as fa
    from exact_attention_32_amd import inputs

    if args.which == "decode":
        return bench_decode(args)
    name = args.workload or inputs.HEADLINE
    w = inputs.WORKLOADS[name]
    if args.dtype and args.dtype != w.dtype:
        w = w.with_shape(dtype=args.dtype, name=f"{w.name}_as_{args.dtype}")
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)   # default priority
    fn = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32
    flops = w.flops

    def step():
        rc = fn(qd, kd, vd, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal, stream)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, fa.fa_strerror(rc))

    if args.which == "fwd" and (w.dtype == "f16" or args.layout == "bnhd"):
        if w.dtype == "f32":
            raise SystemExit("fa_fwd_ex takes bf16 or fp16")
        if args.layout == "bnhd":
            qd, kd, vd, o = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
                             for t in (qd, kd, vd, o))
        ex_strides = [x for t in (qd, kd, vd, o) for x in t.stride()[:3]]
        ex_dtype = fa.FA_DTYPE_FP16 if w.dtype == "f16" else fa.FA_DTYPE_BF16

        def step():  # noqa: F811
            rc = fa.fa_fwd_ex(ex_dtype, qd, kd, vd, o, lse, w.B, w.H, w.N, w.d, w.scale,
                              w.causal, ex_strides, stream)
            if rc != fa.FA_OK:
                raise fa.FAError(rc, fa.fa_strerror(rc))

    if args.which == "kvouter":
        if w.dtype != "bf16":
            raise SystemExit("the key/value-outer pass is bf16 only")
        kv_need = fa.fa_fwd_kv_outer_workspace_size(w.B, w.H, w.N, w.d)
        kv_ws = torch.empty(kv_need, dtype=torch.uint8, device=dev)

        def step():  # noqa: F811
            rc = fa.fa_fwd_kv_outer(qd, kd, vd, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal,
                                    kv_ws, kv_need, stream)
            if rc != fa.FA_OK:
                raise fa.FAError(rc, fa.fa_strerror(rc))

    if args.which == "bwd":
        if w.dtype != "bf16":
            raise SystemExit("the backward pass is bf16 only")
        dout = inputs.make_dout(w)
        dd = dout.to(dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
        delta = torch.empty_like(lse)
        with torch.cuda.stream(stream):
            step()                        # the forward pass's O and LSE
        torch.cuda.synchronize(dev)
        flops = 2.5 * w.flops

        def step():  # noqa: F811
            rc = fa.fa_bwd(qd, kd, vd, o, dd, lse, dq, dk, dv, delta, w.B, w.H, w.N, w.d,
                           w.scale, w.causal, stream)
            if rc != fa.FA_OK:
                raise fa.FAError(rc, fa.fa_strerror(rc))

    torch.cuda.synchronize(dev)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize(dev)

    # Timed region: K steps, synchronised on both sides; one event pair on
    # the launch stream around them gives the average launch duration.
    wall, kernel_ms = run_timed(step, stream, dev, args.steps)
    ms_per_step = wall * 1e3 / args.steps

    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    # bf16 and fp16 share the dense MFMA peak
    peak = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    metric = "attention fwd TFLOP/s on 1 MI355X (bf16, causal/non-causal) + % MFMA peak"
    roofline = {"bound": "alu" if w.dtype == "f32" else "mfma", "achieved": round(achieved, 2),
                "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": read_traffic(w.name) if args.which == "fwd" else None,
                "kernel_ms": round(kernel_ms, 4)}
    if args.which == "kvouter":
        nbytes = kvouter_bytes(w)
        gbs = nbytes / (kernel_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                    "kernel_ms": round(kernel_ms, 4), "algorithmic_bytes": nbytes}
    if args.which == "bwd":
        metric = "attention bwd TFLOP/s on 1 MI355X (bf16, causal/non-causal) + % MFMA peak"
    line = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "inputs": w.dist, "pass": args.which,
                   "layout": args.layout,
                   "flops_per_step": flops,
                   "pct_mfma_peak": round(100 * tflops / peak, 2)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        if args.which == "bwd":
            line["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, dout, args.cpu_seconds)
        else:
            line["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
