"""Benchmark of the small-row MXFP8 GEMM path on one MI355X.

A step is one pass of the decode-bucket workload: for each batch size M in
{1, 2, 4, 8}, BF16 activations x [M, 5120] are quantized to MXFP8 and
multiplied by an MXFP8 weight [4096, 5120] (BF16 out), quantize and GEMM in
one mxfp8_gemm launch.  Inputs are resident in HBM before the timed region.
Weights rotate over enough identical copies (>= 1 GB) that no launch finds
its weight in the 256 MB Infinity Cache.  The K timed steps are captured in
one HIP graph (torch.cuda.CUDAGraph); the graph is replayed R >= 30 times,
each replay (exactly K steps) bracketed by HIP events on the launch stream
and a device synchronize, and the median replay gives the figures (the
spread over the replays is reported beside it).

Prints one JSON line: throughput in algorithmic GB/s (weights + weight scales
+ BF16 activations + the MXFP8 activations written + BF16 output, per step),
the dominant kernel's roofline against MI355X's 8 TB/s HBM peak, the launch
floor (a one-workgroup launch in the same graph timing), per-configuration
latencies with the kernel launches per call and the MFMA activity from the
committed counter profile, and the CPU oracle's throughput on the same
workload (all host threads, and one).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--replays R]
                    [--no-cases] [--no-cpu] [--only NAME] [--roofline-only]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mxfp8_block_scaled_gemm_amd as mx  # noqa: E402
from mxfp8_block_scaled_gemm_amd import probe as mxprobe  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MALL_BYTES = 256 << 20         # Infinity Cache
ROTATE_BYTES = 1 << 30         # weight bytes cycled through before a copy is reused (>= 1 GB)


REPLAYS = 30                   # graph replays per timing; the median is reported
MFMA_PEAK_FLOPS = 5.0e15       # MI355X dense FP8 (MXFP8) matrix peak
CASES_PROFILE = os.path.join(ROOT, "profiles", "bench_cases_mfma_and_launches.md")
ROOFLINE_PROFILE = os.path.join(ROOT, "profiles", "gemm_m16_kernel_fq_M1-2-4_N4096_K5120.md")
ROOFLINE_KERNEL = "gemm_m16_kernel<16,3,1,true> (M=1,2,4 with BF16 input, N=4096 K=5120)"
ROOFLINE_MS = (1, 2, 4)
ROOFLINE_SOURCES = [os.path.join(ROOT, "mxfp8_block_scaled_gemm_amd", "csrc", f)
                    for f in ("gemm.hip", "mx_device.hpp")]


def _sources_sha(files=None):
    import hashlib
    return [hashlib.sha256(open(f, "rb").read()).hexdigest() for f in (files or ROOFLINE_SOURCES)]


def _library_sources():
    """Every source of libmxgemm.so (kernels, launchers, host code), sorted."""
    import glob
    d = os.path.join(ROOT, "mxfp8_block_scaled_gemm_amd", "csrc")
    return sorted(glob.glob(os.path.join(d, "*.hip")) + glob.glob(os.path.join(d, "*.hpp")) +
                  glob.glob(os.path.join(d, "*.cpp")))


def profiled_roofline():
    """From the roofline kernel's committed summary: HBM bytes per launch
    (FETCH_SIZE + WRITE_SIZE, calibrated) and the kernel-trace average
    duration in us, each None when the kernel's sources changed since."""
    try:
        fields = dict(l.split(":", 1) for l in open(ROOFLINE_PROFILE).read().splitlines()
                      if l.startswith(("traffic_bytes_per_launch:", "sources_sha256:",
                                       "trace_avg_ns:")))
        if fields["sources_sha256"].split() != _sources_sha():
            return None, None
        return (int(fields["traffic_bytes_per_launch"]),
                float(fields["trace_avg_ns"]) / 1e3 if "trace_avg_ns" in fields else None)
    except (OSError, KeyError, ValueError):
        return None, None


def profiled_cases():
    """Per-case counters from the committed profile of every bench case:
    {case: {"launches": kernel launches per call, "mops": F8 MFMA MOPS per
    call, "busy": SQ_VALU_MFMA_BUSY_CYCLES per call}}, empty when any source of
    the library changed since the profile was taken (its `sources_sha256:`
    line holds the SHA-256 of every csrc file, in sorted path order)."""
    out = {}
    try:
        text = open(CASES_PROFILE).read()
        sha = [l.split(":", 1)[1].split() for l in text.splitlines() if l.startswith("sources_sha256:")]
        if not sha or sha[0] != _sources_sha(_library_sources()):
            return {}
        for line in text.splitlines():
            if line.startswith("| `") and line.count("|") >= 6:
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                name = cells[0].strip("`")
                out[name] = {"launches": int(cells[1]), "mops": float(cells[2]),
                             "busy": float(cells[3])}
    except (OSError, ValueError, IndexError):
        return {}
    return out


def mx_bytes(rows: int, K: int) -> int:
    return rows * K + rows * (K // 32)


def gemm_bytes(M: int, N: int, K: int, bf16_in: bool) -> int:
    """Algorithmic HBM bytes of one call: W codes + scales, activations
    (BF16 read + MXFP8 written when quantizing in-kernel, else MXFP8 read),
    BF16 output."""
    act = 2 * M * K + mx_bytes(M, K) if bf16_in else mx_bytes(M, K)
    return mx_bytes(N, K) + act + 2 * M * N


def weight_copies(N: int, K: int, dev, row_major: bool = False):
    """Identical MXFP8 weight copies, enough to cycle ROTATE_BYTES (packed, or
    [N, K] / [N, K/32] as quantized with row_major)."""
    q, s = mx.mxfp8_quantize(synth.gemm_case(1, N, K, seed=0)["w"].to(dev))
    w = mx.RowMajorWeight(q, s) if row_major else mx.PackedWeight.from_rows(q, s)
    n = max(16, math.ceil(ROTATE_BYTES / mx_bytes(N, K)))
    return [w.clone() for _ in range(n)]


def time_graph(fn, reps: int, stream, replays: int = None) -> dict:
    """Capture fn(i) for i < reps into one graph and replay it `replays`
    times, each replay between HIP events on `stream` followed by a device
    synchronize.  Returns the median, minimum and maximum milliseconds of one
    replay (reps calls)."""
    replays = REPLAYS if replays is None else replays
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fn(i)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()                                     # first replay: not timed
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            start.record(stream)
            g.replay()
            end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end))
    times.sort()
    return {"ms": times[len(times) // 2], "min": times[0], "max": times[-1], "replays": replays}


def per_call_us(t: dict, reps: int) -> dict:
    return {k: t[k] * 1e3 / reps for k in ("ms", "min", "max")}


def decode_bucket(dev, steps: int, warmup: int, stream):
    """The decode-bucket workload (M = 1, 2, 4, 8; N = 4096; K = 5120); returns
    the timing record."""
    N, K, Ms = 4096, 5120, (1, 2, 4, 8)
    copies = weight_copies(N, K, dev)
    x8 = synth.gemm_case(8, N, K, seed=0)["x"].to(dev)
    bufs = {}
    for M in Ms:
        bufs[M] = (x8[:M].contiguous(),
                   torch.empty(M, K, dtype=torch.uint8, device=dev),
                   torch.empty(M, K // 32, dtype=torch.uint8, device=dev),
                   torch.empty(M, N, dtype=torch.bfloat16, device=dev))

    def step(i):
        for j, M in enumerate(Ms):
            w = copies[(len(Ms) * i + j) % len(copies)]
            x, aq, as_, out = bufs[M]
            mx.mxfp8_gemm(aq, as_, w, out=out, x=x)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()
    t = time_graph(lambda i: step(warmup + i), steps, stream)
    step_bytes = sum(gemm_bytes(M, N, K, True) for M in Ms)
    per_m = {}
    for M in Ms:     # one graph per M, for the per-size latency
        def one(i, M=M):
            x, aq, as_, out = bufs[M]
            mx.mxfp8_gemm(aq, as_, copies[i % len(copies)], out=out, x=x)
        u = per_call_us(time_graph(one, 400, stream), 400)
        per_m[str(M)] = {"us": round(u["ms"], 3), "us_min": round(u["min"], 3),
                         "us_max": round(u["max"], 3),
                         "GBs": round(gemm_bytes(M, N, K, True) / (u["ms"] * 1e-6) / 1e9, 1)}
    # Warm cache: the same step on one weight copy, reused by every call, so
    # the weights come from the 256 MB MALL rather than HBM (labelled as such,
    # never the headline).
    def warm_step(i):
        for M in Ms:
            x, aq, as_, out = bufs[M]
            mx.mxfp8_gemm(aq, as_, copies[0], out=out, x=x)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            warm_step(i)
    tw = time_graph(warm_step, steps, stream)
    return {
        "ms_per_step": t["ms"] / steps,
        "ms_per_step_min": t["min"] / steps,
        "ms_per_step_max": t["max"] / steps,
        "replays": t["replays"],
        "step_bytes": step_bytes,
        "GBs": step_bytes * steps / (t["ms"] * 1e-3) / 1e9,
        "kernel_us": t["ms"] * 1e3 / (steps * len(Ms)),
        "per_m": per_m,
        "copies": len(copies),
        "warm": {"ms_per_step": tw["ms"] / steps,
                 "GBs": step_bytes * steps / (tw["ms"] * 1e-3) / 1e9},
    }


def roofline_kernel(dev, stream, reps: int = 200):
    """The step's dominant kernel alone: the M <= 16 GEMM kernel with the
    quantize fused (one 32-block per thread), which serves the M = 1, 2 and 4
    GEMMs of the step (three of its four launches, about 70 % of its time).
    `reps` rounds of those three launches on rotated weights in one HIP
    graph, timed with HIP events on its launch stream; per launch: the mean
    algorithmic bytes over the three, and the median replay's mean duration."""
    N, K = 4096, 5120
    copies = weight_copies(N, K, dev)
    x8 = synth.gemm_case(8, N, K, seed=0)["x"].to(dev)
    bufs = [(x8[:M].contiguous(),
             torch.empty(M, K, dtype=torch.uint8, device=dev),
             torch.empty(M, K // 32, dtype=torch.uint8, device=dev),
             torch.empty(M, N, dtype=torch.bfloat16, device=dev)) for M in ROOFLINE_MS]

    def call(i):
        for j, (x, aq, as_, out) in enumerate(bufs):
            mx.mxfp8_gemm(aq, as_, copies[(len(bufs) * i + j) % len(copies)], out=out, x=x)
    with torch.cuda.stream(stream):
        for i in range(10):
            call(i)
    launches = reps * len(ROOFLINE_MS)
    u = per_call_us(time_graph(call, reps, stream), launches)
    b = sum(gemm_bytes(M, N, K, True) for M in ROOFLINE_MS) / len(ROOFLINE_MS)
    return {"us": u["ms"], "us_min": u["min"], "us_max": u["max"], "bytes": b,
            "GBs": b / (u["ms"] * 1e-6) / 1e9, "launches": launches}


def stream_ceiling(dev, stream, reps: int = 600):
    """The single-launch streaming floor for the roofline kernel's weight:
    the library's read-only probe reading the same rotated weight copies
    (N=4096, K=5120) with the same load pattern, one HIP graph of `reps`
    launches timed with HIP events on its launch stream."""
    N, K = 4096, 5120
    copies = weight_copies(N, K, dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def call(i):
        mxprobe.hbm_read_probe(copies[i % len(copies)], sink)
    with torch.cuda.stream(stream):
        for i in range(20):
            call(i)
    u = per_call_us(time_graph(call, reps, stream), reps)
    b = mx_bytes(N, K)
    return {"us": u["ms"], "bytes": b, "GBs": b / (u["ms"] * 1e-6) / 1e9}


def launch_floor(dev, stream, reps: int = 600):
    """The per-launch floor in the same graph timing: the read-only probe on
    one 16 x 128 tile (one workgroup, 2 KiB), launched back to back."""
    w = mx.PackedWeight.from_bf16(synth.gemm_case(1, 16, 128, seed=0)["w"].to(dev))
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def call(i):
        mxprobe.hbm_read_probe(w, sink)
    with torch.cuda.stream(stream):
        for i in range(20):
            call(i)
    return per_call_us(time_graph(call, reps, stream), reps)["ms"]


def case_record(name: str, u: dict, nbytes: int, prof: dict, floor_us: float, **extra) -> dict:
    """One bench case: median us per call (and the replays' spread), GB/s,
    fraction of 8 TB/s, kernel launches per call and their floor, and MFMA
    activity from the committed counter profile (null when not profiled for
    the current sources)."""
    rec = {"us": round(u["ms"], 3), "us_min": round(u["min"], 3), "us_max": round(u["max"], 3),
           "GBs": round(nbytes / (u["ms"] * 1e-6) / 1e9, 1),
           "frac": round(nbytes / (u["ms"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    rec.update(extra)
    pc = prof.get(name)
    if pc:
        rec["launches"] = pc["launches"]
        rec["launch_floor_us"] = round(pc["launches"] * floor_us, 3)
        # issued scaled-MFMA FLOPs (one MOP = 512 flops) over the call's time
        # against the dense FP8 peak, and the matrix-core busy fraction
        rec["mfma_util"] = round(pc["mops"] * 512 / (u["ms"] * 1e-6) / MFMA_PEAK_FLOPS, 5)
        rec["mfma_busy"] = round(pc["busy"] / (256 * 4 * u["ms"] * 1e-6 * 2.4e9), 5)
    else:
        rec["launches"] = rec["launch_floor_us"] = rec["mfma_util"] = rec["mfma_busy"] = None
    return rec


def chain_case(dev, stream, M: int, reps: int = 200, norm: bool = False):
    """The three-projection chain (A 2048x5120, requantize 1536 columns, B
    8192x1536, C 5120x8192), weights rotated over copies.  norm: the 1536
    columns are RMS-normalised before the requantize (the gain's 3 KB and the
    normalised BF16 are counted).  Returns (per-call us, algorithmic bytes)."""
    case = synth.chain_case(M, seed=0)
    w = {k: mx.PackedWeight.from_bf16(case[k].to(dev)) for k in ("w_a", "w_b", "w_c")}
    per = sum(mx_bytes(v.N, v.K) for v in w.values())
    n = max(16, math.ceil(ROTATE_BYTES / per))
    cop = [{k: v.clone() for k, v in w.items()} for _ in range(n)]
    a = mx.mxfp8_quantize(case["x_a"].to(dev))
    c = mx.mxfp8_quantize(case["x_c"].to(dev))
    outs = (torch.empty(M, 2048, dtype=torch.bfloat16, device=dev),
            torch.empty(M, 1536, dtype=torch.uint8, device=dev),
            torch.empty(M, 48, dtype=torch.uint8, device=dev),
            torch.empty(M, 8192, dtype=torch.bfloat16, device=dev),
            torch.empty(M, 5120, dtype=torch.bfloat16, device=dev))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    gain = synth.rmsnorm_case(1, 1536, seed=1)["w"].to(dev) if norm else None
    b_bf16 = torch.empty(M, 1536, dtype=torch.bfloat16, device=dev) if norm else None

    def call(i):
        cw = cop[i % n]
        mx.mxfp8_proj_chain(*a, cw["w_a"], cw["w_b"], *c, cw["w_c"], outs=outs, workspace=ws,
                            norm_weight=gain, norm_eps=synth.RMSNORM_EPS, b_bf16=b_bf16)
    with torch.cuda.stream(stream):
        for i in range(10):
            call(i)
    u = per_call_us(time_graph(call, reps, stream), reps)
    b = per + mx_bytes(M, 5120) + mx_bytes(M, 8192) + 2 * M * (2048 + 8192 + 5120) \
        + 2 * M * 1536 + mx_bytes(M, 1536) + ((2 * 1536 + 2 * M * 1536) if norm else 0)
    return u, b


def rmsnorm_case(dev, stream, M: int, K: int, ld: int, reps: int = 400):
    """RMSNorm + MXFP8 of the leading K columns of BF16 rows of stride ld
    (the chain's 1536 of 2048, or a 5120-wide layer input), writing the
    normalised BF16 too.  A few KB per row: launch-bound, reported in us."""
    case = synth.rmsnorm_case(M, K, seed=0, ld=ld)
    x, w = case["x"].to(dev), case["w"].to(dev)
    y = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    q = torch.empty(M, K, dtype=torch.uint8, device=dev)
    s = torch.empty(M, K // 32, dtype=torch.uint8, device=dev)

    def call(i):
        mx.mxfp8_rmsnorm_quantize(x, w, case["eps"], K=K, y=y, q=q, s=s)
    with torch.cuda.stream(stream):
        for i in range(10):
            call(i)
    u = per_call_us(time_graph(call, reps, stream), reps)
    return u, 2 * M * K + 2 * K + 2 * M * K + mx_bytes(M, K)


def wo_a_case(dev, stream, M: int, reps: int = 200):
    """Rotary + grouped WO-A (8 groups of 8 heads x 512 dims, rank 1024) +
    MXFP8 of z + wo_b 5120x8192, weights rotated over copies."""
    case = synth.wo_a_case(M, seed=0)
    d = case["dims"]
    G, R = d["n_groups"], d["rank"]
    wa = mx.PackedWeight.from_bf16(case["w_a"].reshape(G * R, -1).to(dev))
    wb = mx.PackedWeight.from_bf16(case["w_b"].to(dev))
    per = mx_bytes(wa.N, wa.K) + mx_bytes(wb.N, wb.K)
    n = max(16, math.ceil(ROTATE_BYTES / per))
    cop = [(wa.clone(), wb.clone()) for _ in range(n)]
    o = case["o"].to(dev)
    pos = case["positions"].to(dev)
    cs = torch.from_numpy(case["cos_sin"]).to(dev)
    outs = (None, torch.empty(M, G * R, dtype=torch.uint8, device=dev),
            torch.empty(M, G * R // 32, dtype=torch.uint8, device=dev),
            torch.empty(M, wb.N, dtype=torch.bfloat16, device=dev))
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device=dev)

    def call(i):
        a, b = cop[i % n]
        mx.wo_a_fused_quantize(o, pos, cs, a, n_groups=G, nope_dim=d["nope"], wb=b, outs=outs,
                               workspace=ws)
    with torch.cuda.stream(stream):
        for i in range(10):
            call(i)
    u = per_call_us(time_graph(call, reps, stream), reps)
    H, D = d["n_heads"], d["head_dim"]
    b = per + 2 * M * H * D + 8 * M + 4 * M * (D - d["nope"]) + mx_bytes(M, G * R) + 2 * M * wb.N
    return u, b


def gemm_case_timing(dev, stream, copies, M, N, K, outliers, reps):
    x = synth.gemm_case(M, 16, K, seed=0, outliers=outliers)["x"].to(dev)
    aq, as_ = mx.mxfp8_quantize(x)
    o = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    def call(i):
        mx.mxfp8_gemm(aq, as_, copies[i % len(copies)], out=o)
    with torch.cuda.stream(stream):
        for i in range(20):
            call(i)
    return per_call_us(time_graph(call, reps, stream), reps)


def case_names():
    """Every bench case, in run order (names are stable keys of the JSON line
    and of the committed counter profile)."""
    names = ["single M4 N1024 K2048"]
    for (N, K) in ((4096, 5120), (5120, 8192), (8192, 1536)):
        names += [f"M{M} N{N} K{K}" for M in (16, 32, 48)]
    names += [f"rows above 48: M{M} N4096 K5120" for M in (64, 128, 256)]
    names += [f"row-major weights: M{M} N4096 K5120" for M in (1, 8, 48)]
    names += [f"chain M{M}" for M in (1, 8, 32)]
    names += [f"chain+norm M{M}" for M in (1, 8, 32)]
    names += [f"rmsnorm+quantize M{M} K{K}" for M in (1, 8, 48) for K in (1536, 5120)]
    names += [f"wo_a+wo_b M{M}" for M in (1, 4, 16)]
    return names


def extra_cases(dev, stream, floor_us, only=None, reps=None):
    """Latency of every other configuration: single GEMMs with MXFP8 inputs
    (M 4 at N 1024, K 2048; the wide tiles with outliers; rows above 48; the
    weight read row-major without a repack), the chain with and without the
    norm, RMSNorm + MXFP8, WO-A + wo_b.  `only`: run the
    cases whose name contains it (profiling one case at a time)."""
    prof = profiled_cases()
    out = {}
    # a case's exact name selects that case alone, other text every case containing it
    exact = only in case_names()
    want = lambda name: only is None or (name == only if exact else only in name)
    r = lambda default: reps or default
    specs = [("single M4 N1024 K2048", 4, 1024, 2048, False, False)]
    for (N, K) in ((4096, 5120), (5120, 8192), (8192, 1536)):
        specs += [(f"M{M} N{N} K{K}", M, N, K, True, False) for M in (16, 32, 48)]
    specs += [(f"rows above 48: M{M} N4096 K5120", M, 4096, 5120, False, False)
              for M in (64, 128, 256)]
    specs += [(f"row-major weights: M{M} N4096 K5120", M, 4096, 5120, False, True)
              for M in (1, 8, 48)]
    by_weight = {}
    for spec in specs:
        if want(spec[0]):
            by_weight.setdefault((spec[2], spec[3], spec[5]), []).append(spec)
    for (N, K, row_major), group in by_weight.items():
        copies = weight_copies(N, K, dev, row_major)
        for (name, M, _, _, outliers, _) in group:
            u = gemm_case_timing(dev, stream, copies, M, N, K, outliers, r(400 if M <= 48 else 200))
            extra = {}
            if M > 48:
                extra["TFLOPs"] = round(2 * M * N * K / (u["ms"] * 1e-6) / 1e12, 1)
            out[name] = case_record(name, u, gemm_bytes(M, N, K, False), prof, floor_us, **extra)
        del copies
        torch.cuda.empty_cache()
    for M in (1, 8, 32):
        if want(f"chain M{M}"):
            u, b = chain_case(dev, stream, M, reps=r(200))
            out[f"chain M{M}"] = case_record(f"chain M{M}", u, b, prof, floor_us)
    for M in (1, 8, 32):
        if want(f"chain+norm M{M}"):
            u, b = chain_case(dev, stream, M, reps=r(200), norm=True)
            out[f"chain+norm M{M}"] = case_record(f"chain+norm M{M}", u, b, prof, floor_us)
    for M in (1, 8, 48):
        for K, ld in ((1536, 2048), (5120, 5120)):
            name = f"rmsnorm+quantize M{M} K{K}"
            if want(name):
                u, b = rmsnorm_case(dev, stream, M, K, ld, reps=r(400))
                rec = case_record(name, u, b, prof, floor_us)
                rec.pop("frac")          # launch-bound: a few KB per row
                out[name] = rec
    for M in (1, 4, 16):
        if want(f"wo_a+wo_b M{M}"):
            u, b = wo_a_case(dev, stream, M, reps=r(200))
            out[f"wo_a+wo_b M{M}"] = case_record(f"wo_a+wo_b M{M}", u, b, prof, floor_us)
    return out


def cpu_baseline(min_seconds: float = 10.0, t1_seconds: float = 4.0):
    """The oracle (plain C, fp64) on the same decode-bucket step: quantize each
    M-row batch and run the GEMM against the full weight; repeated until
    min_seconds have elapsed with every host thread the process may use, then
    the same step with one thread for t1_seconds."""
    import oracle
    N, K, Ms = 4096, 5120, (1, 2, 4, 8)
    case = synth.gemm_case(8, N, K, seed=0)
    wq, ws = oracle.quantize(synth.bits(case["w"]))       # weight quantize: not timed
    xb = synth.bits(case["x"])
    step_bytes = sum(gemm_bytes(M, N, K, True) for M in Ms)

    def run(threads, seconds):
        used = oracle.set_threads(threads)
        reps, t0 = 0, time.perf_counter()
        while True:
            for M in Ms:
                q, s = oracle.quantize(xb[:M])
                oracle.gemm(q, s, wq, ws)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return used, reps, el
    threads, reps, el = run(len(os.sched_getaffinity(0)), min_seconds)
    _, reps1, el1 = run(1, t1_seconds)
    return {"value": round(step_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} full decode-bucket steps (M=1,2,4,8; N=4096; K=5120) in {el:.1f} s, "
                      f"{el / reps:.3f} s/step",
            "t1": {"value": round(step_bytes * reps1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                   "sample": f"{reps1} steps in {el1:.1f} s, {el1 / reps1:.3f} s/step"}}


def main():
    global REPLAYS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replays", type=int, default=REPLAYS,
                    help="graph replays per timing (the median is reported)")
    ap.add_argument("--no-cases", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run only the bench cases whose name contains this text (profiling)")
    ap.add_argument("--reps", type=int, default=None,
                    help="calls per captured graph in the cases (default per case)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the dominant kernel's timing (for profiler runs)")
    args = ap.parse_args()
    REPLAYS = max(1, args.replays)
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (asked for {args.gpus}); the "
              "multi-GPU sharding of the path is a design note, not a measured mode.",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()
    if args.roofline_only:
        # Calibration for the HBM byte counters: an elementwise kernel that
        # reads and writes exactly 64 MiB each (float32 add), then the kernel.
        src = torch.ones(16 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"roofline_kernel_us": roofline_kernel(dev, stream)["us"],
                          "calibration_bytes_each_way": 64 << 20}), flush=True)
        return
    if args.only is not None:
        floor = launch_floor(dev, stream)
        print(json.dumps({"only": args.only, "launch_floor_us": round(floor, 3),
                          "cases": extra_cases(dev, stream, floor, only=args.only,
                                               reps=args.reps)}), flush=True)
        return
    rec = decode_bucket(dev, args.steps, args.warmup, stream)
    roof = roofline_kernel(dev, stream)
    ceil = stream_ceiling(dev, stream)
    floor = launch_floor(dev, stream)
    cases = {} if args.no_cases else extra_cases(dev, stream, floor, reps=args.reps)
    cpu = None if args.no_cpu else cpu_baseline()
    traffic, prof_us = profiled_roofline()
    line = {
        "metric": "µs per MXFP8 GEMM at M=1..48; achieved HBM GB/s vs 8 TB/s peak",
        "value": round(rec["GBs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 e4m3 (e8m0/32 scales), fp32 accumulate, bf16 out",
        "data": "synthetic: x~N(0,1), W~N(0,0.02), seed 0",
        "config": {"workload": "decode-bucket MXFP8 GEMM with fused bf16->MXFP8 quantize, "
                               "M in {1,2,4,8}, N=4096, K=5120",
                   "M": [1, 2, 4, 8], "N": 4096, "K": 5120,
                   "weight_copies": rec["copies"],
                   "timing": f"median of {rec['replays']} replays of a HIP graph of the K steps, "
                             "each between HIP events"},
        "ms_per_step_min": round(rec["ms_per_step_min"], 5),
        "ms_per_step_max": round(rec["ms_per_step_max"], 5),
        "us_per_gemm": rec["per_m"],
        "roofline": {"bound": "hbm", "kernel": ROOFLINE_KERNEL,
                     "achieved": round(roof["GBs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(roof["GBs"] / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(roof["us"], 3),
                     "bytes_per_launch": int(roof["bytes"]),
                     "traffic": traffic,
                     # the same kernel's average duration under the profiler's
                     # kernel trace (committed summary), and the fraction it gives
                     "profile_avg_launch_us": round(prof_us, 3) if prof_us else None,
                     "frac_profile": (round(roof["bytes"] / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                      if prof_us else None)},
        "stream_ceiling": {"kernel": "hbm_read_kernel: the same weight copies read with the "
                                     "same load pattern, nothing else",
                           "us": round(ceil["us"], 3), "GBs": round(ceil["GBs"], 1),
                           "frac": round(ceil["GBs"] / HBM_PEAK_GBS, 4),
                           "roofline_vs_ceiling": round(roof["GBs"] / ceil["GBs"], 4)},
        "launch_floor_us": round(floor, 3),
        "step_avg_launch_us": round(rec["kernel_us"], 3),
        "warm_cache": {"note": "the same step with one weight copy reused by every call: the "
                               "weights are served from the 256 MB MALL, not HBM; not the headline",
                       "ms_per_step": round(rec["warm"]["ms_per_step"], 5),
                       "GBs": round(rec["warm"]["GBs"], 1)},
        "cases": cases,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
