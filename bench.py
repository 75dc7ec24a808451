"""Benchmark of the small-row MXFP8 GEMM path on one MI355X.

A step is one pass of the decode-bucket workload: for each batch size M in
{1, 2, 4, 8}, BF16 activations x [M, 5120] are quantized to MXFP8 and
multiplied by an MXFP8 weight [4096, 5120] (BF16 out), quantize and GEMM in
one mxfp8_gemm launch.  Inputs are resident in HBM before the timed region.
Weights rotate over enough identical copies (>= 512 MB) that no launch finds
its weight in the 256 MB Infinity Cache.  The K timed steps are captured in a
HIP graph (torch.cuda.CUDAGraph) and replayed once between HIP events on the
launch stream.

Prints one JSON line: throughput in algorithmic GB/s (weights + weight scales
+ BF16 activations + the MXFP8 activations written + BF16 output, per step),
the GEMM kernel's roofline against MI355X's 8 TB/s HBM peak, per-configuration
latencies, and the CPU oracle's throughput on the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cases] [--no-cpu]
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
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MALL_BYTES = 256 << 20         # Infinity Cache
ROTATE_BYTES = 512 << 20       # weight bytes cycled through before a copy is reused


ROOFLINE_PROFILE = os.path.join(ROOT, "profiles", "gemm_m16_kernel_fq_M1-2-4_N4096_K5120.md")
ROOFLINE_KERNEL = "gemm_m16_kernel<16,3,1,true> (M=1,2,4 with BF16 input, N=4096 K=5120)"
ROOFLINE_MS = (1, 2, 4)
ROOFLINE_SOURCES = [os.path.join(ROOT, "mxfp8_block_scaled_gemm_amd", "csrc", f)
                    for f in ("gemm.hip", "mx_device.hpp")]


def profiled_traffic():
    """HBM bytes per launch of the roofline kernel from its committed counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated), or None when the kernel's
    sources changed since the counters were taken."""
    import hashlib
    try:
        fields = dict(l.split(":", 1) for l in open(ROOFLINE_PROFILE).read().splitlines()
                      if l.startswith(("traffic_bytes_per_launch:", "sources_sha256:")))
        want = fields["sources_sha256"].split()
        have = [hashlib.sha256(open(f, "rb").read()).hexdigest() for f in ROOFLINE_SOURCES]
        return int(fields["traffic_bytes_per_launch"]) if want == have else None
    except (OSError, KeyError, ValueError):
        return None


def mx_bytes(rows: int, K: int) -> int:
    return rows * K + rows * (K // 32)


def gemm_bytes(M: int, N: int, K: int, bf16_in: bool) -> int:
    """Algorithmic HBM bytes of one call: W codes + scales, activations
    (BF16 read + MXFP8 written when quantizing in-kernel, else MXFP8 read),
    BF16 output."""
    act = 2 * M * K + mx_bytes(M, K) if bf16_in else mx_bytes(M, K)
    return mx_bytes(N, K) + act + 2 * M * N


def weight_copies(N: int, K: int, dev):
    """Identical MXFP8 weight copies, enough to cycle ROTATE_BYTES."""
    w = mx.PackedWeight.from_bf16(synth.gemm_case(1, N, K, seed=0)["w"].to(dev))
    n = max(2, math.ceil(ROTATE_BYTES / mx_bytes(N, K)))
    return [w.clone() for _ in range(n)]


def time_graph(fn, reps: int, stream) -> float:
    """Capture fn(i) for i < reps into one graph, replay it once between
    events; returns milliseconds for the reps calls."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        g.replay()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)


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
    ms = time_graph(lambda i: step(warmup + i), steps, stream)
    step_bytes = sum(gemm_bytes(M, N, K, True) for M in Ms)
    launches = steps * len(Ms)
    per_launch_s = ms * 1e-3 / launches
    per_launch_bytes = step_bytes / len(Ms)
    per_m = {}
    for M in Ms:     # one graph per M, for the per-size latency
        wq_list = copies

        def one(i, M=M):
            x, aq, as_, out = bufs[M]
            mx.mxfp8_gemm(aq, as_, wq_list[i % len(wq_list)], out=out, x=x)
        reps = 400
        t = time_graph(one, reps, stream) * 1e3 / reps
        per_m[str(M)] = {"us": round(t, 3),
                         "GBs": round(gemm_bytes(M, N, K, True) / (t * 1e-6) / 1e9, 1)}
    return {
        "ms_total": ms,
        "ms_per_step": ms / steps,
        "step_bytes": step_bytes,
        "GBs": step_bytes * steps / (ms * 1e-3) / 1e9,
        "kernel_us": per_launch_s * 1e6,
        "kernel_GBs": per_launch_bytes / per_launch_s / 1e9,
        "per_launch_bytes": per_launch_bytes,
        "per_m": per_m,
        "copies": len(copies),
    }


def roofline_kernel(dev, stream, reps: int = 200):
    """The step's dominant kernel alone: the M <= 16 GEMM kernel with the
    quantize fused (one 32-block per thread), which serves the M = 1, 2 and 4
    GEMMs of the step (three of its four launches, about 70 % of its time).
    `reps` rounds of those three launches on rotated weights in one HIP
    graph, timed with HIP events on its launch stream; per launch: the mean
    algorithmic bytes over the three, and the mean duration."""
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
    us = time_graph(call, reps, stream) * 1e3 / launches
    b = sum(gemm_bytes(M, N, K, True) for M in ROOFLINE_MS) / len(ROOFLINE_MS)
    return {"us": us, "bytes": b, "GBs": b / (us * 1e-6) / 1e9, "launches": launches}


def stream_ceiling(dev, stream, reps: int = 600):
    """The single-launch streaming floor for the roofline kernel's weight:
    the library's read-only probe reading the same rotated weight copies
    (N=4096, K=5120) with the same load pattern, one HIP graph of `reps`
    launches timed with HIP events on its launch stream."""
    N, K = 4096, 5120
    copies = weight_copies(N, K, dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def call(i):
        mx.hbm_read_probe(copies[i % len(copies)], sink)
    with torch.cuda.stream(stream):
        for i in range(20):
            call(i)
    us = time_graph(call, reps, stream) * 1e3 / reps
    b = mx_bytes(N, K)
    return {"us": us, "bytes": b, "GBs": b / (us * 1e-6) / 1e9}


def chain_case(dev, stream, M: int, reps: int = 200, norm: bool = False):
    """The three-projection chain (A 2048x5120, requantize 1536 columns, B
    8192x1536, C 5120x8192), weights rotated over copies; the library's
    default chain path unless MXG_CHAIN_PATH says otherwise.  norm: the
    1536 columns are RMS-normalised before the requantize (one more launch;
    the gain's 3 KB and the normalised BF16 are counted)."""
    case = synth.chain_case(M, seed=0)
    w = {k: mx.PackedWeight.from_bf16(case[k].to(dev)) for k in ("w_a", "w_b", "w_c")}
    per = sum(mx_bytes(v.N, v.K) for v in w.values())
    n = max(2, math.ceil(ROTATE_BYTES / per))
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

    def call(i):
        cw = cop[i % n]
        mx.mxfp8_proj_chain(*a, cw["w_a"], cw["w_b"], *c, cw["w_c"], outs=outs, workspace=ws,
                            norm_weight=gain, norm_eps=synth.RMSNORM_EPS)
    with torch.cuda.stream(stream):
        for i in range(10):
            call(i)
    us = time_graph(call, reps, stream) * 1e3 / reps
    b = per + mx_bytes(M, 5120) + mx_bytes(M, 8192) + 2 * M * (2048 + 8192 + 5120) \
        + 2 * M * 1536 + mx_bytes(M, 1536) + (2 * 1536 if norm else 0)
    return {"us": round(us, 3), "GBs": round(b / (us * 1e-6) / 1e9, 1),
            "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


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
    us = time_graph(call, reps, stream) * 1e3 / reps
    b = 2 * M * K + 2 * K + 2 * M * K + mx_bytes(M, K)
    return {"us": round(us, 3), "GBs": round(b / (us * 1e-6) / 1e9, 1)}


def extra_cases(dev, stream):
    """Latency of the other single-GEMM configurations (MXFP8 inputs)."""
    out = {}
    specs = [("single M4 N1024 K2048", [(4, 1024, 2048)], False)]
    for (N, K) in ((4096, 5120), (5120, 8192), (8192, 1536)):
        specs.append((f"wide N{N} K{K}", [(M, N, K) for M in (16, 32, 48)], True))
    for name, shapes, outliers in specs:
        N, K = shapes[0][1], shapes[0][2]
        copies = weight_copies(N, K, dev)
        for (M, _, _) in shapes:
            x = synth.gemm_case(M, 16, K, seed=0, outliers=outliers)["x"].to(dev)
            aq, as_ = mx.mxfp8_quantize(x)
            o = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

            def call(i):
                mx.mxfp8_gemm(aq, as_, copies[i % len(copies)], out=o)
            with torch.cuda.stream(stream):
                for i in range(20):
                    call(i)
            reps = 400
            us = time_graph(call, reps, stream) * 1e3 / reps
            b = gemm_bytes(M, N, K, False)
            out[f"M{M} N{N} K{K}"] = {"us": round(us, 3), "GBs": round(b / (us * 1e-6) / 1e9, 1),
                                     "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del copies
        torch.cuda.empty_cache()
    # more than 48 rows (64-row blocks, or 64 x 64 tiles above 128 rows)
    N, K = 4096, 5120
    copies = weight_copies(N, K, dev)
    for M in (64, 128, 256):
        x = synth.gemm_case(M, 16, K, seed=0)["x"].to(dev)
        aq, as_ = mx.mxfp8_quantize(x)
        o = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

        def call(i):
            mx.mxfp8_gemm(aq, as_, copies[i % len(copies)], out=o)
        with torch.cuda.stream(stream):
            for i in range(20):
                call(i)
        us = time_graph(call, 200, stream) * 1e3 / 200
        b = gemm_bytes(M, N, K, False)
        out[f"rows above 48: M{M} N{N} K{K}"] = {
            "us": round(us, 3), "GBs": round(b / (us * 1e-6) / 1e9, 1),
            "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(2 * M * N * K / (us * 1e-6) / 1e12, 1)}
    del copies
    torch.cuda.empty_cache()
    for M in (1, 8, 32):
        out[f"chain M{M}"] = chain_case(dev, stream, M)
    for M in (1, 8, 32):
        out[f"chain+norm M{M}"] = chain_case(dev, stream, M, norm=True)
    for M in (1, 8, 48):
        for K, ld in ((1536, 2048), (5120, 5120)):
            out[f"rmsnorm+quantize M{M} K{K}"] = rmsnorm_case(dev, stream, M, K, ld)
    for M in (1, 4, 16):
        out[f"wo_a+wo_b M{M}"] = wo_a_case(dev, stream, M)
    return out


def wo_a_case(dev, stream, M: int, reps: int = 200):
    """Rotary + grouped WO-A (8 groups of 8 heads x 512 dims, rank 1024) +
    MXFP8 of z + wo_b 5120x8192, weights rotated over copies."""
    case = synth.wo_a_case(M, seed=0)
    d = case["dims"]
    G, R = d["n_groups"], d["rank"]
    wa = mx.PackedWeight.from_bf16(case["w_a"].reshape(G * R, -1).to(dev))
    wb = mx.PackedWeight.from_bf16(case["w_b"].to(dev))
    per = mx_bytes(wa.N, wa.K) + mx_bytes(wb.N, wb.K)
    n = max(2, math.ceil(ROTATE_BYTES / per))
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
    us = time_graph(call, reps, stream) * 1e3 / reps
    H, D = d["n_heads"], d["head_dim"]
    b = per + 2 * M * H * D + 8 * M + 4 * M * (D - d["nope"]) + mx_bytes(M, G * R) + 2 * M * wb.N
    return {"us": round(us, 3), "GBs": round(b / (us * 1e-6) / 1e9, 1),
            "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def cpu_baseline(min_seconds: float = 10.0):
    """The oracle (plain C, fp64) on the same decode-bucket step: quantize each
    M-row batch and run the GEMM against the full weight; repeated until
    min_seconds have elapsed."""
    import oracle
    N, K, Ms = 4096, 5120, (1, 2, 4, 8)
    case = synth.gemm_case(8, N, K, seed=0)
    wq, ws = oracle.quantize(synth.bits(case["w"]))       # weight quantize: not timed
    xb = synth.bits(case["x"])
    threads = oracle.set_threads(len(os.sched_getaffinity(0)))
    reps, t0 = 0, time.perf_counter()
    while True:
        for M in Ms:
            q, s = oracle.quantize(xb[:M])
            oracle.gemm(q, s, wq, ws)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    step_bytes = sum(gemm_bytes(M, N, K, True) for M in Ms)
    return {"value": round(step_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} full decode-bucket steps (M=1,2,4,8; N=4096; K=5120) in {el:.1f} s, "
                      f"{el / reps:.3f} s/step"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cases", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the dominant kernel's timing (for profiler runs)")
    args = ap.parse_args()
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
    rec = decode_bucket(dev, args.steps, args.warmup, stream)
    roof = roofline_kernel(dev, stream)
    ceil = stream_ceiling(dev, stream)
    cases = {} if args.no_cases else extra_cases(dev, stream)
    cpu = None if args.no_cpu else cpu_baseline()
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
                   "weight_copies": rec["copies"], "timing": "HIP graph of K steps, HIP events"},
        "us_per_gemm": rec["per_m"],
        "roofline": {"bound": "hbm", "kernel": ROOFLINE_KERNEL,
                     "achieved": round(roof["GBs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(roof["GBs"] / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(roof["us"], 3),
                     "bytes_per_launch": int(roof["bytes"]),
                     "traffic": profiled_traffic()},
        "stream_ceiling": {"kernel": "hbm_read_kernel: the same weight copies read with the "
                                     "same load pattern, nothing else",
                           "us": round(ceil["us"], 3), "GBs": round(ceil["GBs"], 1),
                           "frac": round(ceil["GBs"] / HBM_PEAK_GBS, 4),
                           "roofline_vs_ceiling": round(roof["GBs"] / ceil["GBs"], 4)},
        "step_avg_launch_us": round(rec["kernel_us"], 3),
        "cases": cases,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
