"""GPU parity of mxfp8_proj_chain (three projections back to back)
against the oracle's chain, in the decode step's order: A on the MXFP8 layer input,
the leading columns of A's output requantized for B, C on its own input.

Unique results are compared with the oracle directly (A's and C's outputs,
every code from a BF16 input).  A's BF16 output is only determined to within
the GEMM tolerance, so the requantized codes are checked for validity (they
must be exactly the quantization of the GPU's own A output), and B's output
is compared end to end with the oracle on every row whose requantized codes
match the oracle's, and stage-wise on the others."""
import os

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_gemm_amd as mx
import oracle
import synth
from helpers import check_gemm, dev_bf16, host_bits, host_u8, say

pytestmark = pytest.mark.gpu

SMALL = {"A": (256, 512), "B": (384, 128), "C": (320, 640)}


@pytest.fixture(params=["direct"])
def chain_path(request, monkeypatch):
    """The chain's implementations (selected with MXG_CHAIN_PATH)."""
    monkeypatch.setenv("MXG_CHAIN_PATH", request.param)
    return request.param


def _prep(case, row_major=()):
    """GPU and oracle quantization of every input (must agree bit for bit);
    the weights named in row_major stay [N, K] / [N, K/32], the others are
    packed."""
    g, o = {}, {}
    for name in ("x_a", "x_c", "w_a", "w_b", "w_c"):
        bits = synth.bits(case[name])
        o[name] = oracle.quantize(bits)
        q, s = mx.mxfp8_quantize(dev_bf16(bits))
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(q), o[name][0]) and np.array_equal(host_u8(s), o[name][1]), name
        if name.startswith("x"):
            g[name] = (q, s)
        else:
            g[name] = mx.RowMajorWeight(q, s) if name in row_major else mx.PackedWeight.from_rows(q, s)
    return g, o


def run_chain(M, dims=None, seed=0, row_major=()):
    case = synth.chain_case(M, seed=seed, dims=dims)
    d = case["dims"]
    b_cols = d["B"][1]
    g, o = _prep(case, row_major)
    ref = oracle.chain(*o["x_a"], o["w_a"], b_cols, o["w_b"], *o["x_c"], o["w_c"])
    say(f"chain M={M} dims={d} seed={seed} row_major={row_major}")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    out_a, b_q, b_s, out_b, out_c = mx.mxfp8_proj_chain(*g["x_a"], g["w_a"], g["w_b"], *g["x_c"],
                                                         g["w_c"], workspace=ws)
    torch.cuda.synchronize()
    assert mx.workspace_error(ws) == 0
    assert not ws[:65536].any(), "counters must be back to zero"
    check_gemm(out_a, ref.A, "A")
    check_gemm(out_c, ref.C, "C")
    a_bits = host_bits(out_a)
    vq, vs = oracle.quantize(np.ascontiguousarray(a_bits[:, :b_cols]))
    gq, gs = host_u8(b_q), host_u8(b_s)
    assert np.array_equal(gq, vq) and np.array_equal(gs, vs), "requant must quantize A's output"
    same = np.all(gq == ref.b_q, axis=1) & np.all(gs == ref.b_s, axis=1)
    out_b_bits = host_bits(out_b)
    if same.any():
        got = oracle.bf16_value(out_b_bits[same])
        assert np.all(np.abs(got - ref.B.ref[same]) <= ref.B.tolerance()[same])
    stage = oracle.gemm(gq, gs, o["w_b"][0], o["w_b"][1])
    check_gemm(out_b, stage, "B (stage-wise)")
    frac = 1.0 - np.mean(gq == ref.b_q)
    assert frac < 0.02, f"{frac:.4f} of requantized codes differ from the end-to-end oracle"
    return g, (out_a, b_q, b_s, out_b, out_c), ws


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 48])
def test_chain_small(M, chain_path):
    run_chain(M, dims=SMALL, seed=M)


@pytest.mark.parametrize("plan", ["2,1", "4,1", "2,2", "4,4", "2,8"])
@pytest.mark.parametrize("M", [3, 17, 48])
def test_chain_plans(M, plan, chain_path, monkeypatch):
    # Every GEMM of the chain on the 2D kernel with a forced (tiles, K parts)
    # plan: A then writes B's MXFP8 input in its epilogue (one or several K
    # parts), which must be exactly the quantization of A's BF16 output.
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "2d")
    monkeypatch.setenv("MXG_PLAN", plan)
    run_chain(M, dims=SMALL, seed=M + 7 * len(plan))


@pytest.mark.parametrize("M", [1, 8, 32])
def test_chain_full_size(M, chain_path):
    run_chain(M)


@pytest.mark.parametrize("row_major", [("w_a", "w_b", "w_c"), ("w_b",), ("w_a", "w_c")])
@pytest.mark.parametrize("M,dims", [(1, None), (17, SMALL), (32, None), (48, SMALL)])
def test_chain_row_major_weights(M, dims, row_major):
    """Weights read as [N, K] / [N, K/32] (all, or some of them): within
    tolerance of the oracle as run_chain checks, and bit for bit the outputs
    of the same chain on packed weights."""
    g, outs, _ = run_chain(M, dims=dims, seed=M + 3, row_major=row_major)
    _, ref_outs, _ = run_chain(M, dims=dims, seed=M + 3)
    for name, a, b in zip(("out_a", "b_q", "b_s", "out_b", "out_c"), outs, ref_outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name


@pytest.mark.parametrize("M", [8, 32])
def test_chain_deterministic_and_equal_to_separate_calls(M, chain_path):
    g, outs, ws = run_chain(M)
    first = [t.clone() for t in outs]
    for _ in range(20):
        again = mx.mxfp8_proj_chain(*g["x_a"], g["w_a"], g["w_b"], *g["x_c"], g["w_c"], workspace=ws)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    # the same GEMMs issued one by one give the same bits
    out_a = mx.mxfp8_gemm(*g["x_a"], g["w_a"], workspace=ws)
    b_q, b_s = mx.mxfp8_quantize(out_a, K=g["w_b"].K)
    out_b = mx.mxfp8_gemm(b_q, b_s, g["w_b"], workspace=ws)
    out_c = mx.mxfp8_gemm(*g["x_c"], g["w_c"], workspace=ws)
    torch.cuda.synchronize()
    names = ("out_a", "b_q", "b_s", "out_b", "out_c")
    for name, a, b in zip(names, first, (out_a, b_q, b_s, out_b, out_c)):
        diff = (a.view(torch.uint8) != b.view(torch.uint8))
        if diff.any():
            idx = torch.nonzero(diff)[:8].tolist()
            say(f"{name}: {int(diff.sum())} bytes differ, first {idx}, "
                f"max |d| {(a.float() - b.float()).abs().max().item() if a.dtype == torch.bfloat16 else -1}")
        assert not diff.any(), name


def test_chain_rejects_bad_shapes():
    g, _ = _prep(synth.chain_case(2, dims=SMALL))
    bad = mx.PackedWeight(g["w_b"].q, g["w_b"].s, g["w_b"].N, 100)   # K not a multiple of 128
    with pytest.raises(ValueError):
        mx.mxfp8_proj_chain(*g["x_a"], g["w_a"], bad, *g["x_c"], g["w_c"],
                            outs=(torch.empty(2, 256, dtype=torch.bfloat16, device="cuda"),
                                  torch.empty(2, 100, dtype=torch.uint8, device="cuda"),
                                  torch.empty(2, 3, dtype=torch.uint8, device="cuda"),
                                  torch.empty(2, 384, dtype=torch.bfloat16, device="cuda"),
                                  torch.empty(2, 320, dtype=torch.bfloat16, device="cuda")))


def run_chain_norm(M, dims=None, seed=0):
    """The chain with the RMSNorm of A's leading columns before the
    requantize: every stage is checked on the GPU's own input to it, and B
    end to end on rows whose codes match the oracle's."""
    case = synth.chain_case(M, seed=seed, dims=dims)
    d = case["dims"]
    b_cols = d["B"][1]
    nc = synth.rmsnorm_case(1, b_cols, seed=seed + 1)
    w_bits, eps = synth.bits(nc["w"]), nc["eps"]
    g, o = _prep(case)
    ref = oracle.chain(*o["x_a"], o["w_a"], b_cols, o["w_b"], *o["x_c"], o["w_c"],
                       norm=(w_bits, eps))
    say(f"chain+norm M={M} dims={d} seed={seed}")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    b_bf16 = torch.empty(M, b_cols, dtype=torch.bfloat16, device="cuda")
    out_a, b_q, b_s, out_b, out_c = mx.mxfp8_proj_chain(
        *g["x_a"], g["w_a"], g["w_b"], *g["x_c"], g["w_c"], workspace=ws,
        norm_weight=dev_bf16(w_bits), norm_eps=eps, b_bf16=b_bf16)
    torch.cuda.synchronize()
    check_gemm(out_a, ref.A, "A")
    check_gemm(out_c, ref.C, "C")
    lead = np.ascontiguousarray(host_bits(out_a)[:, :b_cols])
    yref = oracle.rmsnorm(lead, w_bits, eps)
    yb = host_bits(b_bf16)
    assert np.all(np.abs(oracle.bf16_value(yb) - yref) <= oracle.rmsnorm_tolerance(yref, b_cols))
    vq, vs = oracle.quantize(yb)
    gq, gs = host_u8(b_q), host_u8(b_s)
    assert np.array_equal(gq, vq) and np.array_equal(gs, vs), "requant must quantize the norm"
    check_gemm(out_b, oracle.gemm(gq, gs, o["w_b"][0], o["w_b"][1]), "B (stage-wise)")
    same = np.all(gq == ref.b_q, axis=1) & np.all(gs == ref.b_s, axis=1)
    if same.any():
        got = oracle.bf16_value(host_bits(out_b)[same])
        assert np.all(np.abs(got - ref.B.ref[same]) <= ref.B.tolerance()[same])
    assert 1.0 - np.mean(gq == ref.b_q) < 0.02


@pytest.mark.parametrize("form", [None, "2d", "m16", "m16lds", "launch"])
@pytest.mark.parametrize("M", [1, 5, 9, 16, 17, 32, 48])
def test_chain_with_norm_small(M, form, chain_path, monkeypatch):
    # The norm inside B's staging on the 2D kernel (up to 32 rows) or on the
    # M <= 16 kernel (up to 16; per-wave rows, or m16lds: the block sums
    # through LDS), or as a launch of its own: routed, and each form forced
    # (MXG_NORM_KERNEL; a form that does not take the shape leaves it to the
    # next).
    if form:
        monkeypatch.setenv("MXG_NORM_KERNEL", form)
    run_chain_norm(M, dims=SMALL, seed=M)


@pytest.mark.parametrize("form", [None, "2d", "m16", "m16lds"])
@pytest.mark.parametrize("M", [1, 8, 16, 32])
def test_chain_with_norm_full_size(M, form, monkeypatch):
    if form:
        monkeypatch.setenv("MXG_NORM_KERNEL", form)
    run_chain_norm(M)


# B's K above 2048 (more than 64 blocks a row): the M <= 16 kernel's norm
# takes its LDS form (lanes add several blocks each).
WIDE_B = {"A": (2560, 256), "B": (256, 2560), "C": (128, 256)}


@pytest.mark.parametrize("form", [None, "m16"])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_chain_with_norm_wide_k(M, form, monkeypatch):
    if form:
        monkeypatch.setenv("MXG_NORM_KERNEL", form)
    run_chain_norm(M, dims=WIDE_B, seed=100 + M)


# B's K at the per-wave forms' limit (64 blocks a row: every lane of a wave
# holds a block) and one step above it (the M <= 16 kernel's LDS form; the
# 2D form does not take it and leaves it to the next).
@pytest.mark.parametrize("bk", [2048, 2176])
@pytest.mark.parametrize("form", [None, "m16", "m16lds", "2d"])
@pytest.mark.parametrize("M", [1, 8, 16])
def test_chain_with_norm_k_boundary(M, form, bk, monkeypatch):
    if form:
        monkeypatch.setenv("MXG_NORM_KERNEL", form)
    run_chain_norm(M, dims={"A": (bk, 256), "B": (256, bk), "C": (128, 256)}, seed=200 + M)


@pytest.mark.parametrize("M", [1, 3, 8, 12, 16])
def test_chain_norm_forms_bitwise(M, monkeypatch):
    # The M <= 16 kernel's two norm forms add the same terms in the same
    # order: the normalised row, its codes and B's output agree bit for bit.
    case = synth.chain_case(M, seed=7)
    nc = synth.rmsnorm_case(1, case["dims"]["B"][1], seed=8)
    g, _ = _prep(case)
    got = {}
    for form in ("m16", "m16lds"):
        monkeypatch.setenv("MXG_NORM_KERNEL", form)
        say(f"chain+norm M={M} form={form}")
        ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
        y = torch.empty(M, case["dims"]["B"][1], dtype=torch.bfloat16, device="cuda")
        outs = mx.mxfp8_proj_chain(*g["x_a"], g["w_a"], g["w_b"], *g["x_c"], g["w_c"], workspace=ws,
                                   norm_weight=dev_bf16(synth.bits(nc["w"])), norm_eps=nc["eps"],
                                   b_bf16=y)
        torch.cuda.synchronize()
        got[form] = [host_bits(y)] + [host_u8(t) if t.dtype == torch.uint8 else host_bits(t)
                                      for t in outs]
    for a, b in zip(got["m16"], got["m16lds"]):
        assert np.array_equal(a, b)
