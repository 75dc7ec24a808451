"""GPU parity of wo_a_fused_quantize (rotary + grouped WO-A + MXFP8 of z,
optionally wo_b) against the oracle's wo_a.

Unique results are compared bit for bit: the MXFP8 codes of the rotated input
(left in the workspace), and the MXFP8 of z computed from the GPU's own BF16 z
(z itself is only determined to within the GEMM tolerance).  z is compared
with the oracle's grouped projection within tolerance, wo_b's output
stage-wise (oracle GEMM on the GPU's z codes) and end to end on every row
whose z codes match the oracle's."""
import os

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_gemm_amd as mx
import oracle
import synth
from helpers import check_gemm, dev_bf16, dev_u8, host_bits, host_u8, say

pytestmark = pytest.mark.gpu

# Reduced dims (same structure: 448 + 64 head dims, 8 heads per group).
SMALL = dict(n_heads=16, head_dim=512, nope=448, n_groups=2, rank=256, n_out=384)


@pytest.fixture(params=["direct"], autouse=True)
def woa_path(request, monkeypatch):
    """Every test runs on each WO-A implementation (MXG_WOA_PATH)."""
    monkeypatch.setenv("MXG_WOA_PATH", request.param)
    return request.param


def _weights(case):
    """Oracle MXFP8 of W_a (per group) and W_b, and the packed device copies."""
    d = case["dims"]
    G, R = d["n_groups"], d["rank"]
    wa_bits = synth.bits(case["w_a"]).reshape(G * R, -1)
    wa_q, wa_s = oracle.quantize(wa_bits)
    wb_q, wb_s = oracle.quantize(synth.bits(case["w_b"]))
    wa = mx.PackedWeight.from_rows(dev_u8(wa_q), dev_u8(wa_s))
    wb = mx.PackedWeight.from_rows(dev_u8(wb_q), dev_u8(wb_s))
    return (wa_q.reshape(G, R, -1), wa_s.reshape(G, R, -1), (wb_q, wb_s)), (wa, wb)


_FULL = {}


def full_case():
    """The 64-head, 8-group, rank-1024, wo_b 5120 x 8192 case with 16 rows;
    the 1- and 4-row cases take its leading rows (one weight quantization)."""
    if not _FULL:
        case = synth.wo_a_case(16)
        _FULL["case"] = case
        _FULL["w"] = _weights(case)
    return _FULL["case"], _FULL["w"]


def run_wo_a(case, w, M, *, with_wb=True, keep_z=True, positions=None, o_dev=None):
    d = case["dims"]
    H, D, G, R, nope = d["n_heads"], d["head_dim"], d["n_groups"], d["rank"], d["nope"]
    (wa_q, wa_s, wb_o), (wa, wb) = w
    o_bits = synth.bits(case["o"])[:M]
    pos = (case["positions"][:M] if positions is None else positions).clone()
    ref = oracle.wo_a(o_bits, pos.numpy(), case["cos_sin"], wa_q, wa_s,
                      wb_o if with_wb else None, nope=nope, n_groups=G)
    say(f"wo_a M={M} H={H} D={D} G={G} R={R} wb={with_wb} keep_z={keep_z} "
        f"path={os.environ.get('MXG_WOA_PATH')}")
    o = dev_bf16(o_bits) if o_dev is None else o_dev
    ws = torch.zeros(32 << 20, dtype=torch.uint8, device="cuda")
    z, z_q, z_s, out = mx.wo_a_fused_quantize(
        o, pos.cuda(), torch.from_numpy(case["cos_sin"]).cuda(), wa, n_groups=G, nope_dim=nope,
        wb=wb if with_wb else None, keep_z=keep_z, workspace=ws)
    torch.cuda.synchronize()
    assert mx.workspace_error(ws) == 0
    # rotary + MXFP8 of every group: unique, bit-exact
    xq, xs = mx.wo_a_rotary_codes(ws, M, H * D)
    assert np.array_equal(host_u8(xq), np.concatenate(ref.xg_q, axis=1)), "rotary codes"
    assert np.array_equal(host_u8(xs), np.concatenate(ref.xg_s, axis=1)), "rotary scales"
    # grouped projection within tolerance, group by group
    if keep_z:
        for g in range(G):
            check_gemm(z[:, g * R:(g + 1) * R], ref.groups[g], f"z group {g}")
        zb = host_bits(z)
        vq, vs = oracle.quantize(zb)
        assert np.array_equal(host_u8(z_q), vq) and np.array_equal(host_u8(z_s), vs), \
            "z codes must be the MXFP8 of the GPU's z"
    gq, gs = host_u8(z_q), host_u8(z_s)
    frac = 1.0 - np.mean(gq == ref.z_q)
    assert frac < 0.02, f"{frac:.4f} of z codes differ from the end-to-end oracle"
    if with_wb:
        check_gemm(out, oracle.gemm(gq, gs, *wb_o), "wo_b (stage-wise)")
        same = np.all(gq == ref.z_q, axis=1) & np.all(gs == ref.z_s, axis=1)
        if same.any():
            got = oracle.bf16_value(host_bits(out)[same])
            assert np.all(np.abs(got - ref.out.ref[same]) <= ref.out.tolerance()[same])
    return (z, z_q, z_s, out), ws


@pytest.mark.parametrize("M", [1, 3, 16, 17, 33, 48])
def test_wo_a_small(M):
    case = synth.wo_a_case(M, seed=M, dims=SMALL)
    run_wo_a(case, _weights(case), M)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_wo_a_full_size(M):
    case, w = full_case()
    run_wo_a(case, w, M)


def _row_major(w):
    """The same weights as [N, K] codes and [N, K/32] scales (no repack)."""
    (wa_q, wa_s, (wb_q, wb_s)), _ = w
    GR = wa_q.shape[0] * wa_q.shape[1]
    wa = mx.RowMajorWeight(dev_u8(np.ascontiguousarray(wa_q.reshape(GR, -1))),
                           dev_u8(np.ascontiguousarray(wa_s.reshape(GR, -1))))
    return w[0], (wa, mx.RowMajorWeight(dev_u8(wb_q), dev_u8(wb_s)))


@pytest.mark.parametrize("M,full", [(3, False), (17, False), (4, True)])
def test_wo_a_row_major_weights(M, full):
    """W_a and W_b read as [N, K] / [N, K/32]: within tolerance of the oracle
    as run_wo_a checks, and bit for bit the outputs on packed weights."""
    if full:
        case, w = full_case()
    else:
        case = synth.wo_a_case(M, seed=M + 9, dims=SMALL)
        w = _weights(case)
    got, _ = run_wo_a(case, _row_major(w), M)
    ref, _ = run_wo_a(case, w, M)
    for name, a, b in zip(("z", "z_q", "z_s", "out"), got, ref):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name


def test_wo_a_without_wo_b_and_without_z():
    case = synth.wo_a_case(5, seed=7, dims=SMALL)
    run_wo_a(case, _weights(case), 5, with_wb=False, keep_z=False)


def test_wo_a_position_zero_is_a_plain_grouped_gemm():
    # Rotation by angle 0 is the identity: the rotary codes are the MXFP8 of o.
    M = 4
    case = synth.wo_a_case(M, seed=11, dims=SMALL)
    d = case["dims"]
    _, ws = run_wo_a(case, _weights(case), M, positions=torch.zeros(M, dtype=torch.int64))
    HD = d["n_heads"] * d["head_dim"]
    q, s = oracle.quantize(synth.bits(case["o"]).reshape(M, HD))
    xq, xs = mx.wo_a_rotary_codes(ws, M, HD)
    assert np.array_equal(host_u8(xq), q) and np.array_equal(host_u8(xs), s)


def test_wo_a_strided_heads_view():
    # o as the first H heads of a wider attention output (row stride > H*D).
    M = 6
    case = synth.wo_a_case(M, seed=5, dims=SMALL)
    d = case["dims"]
    H, D = d["n_heads"], d["head_dim"]
    wide = torch.zeros(M, H + 3, D, dtype=torch.bfloat16)
    wide[:, :H] = case["o"]
    view = wide.cuda()[:, :H, :]
    assert view.stride(0) == (H + 3) * D
    run_wo_a(case, _weights(case), M, o_dev=view)


def test_wo_a_full_size_deterministic():
    case, w = full_case()
    first, ws = run_wo_a(case, w, 16)
    d = case["dims"]
    for _ in range(10):
        again = mx.wo_a_fused_quantize(
            dev_bf16(synth.bits(case["o"])), case["positions"].cuda(),
            torch.from_numpy(case["cos_sin"]).cuda(), w[1][0], n_groups=d["n_groups"],
            nope_dim=d["nope"], wb=w[1][1], workspace=ws)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_wo_a_position_out_of_range_sets_the_error_word():
    M = 2
    case = synth.wo_a_case(M, seed=3, dims=SMALL)
    d = case["dims"]
    _, (wa, wb) = _weights(case)
    max_pos = case["cos_sin"].shape[0]
    pos = torch.tensor([5, max_pos], dtype=torch.int64, device="cuda")
    ws = torch.zeros(32 << 20, dtype=torch.uint8, device="cuda")
    say("wo_a position out of range")
    mx.wo_a_fused_quantize(dev_bf16(synth.bits(case["o"])), pos,
                           torch.from_numpy(case["cos_sin"]).cuda(), wa, n_groups=d["n_groups"],
                           nope_dim=d["nope"], wb=wb, workspace=ws)
    torch.cuda.synchronize()
    assert mx.workspace_error(ws) & 2


def test_wo_a_then_gemm_share_a_workspace():
    # WO-A leaves its rotated input where a K-split GEMM keeps its partial
    # sums, and its counters at zero: a K-split GEMM that follows on the same
    # workspace gives the same bits as on a fresh one.
    case, w = full_case()
    _, ws = run_wo_a(case, w, 16)
    assert not ws[:65536].any(), "counters must be back to zero"
    M, N, K = 48, 4096, 5120
    g = synth.gemm_case(M, N, K, seed=21)
    wq, wsc = oracle.quantize(synth.bits(g["w"]))
    pw = mx.PackedWeight.from_rows(dev_u8(wq), dev_u8(wsc))
    aq, asc = oracle.quantize(synth.bits(g["x"]))
    say(f"gemm M={M} N={N} K={K} after wo_a on one workspace")
    shared = mx.mxfp8_gemm(dev_u8(aq), dev_u8(asc), pw, workspace=ws)
    fresh = mx.mxfp8_gemm(dev_u8(aq), dev_u8(asc), pw,
                          workspace=torch.zeros_like(ws))
    torch.cuda.synchronize()
    assert torch.equal(shared.view(torch.int16), fresh.view(torch.int16))
    assert mx.workspace_error(ws) == 0
