"""GPU parity of mxfp8_gemm against the oracle.

Both sides start from the same seeded BF16 tensors (synth.py) and quantize
them on their own; the codes must agree bit for bit, and every BF16 output
element must lie within 2^-7 * sum|a_k w_k| + 1e-6 of the oracle's fp64 sum.
Sizes span several workgroups, ragged row counts (every activation-tile
bucket and its edges) and the benchmark's full shapes."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_gemm_amd as mx
import oracle
import synth
from helpers import check_gemm, dev_bf16, dev_u8, host_bits, host_u8, say

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["direct", "direct-m16", "direct-2d", "direct-2d-wl"])
def path(request, monkeypatch):
    """Run a test through the direct kernels: as routed, and with the M <= 16
    kernel, the 2D kernel (staged) or the 2D kernel's wave-local form forced
    wherever it applies."""
    kind, _, kernel = request.param.partition("-")
    monkeypatch.delenv("MXG_DIRECT_KERNEL", raising=False)
    monkeypatch.delenv("MXG_WAVE_LOCAL", raising=False)
    if kernel == "2d-wl":
        monkeypatch.setenv("MXG_DIRECT_KERNEL", "2d")
        monkeypatch.setenv("MXG_WAVE_LOCAL", "1")
    elif kernel:
        monkeypatch.setenv("MXG_DIRECT_KERNEL", kernel)
        if kernel == "2d":
            monkeypatch.setenv("MXG_WAVE_LOCAL", "0")
    return request.param

_wcache = {}


def _weights(N, K, seed):
    """Weight codes from the GPU quantizer and from the oracle (must agree)."""
    key = (N, K, seed)
    if key not in _wcache:
        w_bits = synth.bits(synth.gemm_case(1, N, K, seed=seed)["w"])
        ow = oracle.quantize(w_bits)
        gq, gs = mx.mxfp8_quantize(dev_bf16(w_bits))
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(gq), ow[0]) and np.array_equal(host_u8(gs), ow[1])
        _wcache.clear()
        _wcache[key] = (mx.PackedWeight.from_rows(gq, gs), ow)
    return _wcache[key]


def run_case(M, N, K, seed=0, outliers=False, fused=False, row_major=False):
    """One GEMM against the oracle; row_major: the weight as [N, K] codes and
    [N, K/32] scales, read without a repack."""
    case = synth.gemm_case(M, N, K, seed=seed, outliers=outliers)
    x_bits = synth.bits(case["x"])
    w_bits = synth.bits(case["w"])
    ow_q, ow_s = oracle.quantize(w_bits)
    oa_q, oa_s = oracle.quantize(x_bits)
    ref = oracle.gemm(oa_q, oa_s, ow_q, ow_s)
    say(f"gemm M={M} N={N} K={K} seed={seed} outliers={outliers} fused={fused} "
        f"row_major={row_major}")
    w_q, w_s = mx.mxfp8_quantize(dev_bf16(w_bits))
    w = mx.RowMajorWeight(w_q, w_s) if row_major else mx.PackedWeight.from_rows(w_q, w_s)
    x = dev_bf16(x_bits)
    if fused:
        a_q = torch.full((M, K), 0x55, dtype=torch.uint8, device="cuda")
        a_s = torch.full((M, K // 32), 0x55, dtype=torch.uint8, device="cuda")
        out = mx.mxfp8_gemm(a_q, a_s, w, x=x)
    else:
        a_q, a_s = mx.mxfp8_quantize(x)
        out = mx.mxfp8_gemm(a_q, a_s, w)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(w_q), ow_q) and np.array_equal(host_u8(w_s), ow_s)
    assert np.array_equal(host_u8(a_q), oa_q) and np.array_equal(host_u8(a_s), oa_s)
    return check_gemm(out, ref, f"M={M} N={N} K={K}")


# small shapes: several workgroups, every row bucket and its edges
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 15, 16, 17, 31, 32, 33, 47, 48])
@pytest.mark.parametrize("fused", [False, True])
def test_rows_sweep(M, fused, path):
    run_case(M, 256, 1024, seed=M, fused=fused)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (1024, 128), (128, 8192), (2064, 1664)])
@pytest.mark.parametrize("fused", [False, True])
def test_shapes(N, K, fused, path):
    for M in (1, 20, 48):
        run_case(M, N, K, seed=N + K, fused=fused)


# BF16 input over short K with at least two weight tiles per CU: the 2D
# kernel with two (N 8192) or four (N 16384) tiles per workgroup and no K
# split; the M <= 16 kernel forced for comparison.
@pytest.mark.parametrize("N,K", [(8192, 1536), (16384, 1536), (8192, 512)])
@pytest.mark.parametrize("kernel", [None, "m16"])
def test_bf16_short_k_many_tiles(N, K, kernel, monkeypatch):
    if kernel:
        monkeypatch.setenv("MXG_DIRECT_KERNEL", kernel)
    for M in (1, 7, 16):
        run_case(M, N, K, seed=N + K + M, fused=True)


# MXFP8 input on two tiles per CU where the M <= 16 kernel holds one
# workgroup per CU (16 rows of K 4096): the 2D kernel, one tile per
# workgroup; 12 rows stay on the M <= 16 kernel; both forced for comparison.
@pytest.mark.parametrize("kernel", [None, "m16", "2d"])
def test_two_tiles_per_cu_mxfp8(kernel, monkeypatch):
    if kernel:
        monkeypatch.setenv("MXG_DIRECT_KERNEL", kernel)
    for M in (12, 16):
        run_case(M, 8192, 4096, seed=M + 77, fused=False)


@pytest.mark.parametrize("M", [1, 16, 17, 48])
@pytest.mark.parametrize("fused", [False, True])
def test_largest_contraction(M, fused, path):
    # K = MXG_MAX_K: the longest activation rows (LDS chunking, K split)
    run_case(M, 512, 16384, seed=M, fused=fused)


def test_m4_n1024_k2048(path):
    # M=4, N=1024, K=2048, x ~ N(0,1), W ~ N(0,0.02), seed 0
    run_case(4, 1024, 2048, seed=0)
    run_case(4, 1024, 2048, seed=0, fused=True)


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_decode_bucket_full_size(M, path):
    # N=4096, K=5120 with the activation quantize fused into the GEMM launch
    run_case(M, 4096, 5120, seed=0, fused=True)


@pytest.mark.parametrize("N,K", [(4096, 5120), (5120, 8192), (8192, 1536)])
@pytest.mark.parametrize("M", [16, 32, 48])
def test_wide_tiles_full_size_outliers(M, N, K, path):
    run_case(M, N, K, seed=0, outliers=True)


@pytest.mark.parametrize("M,N,K,fused", [
    (1, 5120, 8192, False), (4, 5120, 8192, True), (5, 5120, 8192, True), (8, 5120, 8192, False),
    (3, 4112, 1024, False),    # one leftover tile: two workgroups take half of it
    (16, 6144, 2048, False),   # every workgroup takes half a leftover tile
    (13, 6144, 2048, True),
    (7, 4352, 4096, False),
])
def test_half_tile_plan(M, N, K, fused, monkeypatch):
    """Weights of G < tiles <= 1.5 G tiles (G = 256 CUs): one tile per
    workgroup plus half a leftover tile for some.  Within tolerance of the
    oracle, and bitwise equal to the one-tile-per-workgroup kernel with 16
    waves, which gives every wave the same steps and sums them in the same
    order."""
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "m16h")
    run_case(M, N, K, seed=N + M, fused=fused)
    case = synth.gemm_case(M, N, K, seed=N + M)
    w, _ = _weights(N, K, 1)
    x = case["x"].cuda()
    aq = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    as_ = torch.empty(M, K // 32, dtype=torch.uint8, device="cuda")
    a_q, a_s = mx.mxfp8_quantize(x)
    half = mx.mxfp8_gemm(aq, as_, w, x=x) if fused else mx.mxfp8_gemm(a_q, a_s, w)
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "m16")
    monkeypatch.setenv("MXG_M16_WAVES", "16")
    monkeypatch.setenv("MXG_M16_RSPLIT", "1")
    one = mx.mxfp8_gemm(a_q, a_s, w)
    torch.cuda.synchronize()
    assert torch.equal(half.view(torch.int16), one.view(torch.int16))


def _force(monkeypatch, kernel):
    monkeypatch.delenv("MXG_DIRECT_KERNEL", raising=False)
    monkeypatch.delenv("MXG_BIG_KERNEL", raising=False)
    if kernel and kernel.startswith("big:"):
        monkeypatch.setenv("MXG_BIG_KERNEL", kernel[4:])
    elif kernel:
        monkeypatch.setenv("MXG_DIRECT_KERNEL", kernel)


# Every kernel form: as routed, and the M <= 16 kernel, the 2D kernel, the
# tile + half-tile form, and above 64 rows the wide and the 64 x 64 forms,
# forced where they apply (N 5120 gives G < tiles <= 1.5 G on 256 CUs);
# M = 130 runs the forms for more than 48 rows (routed: the 64 x 64 form at
# K 1024, the wide form at K 4096).
KERNEL_FORMS = [None, "m16", "2d", "m16h", "big:wide", "big:64"]
BITWISE_SHAPES = [(9, 256, 1024), (9, 5120, 1024), (130, 256, 1024), (130, 256, 4096)]


@pytest.mark.parametrize("kernel", KERNEL_FORMS)
@pytest.mark.parametrize("M,N,K", BITWISE_SHAPES)
def test_one_hot_weights_bitwise(M, N, K, kernel, monkeypatch):
    """W has one 1.0 per row (code 0x38) in a block whose scale varies per
    row (2^-3 .. 2^3); the other blocks' scales vary too but multiply zeros.
    Each output is then one activation value times powers of two, exact in
    BF16, so every kernel must match the oracle bit for bit."""
    _force(monkeypatch, kernel)
    rng = np.random.default_rng(M + N)
    x_bits = oracle.bf16_round(rng.standard_normal((M, K)))
    oa_q, oa_s = oracle.quantize(x_bits)
    kn = rng.integers(0, K, N)
    wq = np.zeros((N, K), np.uint8); wq[np.arange(N), kn] = 0x38
    ws = rng.integers(124, 131, (N, K // 32)).astype(np.uint8)
    ref = oracle.gemm(oa_q, oa_s, wq, ws)
    say(f"gemm one-hot M={M} N={N} K={K} kernel={kernel}")
    out = mx.mxfp8_gemm(dev_u8(oa_q), dev_u8(oa_s), mx.PackedWeight.from_rows(dev_u8(wq), dev_u8(ws)))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), ref.bf16)


@pytest.mark.parametrize("kernel", KERNEL_FORMS)
@pytest.mark.parametrize("M,N,K", [(6, 512, 2048), (6, 5120, 1024), (130, 512, 1024),
                                   (130, 512, 4096)])
def test_weight_scale_plus_one_doubles_output_bitwise(M, N, K, kernel, monkeypatch):
    """Raising every weight scale byte by one doubles every output exactly,
    whatever the kernel's summation order (the sums scale by a power of two)."""
    _force(monkeypatch, kernel)
    case = synth.gemm_case(M, N, K, seed=3)
    say(f"gemm scale+1 metamorphic M={M} N={N} K={K} kernel={kernel}")
    a_q, a_s = mx.mxfp8_quantize(case["x"].cuda())
    w_q, w_s = mx.mxfp8_quantize(case["w"].cuda())
    out1 = mx.mxfp8_gemm(a_q, a_s, mx.PackedWeight.from_rows(w_q, w_s))
    out2 = mx.mxfp8_gemm(a_q, a_s, mx.PackedWeight.from_rows(w_q, w_s + 1))
    torch.cuda.synchronize()
    assert torch.equal(out2.float(), out1.float() * 2)


@pytest.mark.parametrize("form", ["wide", "64"])
def test_rows_above_64_deterministic(form, monkeypatch):
    """Both forms above 64 rows sum in a fixed order (wave order through LDS,
    no cross-workgroup sum): repeated calls give the same bits."""
    monkeypatch.setenv("MXG_BIG_KERNEL", form)
    M, N, K = 200, 4096, 5120
    w, _ = _weights(N, K, 0)
    a_q, a_s = mx.mxfp8_quantize(synth.gemm_case(M, 16, K, seed=4)["x"].cuda())
    say(f"gemm repeats M={M} N={N} K={K} form={form}")
    first = mx.mxfp8_gemm(a_q, a_s, w)
    for _ in range(10):
        again = mx.mxfp8_gemm(a_q, a_s, w)
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_zero_activations_give_positive_zero():
    M, N, K = 3, 256, 512
    w, _ = _weights(N, K, 0)
    say("gemm zero input")
    out = mx.mxfp8_gemm(torch.zeros(M, K, dtype=torch.uint8, device="cuda"),
                        torch.zeros(M, K // 32, dtype=torch.uint8, device="cuda"), w)
    torch.cuda.synchronize()
    assert (out.view(torch.int16) == 0).all()


def test_deterministic_repeats(path):
    M, N, K = 8, 4096, 5120
    w, _ = _weights(N, K, 0)
    x = synth.gemm_case(M, 16, K, seed=1)["x"].cuda()
    a_q = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    a_s = torch.empty(M, K // 32, dtype=torch.uint8, device="cuda")
    say("gemm determinism x100")
    first = mx.mxfp8_gemm(a_q, a_s, w, x=x).clone()
    for _ in range(100):
        out = mx.mxfp8_gemm(a_q, a_s, w, x=x)
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    torch.cuda.synchronize()


def test_rejected_call_writes_nothing():
    M, N, K = 4, 256, 512
    w, _ = _weights(N, K, 0)
    w_q, w_s = w.q, w.s
    a_q = torch.zeros(M, K, dtype=torch.uint8, device="cuda")
    a_s = torch.zeros(M, K // 32, dtype=torch.uint8, device="cuda")
    out = torch.full((M, N), 0x1234, dtype=torch.int16, device="cuda")
    say("gemm rejected call")
    L = mx.lib()
    for m, k in ((0, K), (257, K), (M, 500)):
        st = L.mxfp8_gemm(m, N, k, None, 0, a_q.data_ptr(), a_s.data_ptr(), w_q.data_ptr(),
                          w_s.data_ptr(), out.data_ptr(), None, 0, None)
        assert st == 3
    st = L.mxfp8_gemm(M, N, K, None, 0, a_q.data_ptr() + 8, a_s.data_ptr(), w_q.data_ptr(),
                      w_s.data_ptr(), out.data_ptr(), None, 0, None)
    assert st == 2
    torch.cuda.synchronize()
    assert (out == 0x1234).all()


def _pack_reference(wq: np.ndarray, ws: np.ndarray) -> tuple:
    """The packed order written out from its definition in include/mxgemm.h."""
    N, K = wq.shape
    S = K // 128
    pq = np.empty(N * K, np.uint8)
    ps = np.empty(N * K // 32, np.uint8)
    for t in range(N // 16):
        for s_ in range(S):
            for h in range(2):
                for l in range(64):
                    off = ((t * S + s_) * 2 + h) * 1024 + 16 * l
                    col = 128 * s_ + 64 * h + 16 * (l // 16)
                    pq[off:off + 16] = wq[16 * t + l % 16, col:col + 16]
            for l in range(64):
                ps[(t * S + s_) * 64 + l] = ws[16 * t + l % 16, 4 * s_ + l // 16]
    return pq, ps


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (64, 1024)])
def test_pack_is_the_documented_permutation(N, K):
    rng = np.random.default_rng(N + K)
    wq = rng.integers(0, 256, (N, K)).astype(np.uint8)
    ws = rng.integers(0, 256, (N, K // 32)).astype(np.uint8)
    say(f"pack N={N} K={K}")
    pq, ps = mx.mxfp8_pack_weights(dev_u8(wq), dev_u8(ws))
    torch.cuda.synchronize()
    rq, rs = _pack_reference(wq, ws)
    assert np.array_equal(host_u8(pq), rq) and np.array_equal(host_u8(ps), rs)


@pytest.mark.parametrize("M,N,K", [(8, 4096, 5120), (4, 5120, 8192), (33, 2048, 5120)])
def test_workspace_left_clean(M, N, K, monkeypatch):
    """Repeated calls (K-split tiles) on one workspace keep working: every
    counter is reset by the call that used it (a stale tile counter would
    make the next call's last-arrival test wrong), and the results stay
    bitwise identical."""
    monkeypatch.delenv("MXG_DIRECT_KERNEL", raising=False)
    w, _ = _weights(N, K, 0)
    ws = torch.zeros(int(mx.lib().mxg_gemm_workspace_bytes(M, N, K)) + 4096, dtype=torch.uint8,
                     device="cuda")
    x = synth.gemm_case(M, 16, K, seed=2)["x"].cuda()
    a_q = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    a_s = torch.empty(M, K // 32, dtype=torch.uint8, device="cuda")
    say(f"workspace hygiene M={M} N={N} K={K}")
    first = mx.mxfp8_gemm(a_q, a_s, w, x=x, workspace=ws).clone()
    for _ in range(3):
        o1 = mx.mxfp8_gemm(a_q, a_s, w, x=x, workspace=ws)
        assert torch.equal(o1.view(torch.int16), first.view(torch.int16))
        o2 = mx.mxfp8_gemm(a_q, a_s, w, workspace=ws)
        assert torch.equal(o2.view(torch.int16), first.view(torch.int16))
    torch.cuda.synchronize()
    assert mx.workspace_error(ws) == 0
    assert not ws[:65536].any(), "counters must be back to zero"



@pytest.mark.parametrize("M", [1, 5, 17])
def test_widest_output(M, path):
    # 2048 weight tiles: several rounds of workgroups over the CUs
    run_case(M, 32768, 1024, seed=M)


@pytest.mark.parametrize("M", [3, 16, 40])
def test_strided_bf16_input(M, path):
    # x as the leading K columns of a wider BF16 matrix (row stride > K), as
    # the chain's requantize reads A's output; quantized in whichever kernel
    # serves the shape.
    N, K, ld = 512, 1024, 1024 + 96
    case = synth.gemm_case(M, N, K, seed=M + 1)
    x_bits = synth.bits(case["x"])
    ow_q, ow_s = oracle.quantize(synth.bits(case["w"]))
    oa_q, oa_s = oracle.quantize(x_bits)
    ref = oracle.gemm(oa_q, oa_s, ow_q, ow_s)
    say(f"gemm strided bf16 input M={M} ld={ld}")
    wide = torch.zeros(M, ld, dtype=torch.bfloat16)
    wide[:, :K] = case["x"]
    x = wide.cuda()[:, :K]
    w = mx.PackedWeight.from_rows(dev_u8(ow_q), dev_u8(ow_s))
    a_q = torch.full((M, K), 0x55, dtype=torch.uint8, device="cuda")
    a_s = torch.full((M, K // 32), 0x55, dtype=torch.uint8, device="cuda")
    out = mx.mxfp8_gemm(a_q, a_s, w, x=x)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(a_q), oa_q) and np.array_equal(host_u8(a_s), oa_s)
    check_gemm(out, ref, f"strided M={M}")


@pytest.mark.parametrize("N,K", [(2048, 5120), (8192, 1536), (1024, 4096), (5120, 8192), (256, 128)])
@pytest.mark.parametrize("waves", ["routed", "16"])
def test_one_row_both_wave_counts(N, K, waves, monkeypatch):
    # One MXFP8 row: the M <= 16 kernel runs with 4 waves per workgroup
    # (up to 16 weight steps per wave) except at K = 5120; forcing 16 waves
    # covers the other split on the same shapes.
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "m16")
    if waves == "16":
        monkeypatch.setenv("MXG_M16_WAVES", "16")
    else:
        monkeypatch.delenv("MXG_M16_WAVES", raising=False)
    run_case(1, N, K, seed=K + 7)


@pytest.mark.parametrize("M,N,K", [(1, 256, 1024), (5, 512, 2048), (16, 256, 1024),
                                   (17, 2064, 1664), (33, 512, 16384), (48, 4096, 5120),
                                   (8, 5120, 8192)])
@pytest.mark.parametrize("kernel", ["routed", "m16", "2d"])
def test_scales_in_128x4_tiles(M, N, K, kernel, monkeypatch):
    """Activation scales in 128 x 4 tiles (the oracle's permutation of the
    row-major scales) give the row-major call's output bit for bit, on each
    direct kernel, and stay within tolerance of the oracle."""
    if kernel == "routed":
        monkeypatch.delenv("MXG_DIRECT_KERNEL", raising=False)
    else:
        monkeypatch.setenv("MXG_DIRECT_KERNEL", kernel)
    case = synth.gemm_case(M, N, K, seed=M + N)
    oa_q, oa_s = oracle.quantize(synth.bits(case["x"]))
    ow_q, ow_s = oracle.quantize(synth.bits(case["w"]))
    ref = oracle.gemm(oa_q, oa_s, ow_q, ow_s)
    say(f"gemm 128x4 scales M={M} N={N} K={K} kernel={kernel}")
    w = mx.PackedWeight.from_rows(dev_u8(ow_q), dev_u8(ow_s))
    a_q = dev_u8(oa_q)
    row = mx.mxfp8_gemm(a_q, dev_u8(oa_s), w)
    tiled = mx.mxfp8_gemm_ex(a_q, dev_u8(oracle.scales_to_128x4(oa_s)), w, mx.SCALES_128X4)
    torch.cuda.synchronize()
    assert torch.equal(row.view(torch.int16), tiled.view(torch.int16))
    check_gemm(tiled, ref, f"128x4 M={M}")


@pytest.mark.parametrize("M", [1, 8, 48])
def test_rmsnorm_128x4_output_feeds_the_gemm(M):
    """Producer to consumer with no repack: mxfp8_rmsnorm_quantize writes
    128 x 4 scales, mxfp8_gemm_ex reads them; equal bit for bit to the
    row-major pair, and within tolerance of the oracle on the same codes."""
    K, N = 1536, 8192
    nc = synth.rmsnorm_case(M, K, seed=M)
    x, g = nc["x"].cuda(), nc["w"].cuda()
    ow_q, ow_s = oracle.quantize(synth.bits(synth.gemm_case(1, N, K, seed=3)["w"]))
    w = mx.PackedWeight.from_rows(dev_u8(ow_q), dev_u8(ow_s))
    say(f"rmsnorm 128x4 -> gemm M={M}")
    _, q1, s1 = mx.mxfp8_rmsnorm_quantize(x, g, nc["eps"], scale_layout=mx.SCALES_128X4)
    _, q0, s0 = mx.mxfp8_rmsnorm_quantize(x, g, nc["eps"])
    tiled = mx.mxfp8_gemm_ex(q1, s1, w, mx.SCALES_128X4)
    row = mx.mxfp8_gemm(q0, s0, w)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1)
    assert np.array_equal(host_u8(s1), oracle.scales_to_128x4(host_u8(s0)))
    assert torch.equal(row.view(torch.int16), tiled.view(torch.int16))
    check_gemm(tiled, oracle.gemm(host_u8(q0), host_u8(s0), ow_q, ow_s), f"norm->gemm M={M}")


@pytest.mark.parametrize("M", [49, 64, 96, 100, 128, 200, 256])
@pytest.mark.parametrize("fused", [False, True])
def test_rows_above_48(M, fused, monkeypatch):
    # More than 48 rows: a grid of 64-row blocks on the 2D kernel (BF16 input
    # quantized by its own launch first); ragged last blocks included.
    monkeypatch.delenv("MXG_DIRECT_KERNEL", raising=False)
    run_case(M, 512, 2048, seed=M, fused=fused)


@pytest.mark.parametrize("M,N,K", [(64, 4096, 5120), (128, 5120, 8192), (256, 8192, 1536),
                                   (97, 2064, 16384)])
def test_rows_above_48_full_size(M, N, K):
    run_case(M, N, K, seed=M + 1, outliers=True)


@pytest.mark.parametrize("M", [64, 130, 256])
def test_rows_above_48_with_128x4_scales(M, monkeypatch):
    # rows past 128 sit in the second row of 128 x 4 tiles; the row-major
    # call runs on the same kernel as the 128 x 4 one (the 64-row blocks of
    # the 2D kernel), so the two must agree bit for bit
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "2d")
    N, K = 1024, 2048
    case = synth.gemm_case(M, N, K, seed=M + 2)
    oa_q, oa_s = oracle.quantize(synth.bits(case["x"]))
    ow_q, ow_s = oracle.quantize(synth.bits(case["w"]))
    ref = oracle.gemm(oa_q, oa_s, ow_q, ow_s)
    say(f"gemm 128x4 scales, rows above 48: M={M}")
    w = mx.PackedWeight.from_rows(dev_u8(ow_q), dev_u8(ow_s))
    row = mx.mxfp8_gemm(dev_u8(oa_q), dev_u8(oa_s), w)
    tiled = mx.mxfp8_gemm_ex(dev_u8(oa_q), dev_u8(oracle.scales_to_128x4(oa_s)), w,
                             mx.SCALES_128X4)
    torch.cuda.synchronize()
    assert torch.equal(row.view(torch.int16), tiled.view(torch.int16))
    check_gemm(tiled, ref, f"128x4 M={M}")


def test_rows_above_48_workspace_left_clean():
    M, N, K = 150, 4096, 5120
    w, _ = _weights(N, K, 0)
    ws = torch.zeros(int(mx.lib().mxg_gemm_workspace_bytes(M, N, K)) + 4096, dtype=torch.uint8,
                     device="cuda")
    x = synth.gemm_case(M, 16, K, seed=9)["x"].cuda()
    a_q = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    a_s = torch.empty(M, K // 32, dtype=torch.uint8, device="cuda")
    say(f"workspace hygiene, rows above 48: M={M}")
    first = mx.mxfp8_gemm(a_q, a_s, w, x=x, workspace=ws).clone()
    for _ in range(3):
        o = mx.mxfp8_gemm(a_q, a_s, w, workspace=ws)
        assert torch.equal(o.view(torch.int16), first.view(torch.int16))
    torch.cuda.synchronize()
    assert mx.workspace_error(ws) == 0
    assert not ws[:65536].any(), "counters must be back to zero"


@pytest.mark.parametrize("plan", ["1,1", "2,1", "4,1", "2,2", "4,2", "1,4", "4,4", "2,8"])
@pytest.mark.parametrize("M", [17, 48, 100])
def test_every_2d_plan(M, plan, monkeypatch):
    # MXG_PLAN forces the 2D kernel's (tiles per workgroup, K parts) plan:
    # every plan, with and without K split, one or several row blocks.
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "2d")
    monkeypatch.setenv("MXG_PLAN", plan)
    run_case(M, 512, 2048, seed=M + len(plan))


@pytest.mark.parametrize("plan", ["1,1", "2,1", "4,1", "1,2", "2,2", "4,2", "2,3", "4,4"])
@pytest.mark.parametrize("M", [9, 17, 32, 48])
def test_every_2d_plan_wave_local(M, plan, monkeypatch):
    # The wave-local form (each wave loads its own B operands) on every plan
    # it takes, K parts of 1..3 steps per wave included.
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "2d")
    monkeypatch.setenv("MXG_WAVE_LOCAL", "1")
    monkeypatch.setenv("MXG_PLAN", plan)
    run_case(M, 512, 4096, seed=M + 5 * len(plan))


@pytest.mark.parametrize("plan", ["1,1", "2,1", "4,1", "2,2", "4,2", "1,4", "4,4", "2,8"])
@pytest.mark.parametrize("M", [9, 17, 32])
def test_every_2d_plan_bf16_input(M, plan, monkeypatch):
    # BF16 input on the 2D kernel: quantized while staging (one or two
    # 32-blocks per thread) where the plan's part fits, else by a quantize
    # launch first; the codes the kernel writes out are checked bit for bit.
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "2d")
    monkeypatch.setenv("MXG_PLAN", plan)
    run_case(M, 512, 2048, seed=M + 3 * len(plan), fused=True)


@pytest.mark.parametrize("rsplit", ["1", "2", "4"])
@pytest.mark.parametrize("M,N,K,fused", [(1, 256, 1024, False), (5, 1024, 2048, True),
                                         (16, 2048, 5120, False), (4, 2048, 5120, True),
                                         (1, 1024, 4096, False), (3, 4096, 5120, True)])
def test_weight_tile_row_split(M, N, K, fused, rsplit, monkeypatch):
    # The M <= 16 kernel with each 16-row weight tile shared by 1, 2 or 4
    # workgroups (rows 16/rsplit each).
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "m16")
    monkeypatch.setenv("MXG_M16_RSPLIT", rsplit)
    run_case(M, N, K, seed=M + N + int(rsplit), fused=fused)


@pytest.mark.parametrize("form", [None, "64", "wide"])
@pytest.mark.parametrize("M,N,K", [(129, 64, 128), (129, 512, 1024), (200, 1088, 2048),
                                   (256, 4096, 5120), (100, 5120, 8192), (250, 320, 16384),
                                   (193, 8192, 2048), (200, 5184, 1536), (129, 1040, 4096),
                                   (160, 8192, 4096), (56, 5120, 8192), (64, 8192, 1536),
                                   (49, 1040, 2048)])
def test_big_tile_kernel(M, N, K, form, monkeypatch):
    # Above 48 rows, as routed and with each form forced: the 64 x 64 form
    # above 64 rows (grids up to one workgroup per CU with 8 waves each, and
    # beyond with 4) and the wide form (K split across 8 waves; 4, 2 or 1
    # weight tiles per workgroup, N = 1040 taking 1; one round of workgroups
    # or, at N 8192 K 4096 M 160, two; at 49-64 rows one row block, routed
    # there with two tiles per workgroup).  Ragged row blocks, a single K
    # step (K = 128) and ragged last chunks, N not a multiple of 512 (no XCD
    # grouping), the longest K.
    monkeypatch.delenv("MXG_DIRECT_KERNEL", raising=False)
    if form:
        monkeypatch.setenv("MXG_BIG_KERNEL", form)
    else:
        monkeypatch.delenv("MXG_BIG_KERNEL", raising=False)
    run_case(M, N, K, seed=M + K, outliers=True)


# ------------------------------------------------------ row-major weights
#
# The weight as a layer holds it ([N, K] codes, [N, K/32] scales), read
# without a repack: only the offsets of each lane's bytes change, so every
# kernel form, plan and summation order is that of the packed weight and the
# outputs must be equal bit for bit, besides lying within tolerance of the
# oracle.

def run_layouts(M, N, K, seed=0, fused=False, outliers=False, a_sf128=False):
    case = synth.gemm_case(M, N, K, seed=seed, outliers=outliers)
    x_bits, w_bits = synth.bits(case["x"]), synth.bits(case["w"])
    ow_q, ow_s = oracle.quantize(w_bits)
    oa_q, oa_s = oracle.quantize(x_bits)
    ref = oracle.gemm(oa_q, oa_s, ow_q, ow_s)
    say(f"gemm layouts M={M} N={N} K={K} seed={seed} fused={fused} outliers={outliers} "
        f"a_sf128={a_sf128}")
    w_q, w_s = dev_u8(ow_q), dev_u8(ow_s)
    outs = []
    for w in (mx.RowMajorWeight(w_q, w_s), mx.PackedWeight.from_rows(w_q, w_s)):
        if fused:
            a_q = torch.full((M, K), 0x55, dtype=torch.uint8, device="cuda")
            a_s = torch.full((M, K // 32), 0x55, dtype=torch.uint8, device="cuda")
            out = mx.mxfp8_gemm(a_q, a_s, w, x=dev_bf16(x_bits))
        elif a_sf128:
            a_q, a_s = dev_u8(oa_q), dev_u8(oracle.scales_to_128x4(oa_s))
            out = mx.mxfp8_gemm_ex(a_q, a_s, w, mx.SCALES_128X4)
        else:
            a_q, a_s = dev_u8(oa_q), dev_u8(oa_s)
            out = mx.mxfp8_gemm(a_q, a_s, w)
        torch.cuda.synchronize()
        if fused:
            assert np.array_equal(host_u8(a_q), oa_q) and np.array_equal(host_u8(a_s), oa_s)
        outs.append(out)
    check_gemm(outs[0], ref, f"row-major M={M} N={N} K={K}")
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "layouts differ"


@pytest.mark.parametrize("M", [1, 2, 5, 8, 16, 17, 32, 33, 48])
@pytest.mark.parametrize("fused", [False, True])
def test_row_major_weights_rows_sweep(M, fused, path):
    run_layouts(M, 256, 1024, seed=M + 100, fused=fused)


@pytest.mark.parametrize("M,N,K,fused", [
    (1, 4096, 5120, True), (4, 4096, 5120, True), (8, 4096, 5120, True),   # decode bucket
    (16, 4096, 5120, False), (48, 4096, 5120, False), (32, 5120, 8192, False),
    (48, 8192, 1536, False),                                                # wide tiles
    (4, 5120, 8192, True), (3, 4112, 1024, False),                          # half tiles
    (17, 512, 16384, True), (1, 16, 128, False),                            # edges of K and N
    (64, 4096, 5120, False), (200, 4096, 5120, False), (256, 2048, 8192, True),  # rows above 48
])
def test_row_major_weights_shapes(M, N, K, fused):
    run_layouts(M, N, K, seed=N + M, fused=fused, outliers=not fused)


@pytest.mark.parametrize("M", [3, 20, 48, 100])
def test_row_major_weights_with_128x4_scales(M):
    run_layouts(M, 1024, 2048, seed=M + 5, a_sf128=True)
