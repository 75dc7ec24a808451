"""GPU parity of mxfp8_rmsnorm_quantize against the oracle.

The BF16 row y is compared with the oracle's unrounded fp64 RMSNorm within
the bound of an FP32 evaluation rounded once to BF16 (half a BF16 ulp, 2^-8
relative, plus (K/2 + 4) * 2^-24).  The codes and scales are compared bit for
bit with the oracle's quantize of the GPU's own BF16 row (a stage downstream
of a floating-point step is checked on that step's output); rows whose BF16
values all equal the oracle's rounding are therefore also exact end to end.
The 128 x 4 scale layout is compared byte for byte (padding included) with
the oracle's permutation of the row-major scales."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_gemm_amd as mx
import oracle
import synth
from helpers import dev_bf16, host_bits, host_u8, say

pytestmark = pytest.mark.gpu


def run_case(M, K, seed=0, ld=None, outliers=False, layout=mx.SCALES_ROW_MAJOR):
    case = synth.rmsnorm_case(M, K, seed=seed, ld=ld, outliers=outliers)
    x_bits, w_bits, eps = synth.bits(case["x"]), synth.bits(case["w"]), case["eps"]
    say(f"rmsnorm M={M} K={K} ld={ld} seed={seed} outliers={outliers} layout={layout}")
    x = dev_bf16(x_bits)
    y, q, s = mx.mxfp8_rmsnorm_quantize(x, dev_bf16(w_bits), eps, K=K, scale_layout=layout)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x_bits, w_bits, eps, K=K)
    yg = host_bits(y)
    err = np.abs(oracle.bf16_value(yg) - ref)
    tol = oracle.rmsnorm_tolerance(ref, K)
    assert np.all(err <= tol), f"max excess {np.max(err - tol)}"
    oq, os_ = oracle.quantize(yg)
    assert np.array_equal(host_u8(q), oq)
    if layout == mx.SCALES_128X4:
        assert np.array_equal(host_u8(s), oracle.scales_to_128x4(os_))
    else:
        assert np.array_equal(host_u8(s), os_)
    # most elements round to the same BF16 as the exact value
    same = np.mean(yg == oracle.bf16_round(ref))
    assert same > 0.99, same
    return yg, host_u8(q)


@pytest.mark.parametrize("M", [1, 2, 3, 8, 16, 33, 48])
@pytest.mark.parametrize("K", [128, 1536, 5120])
def test_rows_and_widths(M, K):
    run_case(M, K, seed=M * 7 + K)


@pytest.mark.parametrize("K", [8192, 16384])
def test_widest_rows(K):
    # K = MXG_MAX_K: two 32-blocks per thread
    run_case(5, K, seed=K)


def test_leading_columns_of_wider_rows():
    # qr: the leading 1536 columns of A's 2048-column output
    run_case(8, 1536, seed=1, ld=2048)


def test_outlier_rows():
    run_case(16, 5120, seed=2, outliers=True)


@pytest.mark.parametrize("M", [1, 48, 130])
def test_scales_in_128x4_tiles(M):
    run_case(M, 1536, seed=M, layout=mx.SCALES_128X4)


def test_without_y_gives_the_same_codes():
    case = synth.rmsnorm_case(8, 5120, seed=4)
    x, w = case["x"].cuda(), case["w"].cuda()
    say("rmsnorm without y")
    _, q1, s1 = mx.mxfp8_rmsnorm_quantize(x, w, case["eps"])
    y2, q2, s2 = mx.mxfp8_rmsnorm_quantize(x, w, case["eps"], write_y=False)
    torch.cuda.synchronize()
    assert y2 is None
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


def test_constant_row_returns_the_gain_bitwise():
    K = 5120
    case = synth.rmsnorm_case(1, K, seed=5)
    w = case["w"]
    say("rmsnorm constant rows")
    for c in (3.0, -0.0078125, 1000.0):
        x = torch.full((1, K), c, dtype=torch.bfloat16).cuda()
        y, _, _ = mx.mxfp8_rmsnorm_quantize(x, w.cuda(), 0.0)
        torch.cuda.synchronize()
        want = synth.bits(w)[None, :] ^ (np.uint16(0x8000) if c < 0 else np.uint16(0))
        assert np.array_equal(host_bits(y), want)


def test_zero_row():
    K = 1536
    case = synth.rmsnorm_case(2, K, seed=6)
    x = case["x"].clone()
    x[1] = 0
    say("rmsnorm zero row")
    y, q, s = mx.mxfp8_rmsnorm_quantize(x.cuda(), case["w"].cuda(), case["eps"])
    torch.cuda.synchronize()
    assert not host_bits(y)[1].any() and not host_u8(q)[1].any() and not host_u8(s)[1].any()


def test_rejected_call_writes_nothing():
    K = 1536
    case = synth.rmsnorm_case(4, K, seed=7)
    x, w = case["x"].cuda(), case["w"].cuda()
    q = torch.full((4, K), 0x55, dtype=torch.uint8, device="cuda")
    s = torch.full((4, K // 32), 0x55, dtype=torch.uint8, device="cuda")
    say("rmsnorm rejected call")
    st = mx.lib().mxfp8_rmsnorm_quantize(x.data_ptr(), 4, K, K, w.data_ptr(), -1.0, None, 0,
                                         q.data_ptr(), s.data_ptr(), 0, None)
    torch.cuda.synchronize()
    assert st == 3
    assert (q == 0x55).all() and (s == 0x55).all()
