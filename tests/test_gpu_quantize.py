"""GPU parity of mxfp8_quantize against the oracle: codes and scale bytes
must match bit for bit (they are a unique function of the BF16 input)."""
import os

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_gemm_amd as mx
import oracle
import synth
from helpers import dev_bf16, host_u8, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_quantize(bits: np.ndarray, K=None):
    x = dev_bf16(bits)
    q, s = mx.mxfp8_quantize(x, K=K)
    torch.cuda.synchronize()
    return host_u8(q), host_u8(s)


@pytest.mark.parametrize("shift", [0, 1, 3, 6, 9, 12, 16])
def test_exhaustive_bf16_values(shift):
    """Every finite BF16 x, in a block whose amax is |x| * 2^shift."""
    say(f"quantize exhaustive shift={shift}")
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_value(b)
    comp = np.abs(v) * 2.0 ** shift
    keep = np.isfinite(v) & np.isfinite(comp) & (comp < 3.0e38)
    x = np.zeros((keep.sum(), 32), dtype=np.uint16)
    x[:, 3] = b[keep]
    x[:, 20] = oracle.bf16_round(comp[keep])
    gq, gs = gpu_quantize(x)
    oq, os_ = oracle.quantize(x)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gq, oq)


def test_golden_blocks():
    from test_oracle_quantize import _golden_blocks
    blocks = _golden_blocks()
    x = np.stack([oracle.bf16_round(b) for b, _, _ in blocks])
    say(f"quantize golden blocks n={len(blocks)}")
    gq, gs = gpu_quantize(x)
    for i, (_, scale, codes) in enumerate(blocks):
        assert gs[i, 0] == scale and np.array_equal(gq[i], codes), i


@pytest.mark.parametrize("M,K,ld,seed", [(1, 32, 32, 0), (3, 96, 104, 1), (8, 5120, 5120, 2),
                                         (37, 1536, 2048, 3), (48, 8192, 8192, 4),
                                         (300, 4096, 4096, 5), (70000, 64, 64, 6)])
def test_random_shapes_and_strides(M, K, ld, seed):
    say(f"quantize M={M} K={K} ld={ld} seed={seed}")
    g = torch.Generator().manual_seed(seed)
    full = (torch.randn(M, ld, generator=g) * torch.exp2(torch.randint(-30, 30, (M, 1), generator=g).float()))
    bits = synth.bits(full.to(torch.bfloat16))
    x = dev_bf16(bits)
    q, s = mx.mxfp8_quantize(x, K=K)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize(bits, K=K)
    assert np.array_equal(host_u8(s), os_)
    assert np.array_equal(host_u8(q), oq)


def test_weight_sized_matrix():
    say("quantize weights N=4096 K=5120")
    w = synth.gemm_case(1, 4096, 5120, seed=0)["w"]
    bits = synth.bits(w)
    gq, gs = gpu_quantize(bits)
    oq, os_ = oracle.quantize(bits)
    assert np.array_equal(gs, os_) and np.array_equal(gq, oq)


def test_zero_input():
    say("quantize zeros")
    gq, gs = gpu_quantize(np.zeros((5, 256), np.uint16))
    assert not gq.any() and not gs.any()


def test_rejected_call_writes_nothing():
    say("quantize rejected call")
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    q = torch.full((4, 64), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((4, 2), 0xCD, dtype=torch.uint8, device="cuda")
    st = mx.lib().mxfp8_quantize(x.data_ptr(), 4, 48, 64, q.data_ptr(), s.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == 3
    assert (q == 0xAB).all() and (s == 0xCD).all()


@pytest.mark.parametrize("shift", [0, 3, 9])
def test_exhaustive_bf16_values_fused_in_gemm(shift, monkeypatch):
    """The quantize fused into the M <= 16 GEMM kernel (one 32-block per
    lane) on the same blocks as above: every finite BF16 value, the codes
    and scales it writes out must equal the oracle's."""
    monkeypatch.setenv("MXG_DIRECT_KERNEL", "m16")
    say(f"fused quantize exhaustive shift={shift}")
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_value(b)
    comp = np.abs(v) * 2.0 ** shift
    keep = np.isfinite(v) & np.isfinite(comp) & (comp < 3.0e38)
    x = np.zeros((keep.sum(), 32), dtype=np.uint16)
    x[:, 3] = b[keep]
    x[:, 20] = oracle.bf16_round(comp[keep])
    M, K = 8, 8192                                  # 2048 blocks per call: quantized in-kernel
    per = M * K // 32
    x = np.concatenate([x, np.zeros((-len(x) % per, 32), np.uint16)])
    oq, os_ = oracle.quantize(x)
    w = mx.PackedWeight.from_rows(torch.zeros(16, K, dtype=torch.uint8, device="cuda"),
                                  torch.full((16, K // 32), 127, dtype=torch.uint8, device="cuda"))
    gq = np.empty_like(oq)
    gs = np.empty_like(os_)
    for i in range(0, len(x), per):
        xb = dev_bf16(x[i:i + per].reshape(M, K))
        a_q = torch.empty(M, K, dtype=torch.uint8, device="cuda")
        a_s = torch.empty(M, K // 32, dtype=torch.uint8, device="cuda")
        mx.mxfp8_gemm(a_q, a_s, w, x=xb)
        torch.cuda.synchronize()
        gq[i:i + per] = host_u8(a_q).reshape(per, 32)
        gs[i:i + per] = host_u8(a_s).reshape(per, 1)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gq, oq)
