"""GPU check of mxfp8_gemm_noalloc, the entry point for callers that cannot
allocate: its K-split counters and partial sums live in the library's own
per-GPU device scratch instead of a caller workspace.  It runs the same
kernels with the same plan as mxfp8_gemm, so the two outputs must agree bit
for bit, and both must be within tolerance of the oracle.  Two calls in a
row, the second on a smaller input, so the second runs on the scratch the
first left behind; then the pair again, in the opposite order."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_gemm_amd as mx
import oracle
import synth
from helpers import check_gemm, dev_bf16, dev_u8, host_u8, say

pytestmark = pytest.mark.gpu

# Shapes whose plans split K across workgroups (partials in the scratch):
# the large one first, then a smaller one on the same scratch.
LARGE = (48, 4096, 5120)
SMALL = (24, 1024, 8192)


def _inputs(M, N, K, seed):
    case = synth.gemm_case(M, N, K, seed=seed, outliers=True)
    xb, wb = synth.bits(case["x"]), synth.bits(case["w"])
    oa, ow = oracle.quantize(xb), oracle.quantize(wb)
    w = mx.PackedWeight.from_rows(dev_u8(ow[0]), dev_u8(ow[1]))
    return xb, oa, ow, w


def _one(M, N, K, seed, bf16_in):
    need = int(mx.lib().mxg_gemm_workspace_bytes(M, N, K))
    assert mx.lib().mxg_gemm_workspace_bytes(M, N, K) > 65536, "shape must use K-split partials"
    assert need <= mx.NOALLOC_SCRATCH_BYTES
    xb, oa, ow, w = _inputs(M, N, K, seed)
    say(f"noalloc M={M} N={N} K={K} seed={seed} bf16_in={bf16_in} need={need}")
    if bf16_in:
        x = dev_bf16(xb)
        aq1 = torch.empty(M, K, dtype=torch.uint8, device="cuda")
        as1 = torch.empty(M, K // 32, dtype=torch.uint8, device="cuda")
        aq2, as2 = torch.empty_like(aq1), torch.empty_like(as1)
    else:
        x = None
        aq1, as1 = dev_u8(oa[0]), dev_u8(oa[1])
        aq2, as2 = aq1, as1
    out1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    out2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    mx.mxfp8_gemm(aq1, as1, w, out=out1, x=x, workspace=ws)
    mx.mxfp8_gemm_noalloc(aq2, as2, w, out=out2, x=x)
    torch.cuda.synchronize()
    assert mx.workspace_error(ws) == 0
    if bf16_in:
        assert np.array_equal(host_u8(aq2), oa[0]) and np.array_equal(host_u8(as2), oa[1])
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "noalloc differs from mxfp8_gemm"
    check_gemm(out2, oracle.gemm(oa[0], oa[1], ow[0], ow[1]), f"noalloc M={M} N={N} K={K}")


@pytest.mark.parametrize("bf16_in", [False, True])
def test_noalloc_matches_workspace_call_twice(bf16_in):
    _one(*LARGE, seed=3, bf16_in=bf16_in)
    _one(*SMALL, seed=4, bf16_in=bf16_in)


def test_noalloc_small_then_large():
    _one(*SMALL, seed=5, bf16_in=False)
    _one(*LARGE, seed=6, bf16_in=False)


def test_noalloc_repeated_calls_stay_exact():
    """Ten calls in a row on one stream: each leaves the counters at zero."""
    M, N, K = LARGE
    xb, oa, ow, w = _inputs(M, N, K, 7)
    aq, as_ = dev_u8(oa[0]), dev_u8(oa[1])
    ref = mx.mxfp8_gemm(aq, as_, w)
    outs = [mx.mxfp8_gemm_noalloc(aq, as_, w) for _ in range(10)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
