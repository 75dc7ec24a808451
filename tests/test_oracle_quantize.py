"""Pins of the oracle's MXFP8 quantizer: hand-worked blocks
(tests/golden/quantize_blocks.txt), an exhaustive check of the scale rule
against the BF16 bit fields, an exhaustive check of the codes against torch's
float8 rounding, and invariants (idempotence, sign symmetry, power-of-two
covariance, zero)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(tok):
    neg = tok.startswith("-")
    t = tok[1:] if neg else tok
    v = 2.0 ** int(t[3:-1]) if t.startswith("p2(") else float(Fraction(t))
    return -v if neg else v


def _golden_blocks():
    out = []
    with open(os.path.join(GOLDEN, "quantize_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("=>")
            block = np.zeros(32)
            for item in lhs.split():
                i, v = item.split(":")
                block[int(i)] = _val(v)
            toks = rhs.split()
            codes = np.zeros(32, dtype=np.uint8)
            for item in toks[1:]:
                i, c = item.split(":")
                codes[int(i)] = int(c, 16)
            out.append((block, int(toks[0], 16), codes))
    return out


@pytest.mark.parametrize("block,scale,codes", _golden_blocks())
def test_golden_blocks(block, scale, codes):
    x = oracle.bf16_round(block)
    assert np.array_equal(oracle.bf16_value(x), block), "golden values must be BF16"
    q, s = oracle.quantize(x[None, :])
    assert s[0, 0] == scale
    assert np.array_equal(q[0], codes)


def _p_from_bits(b: np.ndarray) -> np.ndarray:
    """floor(log2 |x|) of non-zero BF16 patterns, from the bit fields alone."""
    E = (b >> 7) & 0xFF
    m = (b & 0x7F).astype(np.int64)
    p = E.astype(np.int64) - 127
    sub = E == 0
    # subnormal: m * 2^-133, floor(log2) = bit_length(m) - 1 - 133
    bl = np.floor(np.log2(np.maximum(m, 1))).astype(np.int64)  # exact for m < 128
    p[sub] = bl[sub] - 133
    return p


def test_scale_rule_exhaustive():
    b = np.arange(0x7F80, dtype=np.uint32).astype(np.uint16)   # all finite x >= 0
    expect = np.clip(_p_from_bits(b) - 8 + 127, 0, 254)
    expect[b == 0] = 0
    x = np.zeros((len(b), 32), dtype=np.uint16)
    x[:, 7] = b
    _, s = oracle.quantize(x)
    assert np.array_equal(s[:, 0].astype(np.int64), expect)
    # unclamped blocks: amax / scale lies in [256, 512)
    v = oracle.bf16_value(b)
    sc = np.ldexp(1.0, s[:, 0].astype(np.int64) - 127)
    ok = (b != 0) & (s[:, 0] > 0)
    r = v[ok] / sc[ok]
    assert (r >= 256).all() and (r < 512).all()


def _torch_codes(scaled: np.ndarray) -> np.ndarray:
    """E4M3 codes by torch's rounding, with the saturation reading above 448."""
    c = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    big = np.abs(scaled) >= 448.0
    c[big] = np.where(np.signbit(scaled[big]), 0xFE, 0x7E)
    return c


@pytest.mark.parametrize("shift", [0, 1, 3, 6, 9, 12, 16])
def test_codes_exhaustive_against_torch(shift):
    """Every finite BF16 x in a block whose amax is |x| * 2^shift."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_value(b)
    comp = np.abs(v) * 2.0 ** shift
    keep = np.isfinite(v) & np.isfinite(comp) & (comp < 3.0e38)
    b, v, comp = b[keep], v[keep], comp[keep]
    cb = oracle.bf16_round(comp)
    assert np.array_equal(oracle.bf16_value(cb), comp)
    x = np.zeros((len(b), 32), dtype=np.uint16)
    x[:, 3] = b
    x[:, 20] = cb
    q, s = oracle.quantize(x)
    e = s[:, 0].astype(np.int64) - 127
    want = _torch_codes(np.ldexp(v, -e))
    assert np.array_equal(q[:, 3], want)


def test_invariants_random():
    rng = np.random.default_rng(7)
    f = rng.standard_normal((16, 256)) * np.exp2(rng.integers(-20, 20, (16, 1)))
    x = oracle.bf16_round(f)
    q, s = oracle.quantize(x)
    # idempotence: quantize(dequant(q, s)) == (q, s)
    dq = oracle.dequantize(q, s)
    q2, s2 = oracle.quantize(oracle.bf16_round(dq))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # sign symmetry: codes flip bit 7, scales unchanged
    qn, sn = oracle.quantize(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, q ^ np.uint8(0x80)) and np.array_equal(sn, s)
    # power-of-two covariance: same codes, scale + d
    for d in (-5, 1, 7):
        qd, sd = oracle.quantize(oracle.bf16_round(oracle.bf16_value(x) * 2.0 ** d))
        assert np.array_equal(qd, q)
        assert np.array_equal(sd.astype(int), s.astype(int) + d)


def test_zero_input():
    q, s = oracle.quantize(np.zeros((3, 128), dtype=np.uint16))
    assert not q.any() and not s.any()


def test_row_stride_and_leading_columns():
    rng = np.random.default_rng(3)
    x = oracle.bf16_round(rng.standard_normal((4, 96)))
    q_full, s_full = oracle.quantize(x)
    q_lead, s_lead = oracle.quantize(x, K=64)
    assert np.array_equal(q_lead, q_full[:, :64]) and np.array_equal(s_lead, s_full[:, :2])
