"""Pins of the oracle's format functions (E4M3 / E8M0 / BF16) to things other
than the oracle itself: hand-written values from the OCP format definitions
(tests/golden/e4m3_e8m0_values.txt), torch's own float8_e4m3fn and bfloat16
conversions (library routines), exact rational arithmetic, and invariants."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_value(tok: str):
    if tok == "nan":
        return math.nan
    neg = tok.startswith("-")
    t = tok[1:] if neg else tok
    v = Fraction(2) ** int(t[3:-1]) if t.startswith("p2(") else Fraction(t)
    return -v if neg else v


def _golden_formats():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_e8m0_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, code, val = line.split()
            rows.append((fmt, int(code, 16), val))
    return rows


@pytest.mark.parametrize("fmt,code,val", _golden_formats())
def test_golden_format_values(fmt, code, val):
    got = oracle.e4m3_value([code])[0] if fmt == "e4m3" else oracle.e8m0_value([code])[0]
    want = _parse_value(val)
    if isinstance(want, float) and math.isnan(want):
        assert math.isnan(got)
    else:
        assert Fraction(got) == want
        if val == "-0" or val == "0":
            assert math.copysign(1.0, got) == (-1.0 if val == "-0" else 1.0)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_value(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], theirs[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(theirs[~nan]))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]


def test_e4m3_roundtrip_and_order():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_value(codes)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    pos = oracle.e4m3_value(np.arange(127, dtype=np.uint8))
    assert (np.diff(pos) > 0).all(), "codes 0..126 must increase strictly"
    neg = oracle.e4m3_value(np.arange(128, 255, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_value(b)
    keep = np.isfinite(v)
    return b[keep], v[keep]


def test_e4m3_encode_matches_torch_rne_in_range():
    # torch's float32 -> float8_e4m3fn rounds to nearest even and gives NaN only
    # above 464 (the midpoint of 448 and the NaN slot), so in [-464, 464] it is
    # an independent implementation of the same rounding.
    _, v = _all_finite_bf16()
    v = v[np.abs(v) <= 464.0]
    ours = oracle.e4m3_encode(v)
    theirs = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_encode_saturates():
    big = np.array([448.0, 449.0, 464.0, 464.5, 480.0, 511.9, 1e6, 3e38])
    assert (oracle.e4m3_encode(big) == 0x7E).all()
    assert (oracle.e4m3_encode(-big) == 0xFE).all()


def test_e4m3_encode_ties_and_subnormals_exact():
    # Exact midpoints between neighbouring codes go to the even code.
    pos = [Fraction(x) for x in oracle.e4m3_value(np.arange(127, dtype=np.uint8))]
    mids = [(pos[i] + pos[i + 1]) / 2 for i in range(126)]
    got = oracle.e4m3_encode(np.array([float(m) for m in mids]))
    want = [i if i % 2 == 0 else i + 1 for i in range(126)]
    assert got.tolist() == want
    assert oracle.e4m3_encode([2.0 ** -10, 2.0 ** -10 * 1.0001, -1e-30]).tolist() == [0, 1, 0x80]


def _bf16_rne_exact(x: Fraction) -> int:
    """Nearest BF16 (ties to even) of an exact rational, by exact arithmetic."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    p = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** p > a:
        p -= 1
    while Fraction(2) ** (p + 1) <= a:
        p += 1
    p = max(p, -126)
    q = Fraction(2) ** (p - 7)
    n, r = divmod(a, q)
    n = int(n)
    if r > q / 2 or (r == q / 2 and n % 2 == 1):
        n += 1
    val = n * q
    f = np.float32(float(val))
    assert Fraction(float(f)) == val
    return sign | int(np.array([f]).view(np.uint32)[0] >> 16)


def test_bf16_round_exact_random():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                         rng.standard_normal(200) * 2.0 ** -130])
    ours = oracle.bf16_round(xs)
    for x, o in zip(xs, ours):
        assert o == _bf16_rne_exact(Fraction(float(x))), x


def test_bf16_round_matches_torch_for_float32():
    rng = np.random.default_rng(2)
    xs = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    theirs = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(xs.astype(np.float64)), theirs)


def test_bf16_ties():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even -> 1.0
    assert oracle.bf16_round([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]).tolist() == [
        0x3F80, 0x3F82, 0xBF80]


def test_bf16_value_exact():
    b, v = _all_finite_bf16()
    assert np.array_equal(oracle.bf16_round(v), b)
