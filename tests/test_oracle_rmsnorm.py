"""Pins of the oracle's RMSNorm (and its MXFP8 requantize) against what the
definition fixes on its own: hand-worked rows (tests/golden/rmsnorm_values.txt),
exact rational squares on small rows, invariance under power-of-two scaling,
a constant row giving the gain back, unit mean square, the place of eps, and
planted mistakes that these checks must catch."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(v):
    return oracle.bf16_round(np.asarray(v, dtype=np.float64))


def _golden_rows():
    rows = []
    for line in open(os.path.join(GOLDEN, "rmsnorm_values.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        K, eps, xs, w, ys = [f.strip() for f in line.split("|")]
        K = int(K)
        x = np.zeros(K)
        for e in xs.split():
            k, v = e.split("=")
            x[int(k)] = float(v)
        want = []
        for e in ys.split():
            k, rest = e.split("=")
            val, bits = rest.split(":")
            want.append((int(k), float(val), int(bits, 16)))
        rows.append((K, float(eps), x, float(w), want))
    return rows


@pytest.mark.parametrize("K,eps,x,w,want", _golden_rows())
def test_golden_rows(K, eps, x, w, want):
    xb = _bf16(x)[None, :]
    wb = _bf16(np.full(K, w))
    y, yb, q, s = oracle.rmsnorm_quantize(xb, wb, eps)
    for k, val, bits in want:
        assert y[0, k] == pytest.approx(val, rel=1e-15, abs=0.0)
        assert int(yb[0, k]) == bits


@pytest.mark.parametrize("K", [32, 64, 96])
def test_exact_rational_squares(K):
    # With eps = 0 and rational eps, y_j^2 = x_j^2 w_j^2 / (sum x^2 / K + eps)
    # is rational: compare the oracle's squares with exact fractions.
    rng = np.random.default_rng(K)
    for eps in (0.0, 0.25):
        xb = _bf16(rng.standard_normal((3, K)))
        wb = _bf16(1 + 0.1 * rng.standard_normal(K))
        y = oracle.rmsnorm(xb, wb, eps)
        xv, wv = oracle.bf16_value(xb), oracle.bf16_value(wb)
        for m in range(3):
            ms = sum(Fraction(float(v)) ** 2 for v in xv[m]) / K + Fraction(eps)
            for j in range(K):
                exact = Fraction(float(xv[m, j])) ** 2 * Fraction(float(wv[j])) ** 2 / ms
                assert abs(Fraction(float(y[m, j])) ** 2 - exact) <= exact * Fraction(1, 2 ** 48)


@pytest.mark.parametrize("d", [-20, -3, 1, 7, 30])
def test_power_of_two_scaling_is_exact(d):
    rng = np.random.default_rng(100 + d)
    xb = _bf16(rng.standard_normal((4, 256)))
    wb = _bf16(1 + 0.1 * rng.standard_normal(256))
    y = oracle.rmsnorm(xb, wb, 0.0)
    y2 = oracle.rmsnorm(_bf16(oracle.bf16_value(xb) * 2.0 ** d), wb, 0.0)
    assert np.array_equal(y, y2)


def test_constant_row_gives_the_gain():
    K = 512
    rng = np.random.default_rng(7)
    wb = _bf16(1 + 0.1 * rng.standard_normal(K))
    for c in (3.0, 0.0078125, 1000.0):
        xb = _bf16(np.full((1, K), c))
        _, yb, _, _ = oracle.rmsnorm_quantize(xb, wb, 0.0)
        assert np.array_equal(yb[0], wb)
        _, ybn, _, _ = oracle.rmsnorm_quantize(_bf16(np.full((1, K), -c)), wb, 0.0)
        assert np.array_equal(ybn[0], wb ^ np.uint16(0x8000))


def test_unit_mean_square_and_eps_inside_the_root():
    K = 1536
    rng = np.random.default_rng(11)
    xb = _bf16(3.0 * rng.standard_normal((2, K)))
    ones = _bf16(np.ones(K))
    y = oracle.rmsnorm(xb, ones, 0.0)
    assert np.allclose(np.mean(y ** 2, axis=1), 1.0, rtol=1e-13, atol=0)
    # eps equal to the row's mean square halves the mean square of y
    xv = oracle.bf16_value(xb)
    for m in range(2):
        ms = float(np.mean(xv[m] ** 2))
        ye = oracle.rmsnorm(xb[m:m + 1], ones, ms)
        assert np.allclose(ye[0], y[m] / np.sqrt(2.0), rtol=1e-14, atol=0)
    # zero row: zero output, no NaN
    assert not oracle.rmsnorm(_bf16(np.zeros((1, K))), ones, 1e-6).any()


def test_gain_is_per_column():
    K = 64
    xb = _bf16(np.ones((1, K)))
    w = np.arange(1, K + 1, dtype=np.float64)
    y = oracle.rmsnorm(xb, _bf16(w), 0.0)
    assert np.array_equal(y[0], w)


def test_requantize_is_the_quantizer_of_the_rounded_row():
    rng = np.random.default_rng(5)
    xb = _bf16(rng.standard_normal((5, 1536)))
    wb = _bf16(1 + 0.1 * rng.standard_normal(1536))
    y, yb, q, s = oracle.rmsnorm_quantize(xb, wb, 1e-6)
    q2, s2 = oracle.quantize(yb)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.all(np.abs(oracle.bf16_value(yb) - y) <= oracle.rmsnorm_tolerance(y, 1536))


def test_planted_mistakes_are_caught():
    # A mean over K + 1 columns, eps added to the sum instead of the mean, or
    # a missing gain each moves the first golden row off its hand value.
    K, eps, x, w, want = _golden_rows()[0]
    xv = oracle.bf16_value(_bf16(x))
    k, val, _ = want[0]
    wrong = [xv[k] * w / np.sqrt(np.sum(xv ** 2) / (K + 1) + eps),
             xv[k] * w / np.sqrt((np.sum(xv ** 2) + 1.0) / K),
             xv[k] / np.sqrt(np.mean(xv ** 2) + eps) * 0.5]
    for v in wrong:
        assert v != pytest.approx(val, rel=1e-6)
