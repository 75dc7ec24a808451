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


# ---------------------------------------------------- 128 x 4 scale tiles
# Parity unpinned against the real F8_128x4 producers (the pages name the
# layout but do not print it); these pin the oracle's permutation to its own
# stated structure: a tile holds exactly a 128-row x 4-column block, each
# 16-byte line holds one row of each 32-row quarter, nothing is lost.

def test_128x4_is_a_permutation_into_padded_tiles():
    rng = np.random.default_rng(3)
    for M, KB in ((1, 4), (5, 48), (48, 160), (130, 8)):
        s = rng.integers(1, 256, (M, KB)).astype(np.uint8)
        out = oracle.scales_to_128x4(s)
        assert out.size == ((M + 127) // 128) * 128 * KB
        assert np.count_nonzero(out) == M * KB          # every byte placed once
        assert sorted(out[out != 0].tolist()) == sorted(s.ravel().tolist())


def test_128x4_tile_contents():
    M, KB = 130, 8
    m_idx, b_idx = np.meshgrid(np.arange(M), np.arange(KB), indexing="ij")
    # each byte names its (row, column) modulo 255, never 0
    lo = oracle.scales_to_128x4(((m_idx * KB + b_idx) % 255 + 1).astype(np.uint8))
    tiles = lo.reshape(-1, 512)
    assert tiles.shape[0] == 2 * (KB // 4)
    # tile 1 is rows 0..127, columns 4..7; its line 5 holds rows 5, 37, 69, 101
    line = tiles[1][5 * 16:(5 + 1) * 16].reshape(4, 4)
    for q in range(4):
        m = 5 + 32 * q
        assert list(line[q]) == [(m * KB + b) % 255 + 1 for b in range(4, 8)]
    # the third row tile (rows 128, 129) starts at tile index 2 (columns 0..3)
    assert list(tiles[2][0:4]) == [(128 * KB + b) % 255 + 1 for b in range(4)]
    assert list(tiles[2][16:20]) == [(129 * KB + b) % 255 + 1 for b in range(4)]
    assert not tiles[2][32:].any()                      # padding rows 130..255
