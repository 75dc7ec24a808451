"""Pins of the oracle's block-scaled GEMM: hand-worked dot products
(tests/golden/gemm_dot.txt), brute force in exact rationals on tiny shapes
(with element values decoded by torch, not by the oracle), numpy's fp64
matmul of independently dequantized operands, linearity in one block's scale
exponent, one-hot weights and zero input."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_dequant(q, s):
    """fp64 dequantization with torch's float8 decode (independent of oracle)."""
    return _torch_e4m3(q) * np.repeat(np.exp2(s.astype(np.float64) - 127.0), 32, axis=1)


def _bf16_rne(x: Fraction) -> int:
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
    quantum = Fraction(2) ** (p - 7)
    n, r = divmod(a, quantum)
    n = int(n)
    if r > quantum / 2 or (r == quantum / 2 and n % 2):
        n += 1
    f = np.float32(float(n * quantum))
    return sign | int(np.array([f]).view(np.uint32)[0] >> 16)


def _golden_dots():
    rows = []
    with open(os.path.join(GOLDEN, "gemm_dot.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("=>")
            K, rest = lhs.split(None, 1)
            K = int(K)
            a_part, w_part = rest.split("|")

            def parse(part):
                codes_tok, scale_tok = part.split(";")
                q = np.zeros((1, K), dtype=np.uint8)
                for item in codes_tok.split():
                    k, c = item.split(":")
                    q[0, int(k)] = int(c, 16)
                s = np.array([[int(t, 16) for t in scale_tok.split()]], dtype=np.uint8)
                return q, s

            aq, as_ = parse(a_part)
            wq, ws = parse(w_part)
            val, bits = rhs.split()
            rows.append((aq, as_, wq, ws, Fraction(val), int(bits, 16)))
    return rows


@pytest.mark.parametrize("aq,as_,wq,ws,exact,bits", _golden_dots())
def test_golden_dots(aq, as_, wq, ws, exact, bits):
    r = oracle.gemm(aq, as_, wq, ws)
    assert Fraction(r.ref[0, 0]) == exact
    assert r.bf16[0, 0] == bits


def _random_mx(rng, rows, K, scale_lo=110, scale_hi=140):
    q = rng.integers(0, 256, (rows, K)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38          # no NaN codes
    s = rng.integers(scale_lo, scale_hi, (rows, K // 32)).astype(np.uint8)
    return q, s


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (3, 2, 96), (3, 3, 96), (1, 3, 64)])
def test_brute_force_exact(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    aq, as_ = _random_mx(rng, M, K)
    wq, ws = _random_mx(rng, N, K)
    r = oracle.gemm(aq, as_, wq, ws)
    av = _torch_e4m3(aq); wv = _torch_e4m3(wq)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            sabs = Fraction(0)
            for k in range(K):
                t = (Fraction(av[m, k]) * Fraction(2) ** (int(as_[m, k // 32]) - 127)
                     * Fraction(wv[n, k]) * Fraction(2) ** (int(ws[n, k // 32]) - 127))
                exact += t
                sabs += abs(t)
            assert abs(Fraction(r.ref[m, n]) - exact) <= sabs * Fraction(2) ** -50
            assert Fraction(r.absref[m, n]) == sabs or abs(Fraction(r.absref[m, n]) - sabs) <= sabs * Fraction(2) ** -50
            assert r.bf16[m, n] == _bf16_rne(exact)


def test_matches_numpy_fp64_matmul():
    rng = np.random.default_rng(11)
    M, N, K = 5, 37, 256
    aq, as_ = _random_mx(rng, M, K)
    wq, ws = _random_mx(rng, N, K)
    r = oracle.gemm(aq, as_, wq, ws)
    A = _torch_dequant(aq, as_); W = _torch_dequant(wq, ws)
    ref = A @ W.T
    assert np.all(np.abs(r.ref - ref) <= 1e-12 * np.abs(A) @ np.abs(W).T)
    assert np.allclose(r.absref, np.abs(A) @ np.abs(W).T, rtol=1e-12, atol=0)


def test_linearity_in_block_scale_exponent():
    rng = np.random.default_rng(5)
    M, N, K = 3, 4, 128
    aq, as_ = _random_mx(rng, M, K)
    wq, ws = _random_mx(rng, N, K)
    r0 = oracle.gemm(aq, as_, wq, ws)
    base = r0.ref
    for blk, d in ((0, 3), (2, -4), (3, 1)):
        only = aq.copy()
        mask = np.ones(K, dtype=bool); mask[blk * 32:(blk + 1) * 32] = False
        only[:, mask] = 0
        part = oracle.gemm(only, as_, wq, ws).ref
        s2 = as_.astype(np.int64); s2[:, blk] += d; s2 = s2.astype(np.uint8)
        r1 = oracle.gemm(aq, s2, wq, ws)
        # exact up to fp64 summation error, which is bounded by the abs-sums
        bound = 2.0 ** -44 * (r0.absref + r1.absref)
        assert np.all(np.abs((r1.ref - base) - (2.0 ** d - 1) * part) <= bound)
        assert np.any(np.abs(part) > 1e3 * bound), "the test must be able to fail"


def test_one_hot_weights_exact():
    rng = np.random.default_rng(9)
    M, N, K = 4, 16, 256
    aq, as_ = _random_mx(rng, M, K)
    kn = rng.integers(0, K, N)
    wq = np.zeros((N, K), dtype=np.uint8); wq[np.arange(N), kn] = 0x38   # 1.0
    ws = np.full((N, K // 32), 127, dtype=np.uint8)
    r = oracle.gemm(aq, as_, wq, ws)
    A = _torch_dequant(aq, as_)
    want = A[:, kn] + 0.0     # exact in BF16 (4 significant bits); a sum of -0 is +0
    want_bits = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(r.ref, want)
    assert np.array_equal(r.bf16, want_bits)


def test_zero_input_gives_positive_zero():
    rng = np.random.default_rng(4)
    wq, ws = _random_mx(rng, 8, 128)
    r = oracle.gemm(np.zeros((2, 128), np.uint8), np.zeros((2, 4), np.uint8), wq, ws)
    assert not r.bf16.any() and not r.ref.any() and not np.signbit(r.ref).any()


def test_operands_not_transposed():
    # A shape-asymmetric case: out[m, n] must pair row m of a with row n of w.
    aq = np.zeros((2, 32), np.uint8); aq[0, 0] = 0x38; aq[1, 1] = 0x40   # a0 = e0, a1 = 2 e1
    wq = np.zeros((3, 32), np.uint8); wq[0, 1] = 0x38; wq[2, 0] = 0x48   # w0 = e1, w2 = 4 e0
    ones = lambda r: np.full((r, 1), 127, np.uint8)
    r = oracle.gemm(aq, ones(2), wq, ones(3))
    assert r.ref.tolist() == [[0.0, 0.0, 4.0], [2.0, 0.0, 0.0]]
