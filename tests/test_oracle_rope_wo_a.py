"""Pins of the oracle's rotary step and of the WO-A -> wo_b composition:
position 0 is the identity, the rotation agrees with complex multiplication
(an independent formula) to within BF16/FP32 rounding, pair norms are kept,
and with position 0 WO-A equals one ungrouped GEMM against the
block-diagonal weight (which pins the head -> group -> weight indexing)."""
import numpy as np
import pytest

import oracle
import synth


def test_rope_table_basics():
    cs = synth.rope_table(64, 4096)
    assert cs.shape == (4096, 64) and cs.dtype == np.float32
    assert (cs[0, :32] == 1).all() and (cs[0, 32:] == 0).all()
    assert np.allclose(cs[:, :32].astype(np.float64) ** 2 + cs[:, 32:].astype(np.float64) ** 2, 1, atol=1e-6)
    # theta_1 at position 1 is 10000^(-2/64)
    assert abs(np.arctan2(cs[1, 33], cs[1, 1]) - 10000.0 ** (-2 / 64)) < 1e-6


def _case(M=3, H=4, D=64, nope=32, seed=0, max_pos=512):
    rng = np.random.default_rng(seed)
    o = oracle.bf16_round(rng.standard_normal((M, H, D)))
    pos = rng.integers(0, max_pos, M).astype(np.int64)
    return o, pos, synth.rope_table(D - nope, max_pos)


def test_rope_position_zero_is_identity():
    o, pos, cs = _case()
    y = oracle.rope(o, np.zeros_like(pos), cs, 32)
    assert np.array_equal(y, o)


def test_rope_matches_complex_rotation():
    o, pos, cs = _case(M=5, H=3, D=128, nope=64, seed=2, max_pos=65536)
    y = oracle.rope(o, pos, cs, 64)
    assert np.array_equal(y[..., :64], o[..., :64]), "nope dims pass through"
    x = oracle.bf16_value(o[..., 64:])
    z = x[..., 0::2] + 1j * x[..., 1::2]                 # adjacent pairs
    c = cs[pos, :32].astype(np.float64); s = cs[pos, 32:].astype(np.float64)
    rot = z * (c + 1j * s)[:, None, :]                     # forward rotation
    yv = oracle.bf16_value(y[..., 64:])
    mag = np.abs(z)[..., None].repeat(2, -1).reshape(yv.shape)
    want = np.stack([rot.real, rot.imag], -1).reshape(yv.shape)
    assert np.all(np.abs(yv - want) <= 2.0 ** -8 * mag + 1e-30)
    # the pair's norm is kept to within BF16 rounding
    ny = np.hypot(yv[..., 0::2], yv[..., 1::2])
    assert np.allclose(ny, np.abs(z), rtol=2.0 ** -7, atol=0)


def test_rope_wrong_conventions_would_fail():
    # The half-split (neox) pairing or the inverse rotation gives a different
    # result, so the comparison above does distinguish the conventions.
    o, pos, cs = _case(M=2, H=1, D=64, nope=32, seed=4, max_pos=65536)
    pos[:] = [1234, 40000]
    y = oracle.bf16_value(oracle.rope(o, pos, cs, 32)[..., 32:])
    x = oracle.bf16_value(o[..., 32:])
    c = cs[pos, :16].astype(np.float64)[:, None, :]; s = cs[pos, 16:].astype(np.float64)[:, None, :]
    inv = np.stack([x[..., 0::2] * c + x[..., 1::2] * s, x[..., 1::2] * c - x[..., 0::2] * s], -1).reshape(x.shape)
    neox = np.concatenate([x[..., :16] * c - x[..., 16:] * s, x[..., 16:] * c + x[..., :16] * s], -1)
    assert np.abs(y - inv).max() > 0.1 and np.abs(y - neox).max() > 0.1


def _wo_a_small(M=3, H=4, D=64, nope=32, G=2, R=64, N=96, seed=0, zero_pos=False):
    rng = np.random.default_rng(seed)
    o = oracle.bf16_round(rng.standard_normal((M, H, D)))
    pos = np.zeros(M, np.int64) if zero_pos else rng.integers(0, 4096, M).astype(np.int64)
    cs = synth.rope_table(D - nope, 4096)
    Kg = (H // G) * D
    wa = oracle.bf16_round(rng.standard_normal((G * R, Kg)) * 0.02)
    wa_q, wa_s = oracle.quantize(wa)
    wb_q, wb_s = oracle.quantize(oracle.bf16_round(rng.standard_normal((N, G * R)) * 0.02))
    return o, pos, cs, wa_q.reshape(G, R, Kg), wa_s.reshape(G, R, Kg // 32), (wb_q, wb_s)


def test_wo_a_position_zero_equals_block_diagonal_gemm():
    M, H, D, G, R = 3, 4, 64, 2, 64
    o, pos, cs, wa_q, wa_s, wb = _wo_a_small(M, H, D, 32, G, R, zero_pos=True)
    res = oracle.wo_a(o, pos, cs, wa_q, wa_s, wb, nope=32, n_groups=G)
    Kg = (H // G) * D
    # one ungrouped GEMM: x [M, H*D] against the block-diagonal [G*R, H*D] weight
    x_q, x_s = oracle.quantize(o.reshape(M, H * D))
    bq = np.zeros((G * R, H * D), np.uint8)
    bs = np.zeros((G * R, H * D // 32), np.uint8)
    for g in range(G):
        bq[g * R:(g + 1) * R, g * Kg:(g + 1) * Kg] = wa_q[g]
        bs[g * R:(g + 1) * R, g * Kg // 32:(g + 1) * Kg // 32] = wa_s[g]
    full = oracle.gemm(x_q, x_s, bq, bs)
    assert np.array_equal(res.z_bf16, full.bf16)
    zq, zs = oracle.quantize(full.bf16)
    assert np.array_equal(res.z_q, zq) and np.array_equal(res.z_s, zs)
    assert np.array_equal(res.out.bf16, oracle.gemm(zq, zs, *wb).bf16)


def test_wo_a_groups_follow_heads():
    # Zeroing every head of group 1 zeroes exactly z's group-1 columns.
    M, H, D, G, R = 2, 4, 64, 2, 64
    o, pos, cs, wa_q, wa_s, wb = _wo_a_small(M, H, D, 32, G, R, seed=3)
    o[:, 2:, :] = 0
    res = oracle.wo_a(o, pos, cs, wa_q, wa_s, None, nope=32, n_groups=G)
    assert not res.z_bf16[:, R:].any()
    assert res.z_bf16[:, :R].any()
