"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and rounds them to BF16 (the activation
dtype); it holds none of the method's arithmetic (no quantization, no GEMM, no
rotary).  Every draw uses a CPU ``torch.Generator`` seeded explicitly, in a
fixed order per workload, so that both sides see identical inputs.

Recipes (the pages print no workloads; these follow the benchmark's
definition of the decode projections):
  * activations x ~ N(0, 1), weights W ~ N(0, 0.02), drawn in FP32 and rounded
    once to BF16;
  * outlier variant: a Bernoulli(0.01) mask, drawn after x and W, multiplies
    the matching x entries by 100 in FP32 before the BF16 rounding;
  * RMSNorm + requantize: rows x ~ N(0, 1) (optionally the leading K columns
    of wider rows, as the chain's A output), a per-column gain
    w = 1 + 0.1 * N(0, 1), eps = 1e-6 (the pages give none of these);
  * WO-A: attention output o ~ N(0, 1) of shape [M, 64 heads, 512], positions
    uniform in [0, 65536), and the rotary table cos/sin(pos * 10000^(-2i/64))
    for i = 0..31, computed in fp64 and rounded to FP32 (an input table, like
    the layer's cos_sin_cache).
BF16 tensors are returned as torch.bfloat16 CPU tensors; ``bits()`` gives the
uint16 view as a numpy array.
"""
from __future__ import annotations

import numpy as np
import torch

ROPE_BASE = 10000.0
MAX_POS = 65536


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _normal(g: torch.Generator, shape, std: float) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a BF16 tensor (a copy on the host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def from_bits(b: np.ndarray) -> torch.Tensor:
    """BF16 tensor with the given uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


def gemm_case(M: int, N: int, K: int, seed: int = 0, outliers: bool = False):
    """x [M, K] and W [N, K] in BF16; draw order x, W, then the outlier mask."""
    g = _gen(seed)
    x = _normal(g, (M, K), 1.0)
    w = _normal(g, (N, K), 0.02)
    if outliers:
        mask = torch.rand(M, K, generator=g) < 0.01
        x = torch.where(mask, x * 100.0, x)
    return {"x": x.to(torch.bfloat16), "w": w.to(torch.bfloat16)}


RMSNORM_EPS = 1e-6


def rmsnorm_case(M: int, K: int, seed: int = 0, ld: int | None = None, outliers: bool = False):
    """x [M, ld] (the leading K columns are normalised) and gain w [K] in BF16;
    draw order x, w, then the outlier mask (x100 on 1 % of x's entries)."""
    ld = K if ld is None else ld
    g = _gen(seed)
    x = _normal(g, (M, ld), 1.0)
    w = 1.0 + _normal(g, (K,), 0.1)
    if outliers:
        mask = torch.rand(M, ld, generator=g) < 0.01
        x = torch.where(mask, x * 100.0, x)
    return {"x": x.to(torch.bfloat16), "w": w.to(torch.bfloat16), "eps": RMSNORM_EPS}


CHAIN_DIMS = {"A": (2048, 5120), "B": (8192, 1536), "C": (5120, 8192)}
CHAIN_REQUANT_COLS = 1536


def chain_case(M: int, seed: int = 0, dims=None):
    """Three-projection chain inputs; draw order x_A, W_A, W_B, x_C, W_C.

    ``dims`` maps stage -> (N, K); stage B's K is the requantized width."""
    d = dict(CHAIN_DIMS if dims is None else dims)
    g = _gen(seed)
    xa = _normal(g, (M, d["A"][1]), 1.0)
    wa = _normal(g, d["A"], 0.02)
    wb = _normal(g, d["B"], 0.02)
    xc = _normal(g, (M, d["C"][1]), 1.0)
    wc = _normal(g, d["C"], 0.02)
    bf = torch.bfloat16
    return {"x_a": xa.to(bf), "w_a": wa.to(bf), "w_b": wb.to(bf),
            "x_c": xc.to(bf), "w_c": wc.to(bf), "dims": d}


def rope_table(rope_dim: int = 64, max_pos: int = MAX_POS, base: float = ROPE_BASE):
    """FP32 [max_pos, rope_dim]: cos(theta_i) for i < rope_dim/2, then sin."""
    half = rope_dim // 2
    inv = base ** (-np.arange(0, rope_dim, 2, dtype=np.float64) / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :half]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


WO_A_DIMS = dict(n_heads=64, head_dim=512, nope=448, n_groups=8, rank=1024, n_out=5120)


def wo_a_case(M: int, seed: int = 0, dims=None, max_pos: int = MAX_POS):
    """WO-A + wo_b inputs; draw order o, positions, W_a, W_b."""
    d = dict(WO_A_DIMS if dims is None else dims)
    H, D, G, R = d["n_heads"], d["head_dim"], d["n_groups"], d["rank"]
    g = _gen(seed)
    o = _normal(g, (M, H, D), 1.0)
    pos = torch.randint(0, max_pos, (M,), generator=g, dtype=torch.int64)
    w_a = _normal(g, (G, R, (H // G) * D), 0.02)
    w_b = _normal(g, (d["n_out"], G * R), 0.02)
    bf = torch.bfloat16
    return {"o": o.to(bf), "positions": pos, "w_a": w_a.to(bf), "w_b": w_b.to(bf),
            "cos_sin": rope_table(D - d["nope"], max_pos), "dims": d}
