"""Shared test helpers: host <-> device conversion and the tolerance check.

The tolerance on a BF16 GEMM output element is |gpu - ref| <= 2^-7 * sum_k
|a_k w_k| + 1e-6, with ref the oracle's unrounded fp64 sum: it covers the
output's BF16 rounding (2^-9 relative) and the FP32 accumulation inside and
across the scaled MFMAs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth


def say(*args) -> None:
    """Name the case about to run on the GPU (flushed, so it survives a crash)."""
    print(*args, flush=True)
    sys.stdout.flush()


def dev_u8(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return synth.from_bits(bits).to(device)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return synth.bits(t.detach().cpu())


def check_gemm(out: torch.Tensor, ref: "oracle.GemmResult", what: str = "") -> float:
    """Assert every element is within tolerance; return max |err| / tol."""
    got = oracle.bf16_value(host_bits(out))
    assert got.shape == ref.ref.shape, (got.shape, ref.ref.shape)
    err = np.abs(got - ref.ref)
    tol = ref.tolerance()
    ratio = float(np.max(err / tol)) if err.size else 0.0
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, first {bad[:5].tolist()}, "
                           f"gpu {got[tuple(bad[0])]}, ref {ref.ref[tuple(bad[0])]}, tol {tol[tuple(bad[0])]}")
    assert np.isfinite(got).all()
    return ratio
