"""Build libmxgemm.so (the GEMM library) and libmxprobe.so (the HBM read
probe, a measurement aid) in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
PROBE_SRC = os.path.join(PKG, "probe_src")
LIB = os.path.join(PKG, "libmxgemm.so")
PROBE_LIB = os.path.join(PKG, "libmxprobe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every floating-point operation rounds on its own (the rotary step's
    # precision is fixed that way), and no packed-FP32 instructions are emitted
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    """The HIP sources and the plain C++ host sources (argument checks)."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def _hipcc(srcs: list[str], includes: list[str], out: str, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, *("-I" + d for d in includes), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libmxgemm.so, and the probe into
    libmxprobe.so (always rebuilds both)."""
    _hipcc(sources(), [INCLUDE, CSRC], LIB, verbose)
    _hipcc(sorted(glob.glob(os.path.join(PROBE_SRC, "*.hip"))), [INCLUDE, CSRC, PROBE_SRC],
           PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
