"""CPU oracle for the MXFP8 block-scaled GEMM path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``mxfp8_block_scaled_gemm_amd``) and never imports it; the product path never
imports this.

The arithmetic lives in ``mxoracle.c`` (plain C, fp64 for real numbers, each
function citing the passage it follows).  This module builds that file with
gcc on first use, wraps it with ctypes over numpy arrays, and composes the
multi-stage paths (the three-projection chain and WO-A -> wo_b) from the
single-stage functions, in the order the pages give.

Sources ("pages"): vLLM API documentation pages for
``vllm.models.deepseek_v41.nvidia.specialized_decode.attention.mxfp8`` ([mxfp8]),
``...attention.step`` ([step]), ``vllm.models.deepseek_v41.nvidia.ops.cute_dsl``
([cute]) and ``vllm.models.deepseek_v41.nvidia.ops.o_proj`` ([o_proj]).

Parity unpinned (the pages show no outputs to compare against, and print
neither formula nor layout): fidelity to the real model's rotary convention,
to the scale rule its quantizer used, to its RMSNorm rounding, and to the byte
order of its F8_128x4 scales.  Each function here is pinned to what its own
definition fixes (tests/test_oracle_*.py, tests/golden/).

Array conventions: BF16 tensors are numpy ``uint16`` bit patterns, E4M3 codes and
E8M0 scale bytes are ``uint8``; everything is row-major and C-contiguous unless a
row stride is passed.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxoracle.c")
_LIB = os.path.join(_HERE, "libmxoracle.so")
# MXG_ORACLE_SANITIZE=1: load a build of the same source with AddressSanitizer
# and UndefinedBehaviorSanitizer (the process must have the ASan runtime
# preloaded; tests/test_sanitizers.py runs the oracle tests that way).
_SAN = os.environ.get("MXG_ORACLE_SANITIZE") == "1"
_LIB_SAN = os.path.join(_HERE, "libmxoracle_san.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile mxoracle.c into libmxoracle.so (gcc, OpenMP, no FP contraction),
    or with sanitize into libmxoracle_san.so with ASan and UBSan (any UB report
    aborts)."""
    out = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp%d" % os.getpid()
        flags = ["-O2"]
        if sanitize:
            flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                     "-fno-sanitize-recover=all"]
        subprocess.check_call(
            ["gcc", *flags, "-std=c11", "-fPIC", "-shared", "-fopenmp",
             "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build(sanitize=_SAN))
            u8p = ctypes.POINTER(ctypes.c_uint8)
            u16p = ctypes.POINTER(ctypes.c_uint16)
            f64p = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
            lib.orc_e4m3_value.restype = ctypes.c_double
            lib.orc_e8m0_value.argtypes = [ctypes.c_uint8]
            lib.orc_e8m0_value.restype = ctypes.c_double
            lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
            lib.orc_e4m3_encode.restype = ctypes.c_uint8
            lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
            lib.orc_bf16_value.restype = ctypes.c_double
            lib.orc_bf16_round.argtypes = [ctypes.c_double]
            lib.orc_bf16_round.restype = ctypes.c_uint16
            lib.orc_block_exponent.argtypes = [ctypes.c_double]
            lib.orc_block_exponent.restype = ctypes.c_int
            lib.orc_quantize.argtypes = [u16p, i64, i64, i64, u8p, u8p]
            lib.orc_quantize.restype = ctypes.c_int
            lib.orc_gemm.argtypes = [i64, i64, i64, u8p, u8p, u8p, u8p, f64p, f64p, u16p]
            lib.orc_gemm.restype = ctypes.c_int
            lib.orc_rope.argtypes = [u16p, i64, i64, i64, i64, i64, i64,
                                     ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_float), i64, u16p]
            lib.orc_rope.restype = ctypes.c_int
            lib.orc_rmsnorm.argtypes = [u16p, i64, i64, i64, u16p, ctypes.c_double, f64p]
            lib.orc_rmsnorm.restype = ctypes.c_int
            lib.orc_set_threads.argtypes = [ctypes.c_int]
            lib.orc_set_threads.restype = None
            lib.orc_num_threads.argtypes = []
            lib.orc_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


# ------------------------------------------------------------------ formats

def e4m3_value(codes) -> np.ndarray:
    """fp64 value of each E4M3 code (NaN for 0x7F / 0xFF)."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e4m3_value(int(v)) for v in c.ravel()]).reshape(c.shape)


def e8m0_value(codes) -> np.ndarray:
    """fp64 value 2^(c-127) of each E8M0 scale byte (NaN for 0xFF)."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e8m0_value(int(v)) for v in c.ravel()]).reshape(c.shape)


def e4m3_encode(values) -> np.ndarray:
    """Nearest E4M3 code (ties to even, saturating at +-448) of each fp64 value."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    return np.array([lib.orc_e4m3_encode(float(x)) for x in v.ravel()],
                    dtype=np.uint8).reshape(v.shape)


def bf16_value(bits) -> np.ndarray:
    """Exact fp64 value of BF16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round(values) -> np.ndarray:
    """BF16 bits of the nearest BF16 value (ties to even) of each fp64 value."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    return np.array([lib.orc_bf16_round(float(x)) for x in v.ravel()],
                    dtype=np.uint16).reshape(v.shape)


def block_exponent(amax: float) -> int:
    """Scale exponent e (scale 2^e, byte e + 127) of a block with this amax."""
    return int(_load().orc_block_exponent(float(amax)))


# ---------------------------------------------------------------- quantizer

def quantize(x_bf16: np.ndarray, K: int | None = None, ld: int | None = None):
    """MXFP8 quantize of BF16 rows (per-32 E8M0 scale, E4M3 codes).

    ``x_bf16``: uint16 [M, >=K]; columns [0, K) of each row are quantized (the
    chain requantizes a leading column range).  Returns (codes [M, K] uint8,
    scales [M, K/32] uint8).
    """
    x = np.asarray(x_bf16)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError("x_bf16 must be a 2-D uint16 array")
    M = x.shape[0]
    K = x.shape[1] if K is None else K
    x = np.ascontiguousarray(x)
    ld = x.shape[1]
    q = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros((M, K // 32), dtype=np.uint8)
    rc = _load().orc_quantize(_ptr(x, ctypes.c_uint16), M, K, ld,
                              _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("orc_quantize rejected the input (K % 32 or non-finite)")
    return q, s


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp64 values of an MXFP8 tensor: code value times its block scale."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    table = e4m3_value(np.arange(256, dtype=np.uint8))
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)
    return table[q] * np.repeat(scale, 32, axis=-1)


# --------------------------------------------------------------------- GEMM

class GemmResult:
    """fp64 sum (ref), sum of |a*w| (absref) and BF16 bits of RNE(ref) (bf16)."""

    def __init__(self, ref, absref, bf16):
        self.ref, self.absref, self.bf16 = ref, absref, bf16

    def tolerance(self) -> np.ndarray:
        """Per-element bound 2^-7 * sum|a_k w_k| + 1e-6 on |gpu - ref|."""
        return np.ldexp(self.absref, -7) + 1e-6


def gemm(a_q, a_s, w_q, w_s) -> GemmResult:
    """out = dequant(a) . dequant(w)^T summed in fp64 ([mxfp8] launch_low_latency)."""
    a_q = _c(a_q, np.uint8); a_s = _c(a_s, np.uint8)
    w_q = _c(w_q, np.uint8); w_s = _c(w_s, np.uint8)
    M, K = a_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K or a_s.shape != (M, K // 32) or w_s.shape != (N, K // 32):
        raise ValueError("inconsistent MXFP8 operand shapes")
    ref = np.zeros((M, N)); absref = np.zeros((M, N))
    out = np.zeros((M, N), dtype=np.uint16)
    rc = _load().orc_gemm(M, N, K, _ptr(a_q, ctypes.c_uint8), _ptr(a_s, ctypes.c_uint8),
                          _ptr(w_q, ctypes.c_uint8), _ptr(w_s, ctypes.c_uint8),
                          _ptr(ref, ctypes.c_double), _ptr(absref, ctypes.c_double),
                          _ptr(out, ctypes.c_uint16))
    if rc != 0:
        raise RuntimeError(f"orc_gemm failed ({rc})")
    return GemmResult(ref, absref, out)


def set_threads(n: int) -> int:
    """Set the oracle GEMM's OpenMP thread count; returns the count in effect."""
    lib = _load()
    lib.orc_set_threads(int(n))
    return int(lib.orc_num_threads())


# --------------------------------------------------------------------- RoPE

def rope(o_bf16: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray,
         nope: int) -> np.ndarray:
    """Rotary embedding of the last (D - nope) dims of each head, BF16 out.

    ``o_bf16``: uint16 [M, H, D] (any row/head stride, D contiguous);
    ``positions``: int64 [M]; ``cos_sin``: float32 [max_pos, D - nope].
    Convention and precision readings are stated in mxoracle.c (orc_rope).
    """
    o = np.asarray(o_bf16)
    if o.dtype != np.uint16 or o.ndim != 3 or o.strides[2] != 2:
        raise TypeError("o_bf16 must be uint16 [M, H, D] with D contiguous")
    M, H, D = o.shape
    pos = _c(positions, np.int64)
    cs = _c(cos_sin, np.float32)
    y = np.zeros((M, H, D), dtype=np.uint16)
    rc = _load().orc_rope(
        o.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), M, H, D,
        o.strides[0] // 2, o.strides[1] // 2, nope,
        _ptr(pos, ctypes.c_int64), _ptr(cs, ctypes.c_float), cs.shape[0],
        _ptr(y, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("orc_rope rejected the input")
    return y


# ----------------------------------------------------------------- RMSNorm

def rmsnorm(x_bf16: np.ndarray, w_bf16: np.ndarray, eps: float, K: int | None = None):
    """Unrounded fp64 RMSNorm of the leading K columns of BF16 rows:
    y = x * w / sqrt(mean(x^2) + eps) (the normalisation [step]
    _split_qkv_and_norm and [cute] AllReduceMHC apply before an MXFP8
    quantize).  ``x_bf16``: uint16 [M, >=K]; ``w_bf16``: uint16 [K]."""
    x = np.ascontiguousarray(np.asarray(x_bf16))
    w = np.ascontiguousarray(np.asarray(w_bf16))
    if x.dtype != np.uint16 or x.ndim != 2 or w.dtype != np.uint16:
        raise TypeError("x_bf16 and w_bf16 must be uint16 arrays")
    M = x.shape[0]
    K = x.shape[1] if K is None else K
    if w.shape != (K,):
        raise ValueError("w_bf16 must hold K values")
    y = np.zeros((M, K), dtype=np.float64)
    rc = _load().orc_rmsnorm(_ptr(x, ctypes.c_uint16), M, K, x.shape[1],
                             _ptr(w, ctypes.c_uint16), float(eps), _ptr(y, ctypes.c_double))
    if rc != 0:
        raise ValueError("orc_rmsnorm rejected the input")
    return y


def rmsnorm_quantize(x_bf16: np.ndarray, w_bf16: np.ndarray, eps: float, K: int | None = None):
    """RMSNorm rounded once to BF16, then the MXFP8 quantize of that BF16
    tensor (every inter-stage tensor is BF16 before it is requantized).
    Returns (y fp64 unrounded, y BF16 bits, codes, scales)."""
    y = rmsnorm(x_bf16, w_bf16, eps, K)
    yb = bf16_round(y)
    q, s = quantize(yb)
    return y, yb, q, s


def rmsnorm_tolerance(y_ref: np.ndarray, K: int) -> np.ndarray:
    """Bound on |BF16 result - exact value| for an FP32 evaluation of the
    RMSNorm (sum of K squares in any order, a division, a square root, a
    reciprocal, two products) rounded once to BF16: half a BF16 ulp (BF16
    keeps 8 significant bits, so 2^-8 relative at most) plus (K/2 + 4) units
    of FP32 rounding (2^-24 relative), plus the smallest BF16 subnormal step
    for results near zero."""
    return (2.0 ** -8 + (K / 2 + 4) * 2.0 ** -24) * np.abs(y_ref) + 2.0 ** -133


# ------------------------------------------------------- 128 x 4 scale tiles

def scales_to_128x4(s: np.ndarray) -> np.ndarray:
    """Row-major scale bytes [M, KB] (KB % 4 == 0) laid out in 128 x 4 tiles
    (the F8_128x4 activation scales the [mxfp8] page's low-latency GEMM
    reads; the pages do not print the layout): rows are padded to a multiple
    of 128 and scale columns taken 4 at a time; tiles run along the columns
    first, 512 bytes each; inside a tile, row r and column c sit at byte
    (r % 32) * 16 + (r // 32) * 4 + c.  Padding bytes are 0.  Returns the
    flat uint8 buffer.  Written as plain loops over the definition."""
    s = np.asarray(s, dtype=np.uint8)
    M, KB = s.shape
    if KB % 4:
        raise ValueError("the scale column count must be a multiple of 4")
    row_tiles, col_tiles = (M + 127) // 128, KB // 4
    out = np.zeros(row_tiles * col_tiles * 512, dtype=np.uint8)
    for m in range(M):
        for b in range(KB):
            tile = (m // 128) * col_tiles + b // 4
            r, c = m % 128, b % 4
            out[tile * 512 + (r % 32) * 16 + (r // 32) * 4 + c] = s[m, b]
    return out


# ------------------------------------------------------------ compositions

def linear_bf16(x_bf16: np.ndarray, w_q: np.ndarray, w_s: np.ndarray):
    """One MXFP8 projection of a BF16 input: quantize x, then the GEMM.

    Returns (x codes, x scales, GemmResult)."""
    q, s = quantize(x_bf16)
    return q, s, gemm(q, s, w_q, w_s)


class ChainResult:
    """Stage results of the three-projection chain (see ``chain``)."""

    def __init__(self, A, b_q, b_s, B, C):
        self.A, self.b_q, self.b_s, self.B, self.C = A, b_q, b_s, B, C


def chain(a_q, a_s, wA, b_cols: int, wB, c_q, c_s, wC, norm=None) -> ChainResult:
    """Back-to-back projections in the decode step's order ([step]
    AttentionStep.run: fused_wqa_wkv on the MXFP8 layer input, its leading
    columns requantized to MXFP8 for wq_b, and wo_b on its own MXFP8 input).

    A = gemm(a, wA) -> BF16; B's input = quantize(A.bf16[:, :b_cols]), or with
    ``norm = (gain BF16 bits [b_cols], eps)`` the quantize of the BF16
    RMSNorm of those columns (_split_qkv_and_norm); B = gemm(that, wB);
    C = gemm(c, wC) on C's own (fresh) MXFP8 input.  ``wX`` are (codes,
    scales) pairs.
    """
    A = gemm(a_q, a_s, *wA)
    lead = np.ascontiguousarray(A.bf16[:, :b_cols])
    if norm is None:
        b_q, b_s = quantize(lead)
    else:
        _, _, b_q, b_s = rmsnorm_quantize(lead, norm[0], norm[1])
    B = gemm(b_q, b_s, *wB)
    C = gemm(c_q, c_s, *wC)
    return ChainResult(A, b_q, b_s, B, C)


class WoAResult:
    """Intermediates and output of WO-A followed by wo_b (see ``wo_a``)."""

    def __init__(self, roped, xg_q, xg_s, groups, z_bf16, z_q, z_s, out):
        self.roped, self.xg_q, self.xg_s, self.groups = roped, xg_q, xg_s, groups
        self.z_bf16, self.z_q, self.z_s, self.out = z_bf16, z_q, z_s, out


def wo_a(o_bf16, positions, cos_sin, wa_q, wa_s, wb=None, *, nope: int = 448,
         n_groups: int = 8) -> WoAResult:
    """Grouped WO-A projection with rotary in front, then MXFP8 of its output
    and optionally wo_b ([o_proj] dsv41_o_proj: rotary on each head's rope
    dims, grouped FP8 per-32 projection, BF16 z flattened over groups, wo_b on
    the MXFP8 of z).

    ``o_bf16``: uint16 [M, H, D]; ``wa_q``: [G, R, (H/G)*D]; ``wa_s``:
    [G, R, (H/G)*D/32]; ``wb``: optional (codes, scales) of wo_b [N, G*R].
    Readings: each inter-stage tensor is BF16 before it is requantized (the
    unfused path materialises BF16); WO-A's activation and weight scales are
    E8M0 per 32, like every other MXFP8 operand here.
    """
    o = np.asarray(o_bf16)
    M, H, D = o.shape
    G = n_groups
    hpg = H // G
    roped = rope(o, positions, cos_sin, nope)             # [M, H, D]
    xg = roped.reshape(M, G, hpg * D)                     # group g = heads g*hpg ..
    groups, xg_q, xg_s = [], [], []
    for g in range(G):
        q, s = quantize(np.ascontiguousarray(xg[:, g, :]))
        xg_q.append(q); xg_s.append(s)
        groups.append(gemm(q, s, wa_q[g], wa_s[g]))
    z_bf16 = np.concatenate([r.bf16 for r in groups], axis=1)   # [M, G*R]
    z_q, z_s = quantize(z_bf16)
    out = gemm(z_q, z_s, *wb) if wb is not None else None
    return WoAResult(roped, xg_q, xg_s, groups, z_bf16, z_q, z_s, out)
