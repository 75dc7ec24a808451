"""Python binding of libmxgemm (small-row MXFP8 block-scaled GEMMs on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libmxgemm.so``.  Tensors are torch device tensors (torch supplies memory and
the current stream); BF16 data is ``torch.bfloat16``, E4M3 codes and UE8M0
scale bytes are ``torch.uint8``.  The functions carry the C names of
``include/mxgemm.h``; a non-zero status raises ``MxgError`` (a ValueError) with
the library's message.  There is no fallback: if the shared library is missing
the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxgemm.so")
MAX_ROWS = 48          # chain and WO-A (MXG_MAX_ROWS)
MAX_GEMM_ROWS = 256    # mxfp8_gemm / mxfp8_gemm_ex (MXG_MAX_GEMM_ROWS)
NOALLOC_SCRATCH_BYTES = 16 << 20   # mxfp8_gemm_noalloc's device scratch (MXG_NOALLOC_SCRATCH_BYTES)

_lib = None


class MxgWeight(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("layout", ctypes.c_int32)]


class MxgChain(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64),
                ("a_q", ctypes.c_void_p), ("a_s", ctypes.c_void_p),
                ("wA", MxgWeight), ("wB", MxgWeight), ("wC", MxgWeight),
                ("out_a", ctypes.c_void_p),
                ("b_q", ctypes.c_void_p), ("b_s", ctypes.c_void_p),
                ("out_b", ctypes.c_void_p),
                ("c_q", ctypes.c_void_p), ("c_s", ctypes.c_void_p),
                ("out_c", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("b_bf16", ctypes.c_void_p)]


class MxgWoA(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("o", ctypes.c_void_p),
                ("ld_row", ctypes.c_int64), ("ld_head", ctypes.c_int64),
                ("positions", ctypes.c_void_p), ("cos_sin", ctypes.c_void_p),
                ("max_pos", ctypes.c_int64),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("nope_dim", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("wa", MxgWeight), ("z", ctypes.c_void_p),
                ("z_q", ctypes.c_void_p), ("z_s", ctypes.c_void_p),
                ("wb", MxgWeight), ("out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class MxgError(ValueError):
    """A libmxgemm call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libmxgemm status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libmxgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mxfp8_block_scaled_gemm_amd._build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.mxg_strerror.argtypes = [ctypes.c_int]
        L.mxg_strerror.restype = ctypes.c_char_p
        L.mxg_version.argtypes = []
        L.mxg_version.restype = ctypes.c_int
        L.mxfp8_quantize.argtypes = [vp, i64, i64, i64, vp, vp, vp]
        L.mxfp8_quantize.restype = ctypes.c_int
        L.mxfp8_rmsnorm_quantize.argtypes = [vp, i64, i64, i64, vp, ctypes.c_float, vp, i64,
                                             vp, vp, ctypes.c_int32, vp]
        L.mxfp8_rmsnorm_quantize.restype = ctypes.c_int
        L.mxg_scale_bytes_128x4.argtypes = [i64, i64]
        L.mxg_scale_bytes_128x4.restype = sz
        L.mxfp8_pack_weights.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        L.mxfp8_pack_weights.restype = ctypes.c_int
        L.mxfp8_gemm.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.mxfp8_gemm.restype = ctypes.c_int
        L.mxfp8_gemm_noalloc.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, vp]
        L.mxfp8_gemm_noalloc.restype = ctypes.c_int
        L.mxfp8_gemm_ex.argtypes = [i64, i64, i64, vp, i64, vp, vp, ctypes.c_int32, vp, vp,
                                    ctypes.c_int32, vp, vp, sz, vp]
        L.mxfp8_gemm_ex.restype = ctypes.c_int
        L.mxg_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.mxg_gemm_workspace_bytes.restype = sz
        L.mxfp8_proj_chain.argtypes = [ctypes.POINTER(MxgChain), vp]
        L.mxfp8_proj_chain.restype = ctypes.c_int
        L.mxg_chain_workspace_bytes.argtypes = [ctypes.POINTER(MxgChain)]
        L.mxg_chain_workspace_bytes.restype = sz
        L.wo_a_fused_quantize.argtypes = [ctypes.POINTER(MxgWoA), vp]
        L.wo_a_fused_quantize.restype = ctypes.c_int
        L.mxg_wo_a_workspace_bytes.argtypes = [ctypes.POINTER(MxgWoA)]
        L.mxg_wo_a_workspace_bytes.restype = sz
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().mxg_strerror(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise MxgError(status, strerror(status))


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _expect(t: torch.Tensor, dtype: torch.dtype, name: str, shape=None) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype} CUDA/HIP tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_workspaces: dict = {}


def get_workspace(device, nbytes: int) -> torch.Tensor:
    """A zero-filled, per-device workspace of at least ``nbytes`` bytes.

    The library leaves a workspace zeroed after every call, so one buffer
    serves all calls issued on one stream; calls on different streams need
    workspaces of their own (pass ``workspace=``)."""
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    t = _workspaces.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.zeros(max(int(nbytes), 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = t
    return t


def workspace_error(ws: torch.Tensor) -> int:
    """The error word of a workspace (non-zero: an in-kernel wait expired, or
    for wo_a_fused_quantize bit 1: a position outside the angle table)."""
    return int(ws[20:24].view(torch.int32).item())


def mxfp8_quantize(x: torch.Tensor, K: int | None = None, q: torch.Tensor | None = None,
                   s: torch.Tensor | None = None, stream=None):
    """BF16 [M, >=K] (unit stride along K, any row stride) -> (codes [M, K],
    scales [M, K/32]).  Columns [0, K) are quantized (default: all)."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise TypeError("x must be a 2-D bfloat16 tensor with unit stride along K")
    M = x.shape[0]
    K = x.shape[1] if K is None else int(K)
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(M, K // 32, dtype=torch.uint8, device=x.device)
    _expect(q, torch.uint8, "q", (M, K))
    _expect(s, torch.uint8, "s", (M, K // 32))
    _check(lib().mxfp8_quantize(_ptr(x), M, K, x.stride(0), _ptr(q), _ptr(s), _stream(stream)))
    return q, s


SCALES_ROW_MAJOR = 0   # [M, K/32]
SCALES_128X4 = 1       # 128 x 4 scale tiles (mxg_scale_bytes_128x4 bytes)
WEIGHTS_PACKED = 0     # mxfp8_pack_weights order (MXG_WEIGHTS_PACKED)
WEIGHTS_ROW_MAJOR = 1  # [N, K] codes, [N, K/32] scales (MXG_WEIGHTS_ROW_MAJOR)


def scale_bytes_128x4(M: int, K: int) -> int:
    return int(lib().mxg_scale_bytes_128x4(M, K))


def mxfp8_rmsnorm_quantize(x: torch.Tensor, w: torch.Tensor, eps: float, K: int | None = None,
                           y: torch.Tensor | None = None, q: torch.Tensor | None = None,
                           s: torch.Tensor | None = None, scale_layout: int = SCALES_ROW_MAJOR,
                           write_y: bool = True, stream=None):
    """RMSNorm of the leading K columns of BF16 rows x [M, >=K] with gain w
    [K], then MXFP8 of the BF16 result.  Returns (y BF16 [M, K] or None,
    codes [M, K], scales): scales [M, K/32], or a flat zero-initialised
    buffer of scale_bytes_128x4(M, K) bytes in 128 x 4 tiles."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise TypeError("x must be a 2-D bfloat16 tensor with unit stride along K")
    M = x.shape[0]
    K = x.shape[1] if K is None else int(K)
    _expect(w, torch.bfloat16, "w", (K,))
    if write_y and y is None:
        y = torch.empty(M, K, dtype=torch.bfloat16, device=x.device)
    if y is not None and (y.dim() != 2 or y.dtype != torch.bfloat16 or y.stride(1) != 1 or
                          y.shape[0] != M or y.shape[1] < K or not y.is_cuda):
        raise TypeError("y must be a bfloat16 [M, >=K] tensor with unit stride along K")
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    _expect(q, torch.uint8, "q", (M, K))
    if s is None:
        if scale_layout == SCALES_128X4:
            s = torch.zeros(scale_bytes_128x4(M, K), dtype=torch.uint8, device=x.device)
        else:
            s = torch.empty(M, K // 32, dtype=torch.uint8, device=x.device)
    if scale_layout == SCALES_128X4:
        _expect(s, torch.uint8, "s")
        if s.numel() < scale_bytes_128x4(M, K):
            raise ValueError("s holds fewer than scale_bytes_128x4(M, K) bytes")
    else:
        _expect(s, torch.uint8, "s", (M, K // 32))
    _check(lib().mxfp8_rmsnorm_quantize(_ptr(x), M, K, x.stride(0), _ptr(w), float(eps), _ptr(y),
                                        y.stride(0) if y is not None else 0, _ptr(q), _ptr(s),
                                        int(scale_layout), _stream(stream)))
    return y, q, s


def mxfp8_pack_weights(w_q: torch.Tensor, w_s: torch.Tensor, wp_q: torch.Tensor | None = None,
                       wp_s: torch.Tensor | None = None, stream=None):
    """Repack a row-major MXFP8 weight ([N, K] codes, [N, K/32] scales) into
    the GEMM's streaming order; returns (wp_q [N*K], wp_s [N*K/32]) uint8."""
    N, K = w_q.shape
    _expect(w_q, torch.uint8, "w_q", (N, K))
    _expect(w_s, torch.uint8, "w_s", (N, K // 32))
    if wp_q is None:
        wp_q = torch.empty(N * K, dtype=torch.uint8, device=w_q.device)
    if wp_s is None:
        wp_s = torch.empty(N * K // 32, dtype=torch.uint8, device=w_q.device)
    _expect(wp_q, torch.uint8, "wp_q", (N * K,))
    _expect(wp_s, torch.uint8, "wp_s", (N * K // 32,))
    _check(lib().mxfp8_pack_weights(_ptr(w_q), _ptr(w_s), N, K, _ptr(wp_q), _ptr(wp_s),
                                    _stream(stream)))
    return wp_q, wp_s


class PackedWeight:
    """An MXFP8 weight in the GEMM's streaming order, with its shape."""

    layout = WEIGHTS_PACKED

    def __init__(self, q: torch.Tensor, s: torch.Tensor, N: int, K: int):
        self.q, self.s, self.N, self.K = q, s, N, K

    @classmethod
    def from_rows(cls, w_q: torch.Tensor, w_s: torch.Tensor, stream=None) -> "PackedWeight":
        q, s = mxfp8_pack_weights(w_q, w_s, stream=stream)
        return cls(q, s, w_q.shape[0], w_q.shape[1])

    @classmethod
    def from_bf16(cls, w: torch.Tensor, stream=None) -> "PackedWeight":
        """Quantize a BF16 [N, K] weight (same rule as the activations) and pack it."""
        q, s = mxfp8_quantize(w, stream=stream)
        return cls.from_rows(q, s, stream=stream)

    def clone(self) -> "PackedWeight":
        return PackedWeight(self.q.clone(), self.s.clone(), self.N, self.K)


class RowMajorWeight:
    """An MXFP8 weight as a layer holds it, [N, K] codes and [N, K/32] scale
    bytes, which the GEMMs read without a repack (slower to stream than a
    PackedWeight of the same values; results are equal bit for bit)."""

    layout = WEIGHTS_ROW_MAJOR

    def __init__(self, q: torch.Tensor, s: torch.Tensor):
        N, K = q.shape
        _expect(q, torch.uint8, "q", (N, K))
        _expect(s, torch.uint8, "s", (N, K // 32))
        self.q, self.s, self.N, self.K = q, s, N, K

    @classmethod
    def from_bf16(cls, w: torch.Tensor, stream=None) -> "RowMajorWeight":
        """Quantize a BF16 [N, K] weight (same rule as the activations)."""
        return cls(*mxfp8_quantize(w, stream=stream))

    def clone(self) -> "RowMajorWeight":
        return RowMajorWeight(self.q.clone(), self.s.clone())


# Either weight class: every GEMM entry takes both.
Weight = "PackedWeight | RowMajorWeight"


def _expect_weight(w: Weight) -> None:
    if w.layout == WEIGHTS_PACKED:
        _expect(w.q, torch.uint8, "w.q", (w.N * w.K,))
        _expect(w.s, torch.uint8, "w.s", (w.N * w.K // 32,))
    else:
        _expect(w.q, torch.uint8, "w.q", (w.N, w.K))
        _expect(w.s, torch.uint8, "w.s", (w.N, w.K // 32))


def mxfp8_gemm(a_q: torch.Tensor, a_s: torch.Tensor, w: Weight,
               out: torch.Tensor | None = None, x: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out[M, N] (BF16) = dequant(a) . dequant(w)^T for a PackedWeight or a
    RowMajorWeight w (the latter through the C call mxfp8_gemm_ex).

    With ``x`` (BF16 [M, >=K]) the kernel quantizes x itself and writes its
    codes/scales into ``a_q``/``a_s`` (which must then be allocated by the
    caller); otherwise ``a_q``/``a_s`` are the MXFP8 inputs."""
    if w.layout != WEIGHTS_PACKED:
        return mxfp8_gemm_ex(a_q, a_s, w, SCALES_ROW_MAJOR, out=out, x=x, workspace=workspace,
                             stream=stream)
    M, K = a_q.shape
    N = w.N
    if w.K != K:
        raise ValueError(f"weight K {w.K} != activation K {K}")
    _expect(a_q, torch.uint8, "a_q", (M, K))
    _expect(a_s, torch.uint8, "a_s", (M, K // 32))
    _expect_weight(w)
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=a_q.device)
    _expect(out, torch.bfloat16, "out", (M, N))
    ld_x = 0
    if x is not None:
        if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1 or x.shape[0] != M:
            raise TypeError("x must be a bfloat16 [M, >=K] tensor with unit stride along K")
        ld_x = x.stride(0)
    ws_bytes = int(lib().mxg_gemm_workspace_bytes(M, N, K))
    if workspace is None:
        workspace = get_workspace(a_q.device, ws_bytes)
    wsz = workspace.numel() * workspace.element_size()
    _check(lib().mxfp8_gemm(M, N, K, _ptr(x), ld_x, _ptr(a_q), _ptr(a_s), _ptr(w.q), _ptr(w.s),
                            _ptr(out), _ptr(workspace), wsz, _stream(stream)))
    return out


def mxfp8_gemm_noalloc(a_q: torch.Tensor, a_s: torch.Tensor, w: PackedWeight,
                       out: torch.Tensor | None = None, x: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """mxfp8_gemm without a workspace: the library keeps the K-split state in
    its own per-GPU device scratch (calls on one GPU must not overlap).  With
    ``out`` given, nothing is allocated on this path.  Packed weights only."""
    M, K = a_q.shape
    N = w.N
    if w.K != K:
        raise ValueError(f"weight K {w.K} != activation K {K}")
    if w.layout != WEIGHTS_PACKED:
        raise TypeError("mxfp8_gemm_noalloc takes a PackedWeight")
    _expect(a_q, torch.uint8, "a_q", (M, K))
    _expect(a_s, torch.uint8, "a_s", (M, K // 32))
    _expect_weight(w)
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=a_q.device)
    _expect(out, torch.bfloat16, "out", (M, N))
    ld_x = 0
    if x is not None:
        if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1 or x.shape[0] != M:
            raise TypeError("x must be a bfloat16 [M, >=K] tensor with unit stride along K")
        ld_x = x.stride(0)
    _check(lib().mxfp8_gemm_noalloc(M, N, K, _ptr(x), ld_x, _ptr(a_q), _ptr(a_s), _ptr(w.q),
                                    _ptr(w.s), _ptr(out), _stream(stream)))
    return out


def mxfp8_gemm_ex(a_q: torch.Tensor, a_s: torch.Tensor, w: Weight, a_scale_layout: int,
                  out: torch.Tensor | None = None, x: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mxfp8_gemm with the activation scales a_s row-major [M, K/32]
    (SCALES_ROW_MAJOR) or a flat buffer of scale_bytes_128x4(M, K) bytes in
    128 x 4 tiles (SCALES_128X4, MXFP8 input only), and the weight w a
    PackedWeight or a RowMajorWeight.  ``x`` as in mxfp8_gemm."""
    M, K = a_q.shape
    N = w.N
    if w.K != K:
        raise ValueError(f"weight K {w.K} != activation K {K}")
    _expect(a_q, torch.uint8, "a_q", (M, K))
    if a_scale_layout == SCALES_128X4:
        _expect(a_s, torch.uint8, "a_s")
        if a_s.numel() < scale_bytes_128x4(M, K):
            raise ValueError("a_s holds fewer than scale_bytes_128x4(M, K) bytes")
    else:
        _expect(a_s, torch.uint8, "a_s", (M, K // 32))
    _expect_weight(w)
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=a_q.device)
    _expect(out, torch.bfloat16, "out", (M, N))
    ld_x = 0
    if x is not None:
        if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1 or x.shape[0] != M:
            raise TypeError("x must be a bfloat16 [M, >=K] tensor with unit stride along K")
        ld_x = x.stride(0)
    ws_bytes = int(lib().mxg_gemm_workspace_bytes(M, N, K))
    if workspace is None:
        workspace = get_workspace(a_q.device, ws_bytes)
    wsz = workspace.numel() * workspace.element_size()
    _check(lib().mxfp8_gemm_ex(M, N, K, _ptr(x), ld_x, _ptr(a_q), _ptr(a_s), int(a_scale_layout),
                               _ptr(w.q), _ptr(w.s), int(w.layout), _ptr(out), _ptr(workspace),
                               wsz, _stream(stream)))
    return out


def _w(w: Weight) -> MxgWeight:
    _expect_weight(w)
    return MxgWeight(w.q.data_ptr(), w.s.data_ptr(), w.N, w.K, w.layout)


def mxfp8_proj_chain(a_q: torch.Tensor, a_s: torch.Tensor, wA: Weight, wB: Weight,
                     c_q: torch.Tensor, c_s: torch.Tensor, wC: Weight, outs=None,
                     workspace: torch.Tensor | None = None, norm_weight: torch.Tensor | None = None,
                     norm_eps: float = 0.0, b_bf16: torch.Tensor | None = None, stream=None):
    """Three projections back to back: A on (a_q, a_s); the leading wB.K
    columns of A's output (RMS-normalised with norm_weight / norm_eps when
    given, the normalised BF16 copied to b_bf16 when given) requantized to
    MXFP8 as B's input; C on (c_q, c_s).  Returns (out_a, b_q, b_s, out_b,
    out_c)."""
    M = a_q.shape[0]
    dev = a_q.device
    _expect(a_q, torch.uint8, "a_q", (M, wA.K))
    _expect(a_s, torch.uint8, "a_s", (M, wA.K // 32))
    _expect(c_q, torch.uint8, "c_q", (M, wC.K))
    _expect(c_s, torch.uint8, "c_s", (M, wC.K // 32))
    if outs is None:
        outs = (torch.empty(M, wA.N, dtype=torch.bfloat16, device=dev),
                torch.empty(M, wB.K, dtype=torch.uint8, device=dev),
                torch.empty(M, wB.K // 32, dtype=torch.uint8, device=dev),
                torch.empty(M, wB.N, dtype=torch.bfloat16, device=dev),
                torch.empty(M, wC.N, dtype=torch.bfloat16, device=dev))
    out_a, b_q, b_s, out_b, out_c = outs
    _expect(out_a, torch.bfloat16, "out_a", (M, wA.N))
    _expect(b_q, torch.uint8, "b_q", (M, wB.K))
    _expect(b_s, torch.uint8, "b_s", (M, wB.K // 32))
    _expect(out_b, torch.bfloat16, "out_b", (M, wB.N))
    _expect(out_c, torch.bfloat16, "out_c", (M, wC.N))
    if norm_weight is not None:
        _expect(norm_weight, torch.bfloat16, "norm_weight", (wB.K,))
    if b_bf16 is not None:
        _expect(b_bf16, torch.bfloat16, "b_bf16", (M, wB.K))
    c = MxgChain(M, a_q.data_ptr(), a_s.data_ptr(), _w(wA), _w(wB), _w(wC), out_a.data_ptr(),
                 b_q.data_ptr(), b_s.data_ptr(), out_b.data_ptr(), c_q.data_ptr(), c_s.data_ptr(),
                 out_c.data_ptr(), None, 0,
                 norm_weight.data_ptr() if norm_weight is not None else None, float(norm_eps),
                 b_bf16.data_ptr() if b_bf16 is not None else None)
    need = int(lib().mxg_chain_workspace_bytes(ctypes.byref(c)))
    if workspace is None:
        workspace = get_workspace(dev, need)
    c.workspace = workspace.data_ptr()
    c.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().mxfp8_proj_chain(ctypes.byref(c), _stream(stream)))
    return out_a, b_q, b_s, out_b, out_c


WO_A_ROTARY_OFFSET = 65536    # workspace byte offset of the rotated input's codes


def wo_a_rotary_codes(workspace: torch.Tensor, M: int, HD: int):
    """Views of the MXFP8 rotated input that wo_a_fused_quantize leaves in its
    workspace: codes [M, HD] and scale bytes [M, HD/32]."""
    q0 = WO_A_ROTARY_OFFSET
    s0 = (q0 + M * HD + 255) // 256 * 256
    return (workspace[q0:q0 + M * HD].view(M, HD),
            workspace[s0:s0 + M * HD // 32].view(M, HD // 32))


def wo_a_fused_quantize(o: torch.Tensor, positions: torch.Tensor, cos_sin: torch.Tensor,
                        wa: Weight, *, n_groups: int, nope_dim: int,
                        wb: Weight | None = None, outs=None, keep_z: bool = True,
                        workspace: torch.Tensor | None = None, stream=None):
    """Grouped WO-A with rotary in front and MXFP8 of its output behind,
    optionally followed by wo_b.

    ``o``: BF16 [M, H, D] (any row and head strides, D contiguous);
    ``positions``: int64 [M]; ``cos_sin``: float32 [max_pos, D - nope_dim];
    ``wa``: [G*R, (H/G)*D], packed or row-major.  Returns (z or None, z_q, z_s, out or None)."""
    if o.dim() != 3 or o.dtype != torch.bfloat16 or not o.is_cuda or o.stride(2) != 1:
        raise ValueError("o must be a BF16 [M, H, D] device tensor with contiguous last dim")
    M, H, D = o.shape
    dev = o.device
    GR = wa.N
    _expect(positions, torch.int64, "positions", (M,))
    _expect(cos_sin, torch.float32, "cos_sin")
    if outs is None:
        outs = (torch.empty(M, GR, dtype=torch.bfloat16, device=dev) if keep_z else None,
                torch.empty(M, GR, dtype=torch.uint8, device=dev),
                torch.empty(M, GR // 32, dtype=torch.uint8, device=dev),
                torch.empty(M, wb.N, dtype=torch.bfloat16, device=dev) if wb is not None else None)
    z, z_q, z_s, out = outs
    if z is not None:
        _expect(z, torch.bfloat16, "z", (M, GR))
    _expect(z_q, torch.uint8, "z_q", (M, GR))
    _expect(z_s, torch.uint8, "z_s", (M, GR // 32))
    if wb is not None:
        _expect(out, torch.bfloat16, "out", (M, wb.N))
    p = MxgWoA(M, o.data_ptr(), o.stride(0), o.stride(1), positions.data_ptr(),
               cos_sin.data_ptr(), cos_sin.shape[0], H, D, nope_dim, n_groups, _w(wa),
               z.data_ptr() if z is not None else None, z_q.data_ptr(), z_s.data_ptr(),
               _w(wb) if wb is not None else MxgWeight(None, None, 0, 0, 0),
               out.data_ptr() if wb is not None else None, None, 0)
    need = int(lib().mxg_wo_a_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = get_workspace(dev, need)
    p.workspace = workspace.data_ptr()
    p.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().wo_a_fused_quantize(ctypes.byref(p), _stream(stream)))
    return z, z_q, z_s, out
