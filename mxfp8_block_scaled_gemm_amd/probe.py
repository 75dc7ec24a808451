"""Binding of libmxprobe, the HBM read probe (a measurement aid beside the
GEMM library, declared in probe_src/mxprobe.h): argument marshalling only.
There is no fallback: if the shared library is missing the first call raises."""
from __future__ import annotations

import ctypes
import os

import torch

from . import MxgError, PackedWeight, _ptr, _stream, strerror

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxprobe.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.mxg_hbm_read_probe.argtypes = [vp, vp, i64, i64, vp, vp]
        L.mxg_hbm_read_probe.restype = ctypes.c_int
        _lib = L
    return _lib


def hbm_read_probe(w: PackedWeight, sink: torch.Tensor, stream=None) -> None:
    """Read the packed weight w as the GEMMs' weight stream does, computing
    nothing (mxg_hbm_read_probe); sink is a device int32 word."""
    if not sink.is_cuda or sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("sink must be a device int32 tensor")
    st = lib().mxg_hbm_read_probe(w.q.data_ptr(), w.s.data_ptr(), w.N, w.K, _ptr(sink),
                                  _stream(stream))
    if st != 0:
        raise MxgError(st, strerror(st))
