"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/*.h declares, and rejects bad arguments with the
documented status before anything touches a device.  Pointers passed here
are never dereferenced: every call fails validation first."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mxfp8_block_scaled_gemm_amd", "libmxgemm.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from mxfp8_block_scaled_gemm_amd import _build
        _build.build()
    import mxfp8_block_scaled_gemm_amd as mx
    return mx.lib()


@pytest.fixture(scope="module")
def probe_lib(lib):
    from mxfp8_block_scaled_gemm_amd import probe
    if not os.path.exists(probe.LIB_PATH):
        from mxfp8_block_scaled_gemm_amd import _build
        _build.build()
    return probe.lib()


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M):
            if not m.group(0).lstrip().startswith(("#", "typedef", "return")):
                names.add(m.group(1))
    return sorted(names)


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("mxfp8_quantize", "mxfp8_gemm", "mxg_strerror", "mxg_version"):
        assert n in names, names


@pytest.mark.parametrize("name", declared_functions())
def test_every_declared_symbol_is_exported(lib, name):
    assert hasattr(lib, name), f"{name} is declared in include/ but not exported"


def test_strerror(lib):
    for st in range(6):
        assert lib.mxg_strerror(st)
    assert b"unknown" in lib.mxg_strerror(99)


A = 0x10000   # fake 16-byte-aligned addresses; never dereferenced
P = lambda k: ctypes.c_void_p(A * (k + 1))


def gemm(lib, M=4, N=1024, K=2048, x=None, ld_x=0, a_q=P(1), a_s=P(2), w_q=P(3), w_s=P(4),
         out=P(5), ws=P(7), ws_bytes=1 << 30):
    return lib.mxfp8_gemm(M, N, K, x, ld_x, a_q, a_s, w_q, w_s, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a_q=None), 1), (dict(w_s=None), 1), (dict(out=None), 1),
    (dict(M=0), 3), (dict(M=257), 3), (dict(M=-1), 3),
    (dict(K=100), 3), (dict(K=64), 3), (dict(K=0), 3), (dict(K=16384 + 128, N=128), 3),
    (dict(N=8), 3), (dict(N=1000), 3),
    (dict(x=P(6), ld_x=1024), 3),
    (dict(a_q=ctypes.c_void_p(A + 8)), 2), (dict(w_q=ctypes.c_void_p(A + 1)), 2),
    (dict(out=ctypes.c_void_p(A + 4)), 2),
    (dict(x=ctypes.c_void_p(A + 2), ld_x=2048), 2), (dict(x=P(6), ld_x=2052), 2),
    (dict(ws=None), 4), (dict(ws_bytes=16), 4), (dict(ws=ctypes.c_void_p(A + 4)), 2),
])
def test_gemm_rejects(lib, kw, status):
    assert gemm(lib, **kw) == status


def gemm_noalloc(lib, M=4, N=1024, K=2048, x=None, ld_x=0, a_q=P(1), a_s=P(2), w_q=P(3), w_s=P(4),
                 out=P(5)):
    return lib.mxfp8_gemm_noalloc(M, N, K, x, ld_x, a_q, a_s, w_q, w_s, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a_q=None), 1), (dict(out=None), 1), (dict(M=0), 3), (dict(M=257), 3), (dict(K=100), 3),
    (dict(N=1000), 3), (dict(x=P(6), ld_x=1024), 3), (dict(w_q=ctypes.c_void_p(A + 1)), 2),
    (dict(x=P(6), ld_x=2052), 2),
    # K-split state larger than the library's scratch: rejected before any device call
    (dict(M=192, N=8192, K=16384), 4),
])
def test_gemm_noalloc_rejects(lib, kw, status):
    assert gemm_noalloc(lib, **kw) == status


def test_noalloc_scratch_limit_matches_header(lib):
    import mxfp8_block_scaled_gemm_amd as mx
    text = open(os.path.join(ROOT, "include", "mxgemm.h")).read()
    m = re.search(r"#define MXG_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mx.NOALLOC_SCRATCH_BYTES
    assert lib.mxg_gemm_workspace_bytes(192, 8192, 16384) > mx.NOALLOC_SCRATCH_BYTES
    assert lib.mxg_gemm_workspace_bytes(48, 4096, 5120) <= mx.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("args,status", [
    ((None, 4, 64, 64, P(1), P(2)), 1),
    ((P(0), 0, 64, 64, P(1), P(2)), 3),
    ((P(0), 4, 48, 64, P(1), P(2)), 3),
    ((P(0), 4, 64, 32, P(1), P(2)), 3),
    ((ctypes.c_void_p(A + 2), 4, 64, 64, P(1), P(2)), 2),
    ((P(0), 4, 64, 68, P(1), P(2)), 2),
])
def test_quantize_rejects(lib, args, status):
    assert lib.mxfp8_quantize(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, P(1), 4096, 5120, P(2)), 1),
    ((P(0), P(1), 4096, 5120, None), 1),
    ((P(0), P(1), 4100, 5120, P(2)), 3),
    ((P(0), P(1), 4096, 5000, P(2)), 3),
    ((P(0), P(1), 4096, 8192 + 128, P(2)), 3),
    ((ctypes.c_void_p(A + 8), P(1), 4096, 5120, P(2)), 2),
    ((P(0), P(1), 4096, 5120, ctypes.c_void_p(A + 2)), 2),
])
def test_hbm_read_probe_rejects(probe_lib, args, status):
    assert probe_lib.mxg_hbm_read_probe(*args, None) == status


def test_probe_lives_outside_the_gemm_library(lib, probe_lib):
    # The read probe is a measurement aid: its own library exports it, the
    # GEMM library does not.
    assert hasattr(probe_lib, "mxg_hbm_read_probe")
    assert not hasattr(lib, "mxg_hbm_read_probe")


def test_forced_foreign_arch_is_rejected_before_launch(lib, probe_lib, monkeypatch):
    # A fully valid call on a device that reports another architecture must
    # return MXG_ERR_DEVICE without launching (the pointers are fake).
    monkeypatch.setenv("MXG_FORCE_ARCH", "gfx942")
    assert gemm(lib) == 5
    assert lib.mxfp8_quantize(P(0), 4, 64, 64, P(1), P(2), None) == 5
    assert lib.wo_a_fused_quantize(ctypes.byref(_wo_a()), None) == 5
    assert probe_lib.mxg_hbm_read_probe(P(0), P(1), 4096, 5120, P(2), None) == 5


def test_workspace_size_is_positive(lib):
    assert lib.mxg_gemm_workspace_bytes(4, 1024, 2048) >= 256


def test_chain_rejects_before_launch(lib):
    # Every call below fails validation; the valid base chain is never passed.
    import mxfp8_block_scaled_gemm_amd as mx
    w = lambda k, N, K: mx.MxgWeight(A * k, A * (k + 1), N, K)
    c = mx.MxgChain(8, A, A, w(2, 2048, 5120), w(4, 8192, 1536), w(6, 5120, 8192), A * 8, A * 9,
                    A * 10, A * 11, A * 12, A * 13, A * 14, A * 15, 1 << 30)
    for field, value, status in (("M", 0, 3), ("M", 49, 3), ("out_b", None, 1),
                                 ("workspace", None, 4), ("workspace_bytes", 8, 4)):
        bad = mx.MxgChain.from_buffer_copy(c)
        setattr(bad, field, value)
        assert lib.mxfp8_proj_chain(ctypes.byref(bad), None) == status, field
    bad = mx.MxgChain.from_buffer_copy(c)
    bad.wB = w(4, 8192, 100)                  # K % 128 != 0
    assert lib.mxfp8_proj_chain(ctypes.byref(bad), None) == 3
    bad = mx.MxgChain.from_buffer_copy(c)
    bad.wB = w(4, 8192, 4096)                 # requantized width beyond A's output
    assert lib.mxfp8_proj_chain(ctypes.byref(bad), None) == 3
    for layout in (2, -1):                    # unknown weight layout
        bad = mx.MxgChain.from_buffer_copy(c)
        bad.wC.layout = layout
        assert lib.mxfp8_proj_chain(ctypes.byref(bad), None) == 3
    bad = mx.MxgChain.from_buffer_copy(c)
    bad.a_q = A + 8
    assert lib.mxfp8_proj_chain(ctypes.byref(bad), None) == 2
    # the optional norm: a negative or non-finite eps, misaligned gain or copy
    for field, value, status in (("norm_eps", -1.0, 3), ("norm_eps", float("nan"), 3),
                                 ("norm_eps", float("inf"), 3), ("norm_weight", A + 2, 2)):
        bad = mx.MxgChain.from_buffer_copy(c)
        bad.norm_weight = A * 16
        setattr(bad, field, value)
        assert lib.mxfp8_proj_chain(ctypes.byref(bad), None) == status, field
    bad = mx.MxgChain.from_buffer_copy(c)
    bad.norm_weight, bad.b_bf16 = A * 16, A + 4
    assert lib.mxfp8_proj_chain(ctypes.byref(bad), None) == 2


def test_struct_layouts_match_the_header(tmp_path):
    # The binding's ctypes structures must have the C layout of include/mxgemm.h:
    # compile a probe with the host C compiler and compare every field offset.
    import shutil
    import subprocess
    import mxfp8_block_scaled_gemm_amd as mx
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"mxg_weight": mx.MxgWeight, "mxg_chain": mx.MxgChain, "mxg_wo_a": mx.MxgWoA}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mxgemm.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    c = {tuple(l.split()[:2]): int(l.split()[2]) for l in got if l}
    for cname, py in structs.items():
        assert c[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert c[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def _wo_a(**kw):
    import mxfp8_block_scaled_gemm_amd as mx
    w = lambda k, N, K: mx.MxgWeight(A * k, A * (k + 1), N, K)
    base = dict(M=4, o=A, ld_row=64 * 512, ld_head=512, positions=A * 2, cos_sin=A * 3,
                max_pos=65536, n_heads=64, head_dim=512, nope_dim=448, n_groups=8,
                wa=w(4, 8192, 4096), z=A * 6, z_q=A * 7, z_s=A * 8, wb=w(9, 5120, 8192),
                out=A * 11, workspace=A * 12, workspace_bytes=1 << 30)
    base.update(kw)
    return mx.MxgWoA(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(positions=None), 1), (dict(z_q=None), 1), (dict(out=None), 1),
    (dict(M=0), 3), (dict(M=49), 3), (dict(n_groups=7), 3), (dict(n_groups=4), 3),
    (dict(nope_dim=450), 3), (dict(nope_dim=512), 3), (dict(head_dim=500), 3),
    (dict(ld_head=256), 3), (dict(ld_row=1000), 3),
    (dict(max_pos=0), 3),
    (dict(o=A + 8), 2), (dict(positions=A + 4), 2), (dict(ld_head=516, ld_row=64 * 516), 2),
    (dict(cos_sin=A + 4), 2), (dict(z=A + 2), 2),
    (dict(workspace=None), 4), (dict(workspace_bytes=1024), 4),
])
def test_wo_a_rejects(lib, kw, status):
    import mxfp8_block_scaled_gemm_amd as mx
    p = _wo_a(**kw)
    assert lib.wo_a_fused_quantize(ctypes.byref(p), None) == status


def test_wo_a_rejects_weight_shapes(lib):
    import mxfp8_block_scaled_gemm_amd as mx
    w = lambda k, N, K: mx.MxgWeight(A * k, A * (k + 1), N, K)
    for wa, wb in ((w(4, 8192, 2048), w(9, 5120, 8192)),     # K != hpg * D
                   (w(4, 8 * 1040, 4096), w(9, 5120, 8320)),  # R % 128 != 0
                   (w(4, 8192, 4096), w(9, 5120, 4096))):     # wb.K != G * R
        p = _wo_a(wa=wa, wb=wb)
        assert lib.wo_a_fused_quantize(ctypes.byref(p), None) == 3
    for field in ("wa", "wb"):                                 # unknown weight layout
        p = _wo_a()
        getattr(p, field).layout = 2
        assert lib.wo_a_fused_quantize(ctypes.byref(p), None) == 3


def test_wo_a_workspace_size(lib):
    import mxfp8_block_scaled_gemm_amd as mx
    p = _wo_a(z=None)
    with_z = lib.mxg_wo_a_workspace_bytes(ctypes.byref(_wo_a()))
    without = lib.mxg_wo_a_workspace_bytes(ctypes.byref(p))
    assert with_z >= 65536 + 4 * 32768 + 4 * 1024
    assert without >= with_z + 2 * 4 * 8192


def rmsnorm(lib, x=P(0), M=4, K=1536, ld_x=2048, w=P(1), eps=1e-6, y=P(2), ld_y=1536, q=P(3),
            s=P(4), layout=0):
    return lib.mxfp8_rmsnorm_quantize(x, M, K, ld_x, w, eps, y, ld_y, q, s, layout, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(w=None), 1), (dict(q=None), 1), (dict(s=None), 1),
    (dict(M=0), 3), (dict(M=65536), 3), (dict(K=96, ld_x=96), 3), (dict(K=1600), 3),
    (dict(K=16384 + 128, ld_x=20000), 3), (dict(ld_x=1024), 3), (dict(ld_y=1024), 3),
    (dict(eps=-1.0), 3), (dict(eps=float("nan")), 3), (dict(eps=float("inf")), 3),
    (dict(layout=2), 3), (dict(layout=-1), 3),
    (dict(x=ctypes.c_void_p(A + 2)), 2), (dict(w=ctypes.c_void_p(A + 8)), 2),
    (dict(q=ctypes.c_void_p(A + 4)), 2), (dict(y=ctypes.c_void_p(A + 2)), 2),
    (dict(ld_x=2052), 2), (dict(ld_y=1540), 2),
])
def test_rmsnorm_quantize_rejects(lib, kw, status):
    assert rmsnorm(lib, **kw) == status


def test_scale_bytes_128x4(lib):
    # ceil(M/128)*128 rows times K/32 scale columns (K a multiple of 128)
    assert lib.mxg_scale_bytes_128x4(1, 5120) == 128 * 160
    assert lib.mxg_scale_bytes_128x4(128, 1536) == 128 * 48
    assert lib.mxg_scale_bytes_128x4(129, 1536) == 256 * 48
    assert lib.mxg_scale_bytes_128x4(0, 1536) == 0


def gemm_ex(lib, M=4, N=1024, K=2048, x=None, ld_x=0, a_q=P(1), a_s=P(2), layout=1, w_q=P(3),
            w_s=P(4), w_layout=0, out=P(5), ws=P(7), ws_bytes=1 << 30):
    return lib.mxfp8_gemm_ex(M, N, K, x, ld_x, a_q, a_s, layout, w_q, w_s, w_layout, out, ws,
                             ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a_s=None), 1), (dict(a_q=None), 1), (dict(layout=0, out=None), 1),
    (dict(w_layout=1, w_s=None), 1),
    (dict(layout=2), 3), (dict(layout=-1), 3), (dict(M=0), 3), (dict(M=257), 3),
    (dict(K=1000), 3), (dict(layout=0, M=257), 3),
    (dict(w_layout=2), 3), (dict(w_layout=-1), 3), (dict(layout=0, w_layout=2), 3),
    # 128 x 4 scales take MXFP8 input only; BF16 input needs ld_x >= K
    (dict(x=P(6), ld_x=2048), 3), (dict(layout=0, x=P(6), ld_x=1024), 3),
    (dict(a_q=ctypes.c_void_p(A + 8)), 2), (dict(a_s=ctypes.c_void_p(A + 4)), 2),
    (dict(w_layout=1, w_q=ctypes.c_void_p(A + 8)), 2),
    (dict(layout=0, x=ctypes.c_void_p(A + 2), ld_x=2048), 2),
    (dict(layout=0, x=P(6), ld_x=2052), 2),
    (dict(ws=None), 4), (dict(w_layout=1, ws=None), 4),
])
def test_gemm_ex_rejects(lib, kw, status):
    assert gemm_ex(lib, **kw) == status
