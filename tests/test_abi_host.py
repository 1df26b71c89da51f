"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and answers argument errors without touching a GPU."""
import ctypes
import math
import os
import re

import pytest

from ternary_weight_only_tern_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tern.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tern_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = _declared()
    assert set(names) == set(L.SYMBOLS)
    for name in names:
        assert hasattr(lib, name), name


def test_row_stride():
    assert L.tern_row_stride(4096, 128, L.TERN_FMT_2BIT) == 1024
    assert L.tern_row_stride(4096, 128, L.TERN_FMT_B3) == 832      # 32 groups x 26 bytes
    assert L.tern_row_stride(12288, 128, L.TERN_FMT_B3) == 2496    # 96 x 26
    assert L.tern_row_stride(2560, 128, L.TERN_FMT_B3) == 528      # 20 x 26 = 520 -> 528
    assert L.tern_row_stride(256, 64, L.TERN_FMT_B3) == 64         # 4 x 13 = 52 -> 64
    assert L.tern_row_stride(100, 64, L.TERN_FMT_2BIT) == 0        # unsupported k
    assert L.tern_row_stride(4096, 96, L.TERN_FMT_2BIT) == 0       # unsupported group


def test_packed_sizes_and_bits():
    sz = L.tern_packed_sizes(4096, 12288, 128, L.TERN_FMT_2BIT, 3, [78643, 78643], L.TERN_OFF_ROW)
    assert sz[L.TERN_BUF_PLANE0] == 4096 * 3072
    assert sz[L.TERN_BUF_SCALE0] == 4096 * 96 * 2
    assert sz[L.TERN_BUF_OFFSET] == 4096 * 2
    assert sz[L.TERN_BUF_MASK] == 4096 * 3 * 4
    assert sz[L.TERN_BUF_ROWPTR] == 4097 * 4
    assert sz[L.TERN_BUF_BLOCKS1] == sz[L.TERN_BUF_BLOCKS2] == 78643 * 32
    d = L.tern_matrix(n=4096, k=12288, group=128, planes=3, format=L.TERN_FMT_2BIT, offset_mode=L.TERN_OFF_ROW)
    d.nnz[0] = d.nnz[1] = 78643
    info, plane, storage = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    L.check(L.load().tern_bits(ctypes.byref(d), ctypes.byref(info), ctypes.byref(plane), ctypes.byref(storage)))
    f = 78643 / (4096 * 96)
    assert math.isclose(info.value, math.log2(3) * (1 + 2 * f), rel_tol=1e-12)
    assert math.isclose(plane.value, 2.0 * (1 + 2 * f), rel_tol=1e-12)
    total = sum(sz) + sz[L.TERN_BUF_MASK] + sz[L.TERN_BUF_ROWPTR]
    assert math.isclose(storage.value, 8.0 * total / (4096 * 12288), rel_tol=1e-12)


def _desc(**kw):
    d = L.tern_matrix(n=kw.get("n", 128), k=kw.get("k", 256), group=kw.get("group", 64),
                      planes=kw.get("planes", 1), format=kw.get("fmt", 0), offset_mode=kw.get("off", 0))
    d.plane0 = kw.get("plane0", 0x10000)
    d.scale0 = kw.get("scale0", 0x20000)
    return d


def test_check_errors_without_gpu():
    lib = L.load()
    assert lib.tern_check(ctypes.byref(_desc())) == L.TERN_OK
    assert lib.tern_check(ctypes.byref(_desc(plane0=0x10001))) == L.TERN_E_ALIGN
    d = _desc()
    d.plane0 = None
    assert lib.tern_check(ctypes.byref(d)) == L.TERN_E_INVAL
    assert lib.tern_check(ctypes.byref(_desc(k=100))) == L.TERN_E_UNSUPPORTED
    assert lib.tern_check(ctypes.byref(_desc(group=96))) == L.TERN_E_UNSUPPORTED
    assert lib.tern_check(ctypes.byref(_desc(k=256, group=128 * 3))) == L.TERN_E_UNSUPPORTED
    assert lib.tern_check(ctypes.byref(_desc(planes=4))) == L.TERN_E_UNSUPPORTED
    assert lib.tern_check(ctypes.byref(_desc(fmt=7))) == L.TERN_E_UNSUPPORTED
    assert lib.tern_check(ctypes.byref(_desc(off=1))) == L.TERN_E_INVAL       # offset missing
    assert lib.tern_check(ctypes.byref(_desc(planes=2))) == L.TERN_E_INVAL    # mask missing
    assert lib.tern_check(ctypes.byref(_desc(n=-1))) == L.TERN_E_INVAL
    assert "offset" in L.last_error() or "shape" in L.last_error() or L.last_error()


def test_products_reject_bad_arguments_before_any_launch():
    lib = L.load()
    d = _desc()
    ws = ctypes.c_void_p(0x40000)
    for fn in (lib.tern_gemv,):
        assert fn(ctypes.byref(d), 0x30000, 64, 0x50000, 0, ws, 1 << 20, None) == L.TERN_E_UNSUPPORTED
    assert lib.tern_gemv(ctypes.byref(d), None, 1, 0x50000, 0, ws, 1 << 20, None) == L.TERN_E_INVAL
    assert lib.tern_gemv(ctypes.byref(d), 0x30008, 1, 0x50000, 0, ws, 1 << 20, None) == L.TERN_E_ALIGN
    assert lib.tern_gemv(ctypes.byref(d), 0x30000, 1, 0x50001, 0, ws, 1 << 20, None) == L.TERN_E_ALIGN
    assert lib.tern_gemv(ctypes.byref(d), 0x30000, 1, 0x50000, 5, ws, 1 << 20, None) == L.TERN_E_UNSUPPORTED
    assert lib.tern_gemv(ctypes.byref(d), 0x30000, -1, 0x50000, 0, ws, 1 << 20, None) == L.TERN_E_INVAL
    # empty products are no-ops that never touch memory
    assert lib.tern_gemv(ctypes.byref(d), 0x30000, 0, 0x50000, 0, ws, 0, None) == L.TERN_OK
    assert lib.tern_gemm(ctypes.byref(_desc(n=0)), 0x30000, 7, 0x50000, 0, ws, 0, None) == L.TERN_OK
    # group 256 is packable but not multiplied
    g = _desc(k=512, group=256)
    assert lib.tern_gemm(ctypes.byref(g), 0x30000, 70, 0x50000, 0, ws, 0, None) == L.TERN_E_UNSUPPORTED


def test_pack_rejects_bad_arguments():
    lib = L.load()
    d = _desc(planes=2)
    d.mask[0] = 0x60000
    d.rowptr[0] = 0x70000
    d.nnz[0] = 3
    d.blocks[0] = 0x80000
    d.rscale[0] = 0x90000
    assert lib.tern_pack(0x1000, None, ctypes.byref(d), 0x2000, 4096, None) == L.TERN_E_INVAL  # rscale_dense
    assert lib.tern_pack(0x1000, 0x3001, ctypes.byref(d), 0x2000, 4096, None) == L.TERN_E_ALIGN
    assert lib.tern_pack(0x1008, 0x3000, ctypes.byref(d), 0x2000, 4096, None) == L.TERN_E_ALIGN
    assert lib.tern_pack(0x1000, 0x3000, ctypes.byref(d), None, 0, None) == L.TERN_E_WORKSPACE


def test_status_strings():
    for s in range(-6, 1):
        assert L.status_str(s).startswith("TERN_")


def test_quantize_rejects_bad_arguments_before_any_launch():
    lib = L.load()
    nul = ctypes.c_void_p(0)
    q = lambda n, k, g, it: lib.tern_quantize(nul, n, k, g, nul, it, nul, nul, nul, nul)
    assert q(4, 256, 96, 15) == L.TERN_E_UNSUPPORTED
    assert q(4, 200, 128, 15) == L.TERN_E_UNSUPPORTED
    assert q(-1, 256, 128, 15) == L.TERN_E_INVAL
    assert q(4, 256, 128, -1) == L.TERN_E_INVAL
    assert q(4, 256, 128, 1001) == L.TERN_E_INVAL
    assert q(0, 256, 128, 15) == L.TERN_OK  # empty: nothing to do, no pointer touched
    assert q(4, 256, 128, 15) == L.TERN_E_INVAL  # NULL weights


def test_rotate_rejects_bad_arguments_before_any_launch():
    lib = L.load()
    nul = ctypes.c_void_p(0)
    r = lambda block, m, k: lib.tern_rotate(nul, block, nul, m, k, nul, nul)
    assert r(96, 1, 384) == L.TERN_E_UNSUPPORTED
    assert r(128, 1, 200) == L.TERN_E_UNSUPPORTED
    assert r(128, -1, 256) == L.TERN_E_INVAL
    assert r(128, 0, 256) == L.TERN_OK
    assert r(128, 2, 256) == L.TERN_E_INVAL  # NULL pointers


def test_rotate_batched_rejects_bad_arguments_before_any_launch():
    lib = L.load()
    ks = (ctypes.c_int32 * 2)(256, 200)
    ptrs = (ctypes.c_void_p * 2)(None, None)
    assert lib.tern_rotate_batched(9, ptrs, 128, ptrs, ks, 1, ptrs, None) == L.TERN_E_UNSUPPORTED
    assert lib.tern_rotate_batched(2, ptrs, 128, ptrs, ks, 1, ptrs, None) == L.TERN_E_UNSUPPORTED  # 200 % 128
    assert lib.tern_rotate_batched(1, ptrs, 96, ptrs, ks, 1, ptrs, None) == L.TERN_E_UNSUPPORTED
    assert lib.tern_rotate_batched(1, ptrs, 128, ptrs, ks, -1, ptrs, None) == L.TERN_E_INVAL
    assert lib.tern_rotate_batched(0, None, 128, None, None, 1, None, None) == L.TERN_OK
    assert lib.tern_rotate_batched(1, ptrs, 128, ptrs, ks, 1, ptrs, None) == L.TERN_E_INVAL  # NULL device pointers
