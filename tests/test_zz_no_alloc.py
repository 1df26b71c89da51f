"""tern_gemv_noalloc (the product with the library's fixed per-GPU workspace
array, for callers that cannot allocate) against tern_gemv with a caller
workspace: bit-identical outputs on two calls in a row, the second on a
smaller input (the array keeps the first call's contents), on each route that
uses the workspace -- K parts with a reduce (2-bit, m = 1), the 16-row tiles'
tables (m = 8), and the base-3 stream kernel with residual-pass counters
(m = 1, 4) -- and within the oracle's bound; a product whose workspace
exceeds the array is rejected with TERN_E_WORKSPACE."""
import ctypes

import numpy as np
import pytest

import oracle as O
from ternary_weight_only_tern_amd import lib as L
from ternary_weight_only_tern_amd import synth
from gpu_util import b3_route, check_y, oracle_y, say, small_matrix, to_dev, upload_pack

pytestmark = pytest.mark.gpu


def _pair(mat, fmt, m, seed):
    import torch
    rng = np.random.default_rng(seed)
    x = synth.draw_x(rng, m, mat["k"], "student_t3")
    pm = upload_pack(mat, fmt)
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    y_ref = L.tern_gemv(pm, xd, L.TERN_F32)
    y = torch.full((m, mat["n"]), float("nan"), dtype=torch.float32, device="cuda")
    L.tern_gemv_noalloc(pm, xd, y, L.TERN_F32)
    torch.cuda.synchronize()
    return pm, x, y, y_ref


@pytest.mark.parametrize("fmt,m,route", [(O.FMT_2BIT, 1, "auto"), (O.FMT_2BIT, 8, "auto"),
                                         (O.FMT_B3, 1, "stream"), (O.FMT_B3, 4, "stream"),
                                         (O.FMT_B3, 1, "auto")])
def test_noalloc_matches_gemv_two_calls(fmt, m, route):
    import torch
    big, _ = small_matrix(1030, 12288, 128, 3, 0.2, seed=5, offset_mode=O.OFF_ROW)
    small, _ = small_matrix(129, 2560, 128, 2, 0.5, seed=6, offset_mode=O.OFF_GROUP)
    with b3_route(route):
        for name, mat, mm in (("first (larger)", big, m), ("second (smaller)", small, max(1, m // 2))):
            say("noalloc", name, fmt, mm, route)
            pm, x, y, y_ref = _pair(mat, fmt, mm, seed=mm + fmt)
            assert torch.equal(y, y_ref), f"{name}: tern_gemv_noalloc differs from tern_gemv"
            check_y(y, *oracle_y(mat, x), f"noalloc {name}")


def test_noalloc_rejects_oversized_workspace():
    lib = L.load()
    d = L.tern_matrix()
    d.n, d.k, d.group, d.planes, d.format, d.offset_mode = 32768, 65536, 128, 2, O.FMT_2BIT, O.OFF_NONE
    d.nnz[0] = int(0.1 * d.n * (d.k // d.group))
    need = lib.tern_workspace_bytes(ctypes.byref(d), 63)
    assert need > (16 << 20)
    # rejected before any pointer is used
    st = lib.tern_gemv_noalloc(ctypes.byref(d), None, 63, None, L.TERN_F16, None)
    assert st == L.TERN_E_WORKSPACE
    assert b"tern_gemv_noalloc" in L.load().tern_last_error()
