"""Helpers for GPU tests: upload synthetic matrices, pack them through the C
ABI, and compare against the CPU oracle."""
from __future__ import annotations

import contextlib
import sys

import numpy as np

import oracle as O
from ternary_weight_only_tern_amd import lib as L
from ternary_weight_only_tern_amd import synth


@contextlib.contextmanager
def b3_route(route: str):
    """route "stream": every base-3 launch at m <= 4 takes the matrix-core
    stream kernel (threshold 0); "auto": the library's default threshold
    (small launches take the lane-per-row decode)."""
    if route == "stream":
        L.tern_b3_min_stages(0)
    try:
        yield
    finally:
        L.tern_b3_min_stages(-1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def upload_pack(mat: dict, fmt: int) -> L.PackedMatrix:
    """Pack a synth matrix on the GPU (tern_pack) and return its buffers."""
    import torch
    planes = mat["planes"]
    nnz = [int(m.sum()) for m in mat["masks"]]
    pm = L.PackedMatrix(mat["n"], mat["k"], mat["group"], planes, fmt, mat["offset_mode"], nnz)
    trits = to_dev(mat["trits"])
    scales = to_dev(mat["scales"])
    masks = to_dev(np.stack(mat["mask_bits"]).view(np.int32)) if planes > 1 else None
    off = to_dev(mat["offset"]) if mat["offset"] is not None else None
    L.tern_pack(pm, trits, scales, masks, off)
    torch.cuda.synchronize()
    return pm


def oracle_pack(mat: dict, fmt: int) -> dict:
    return O.pack(mat["trits"], mat["scales"], mat["mask_bits"], mat["offset"], mat["group"], fmt)


def assert_bytes_equal(pm: L.PackedMatrix, ref: dict):
    n = pm.n
    stride = L.tern_row_stride(pm.k, pm.group, pm.fmt)
    got0 = pm.plane0.cpu().numpy()[: n * stride].reshape(n, stride)
    assert np.array_equal(got0, ref["plane0"]), "plane-0 bytes differ"
    for p in range(pm.planes - 1):
        assert np.array_equal(pm.rowptr[p].cpu().numpy().view(np.uint32), ref["rowptr"][p]), "rowptr differs"
        nb = pm.nnz[p] * (pm.group // 4)
        assert np.array_equal(pm.blocks[p].cpu().numpy()[:nb], ref["blocks"][p].reshape(-1)), "blocks differ"
        assert np.array_equal(pm.rscale[p].cpu().numpy()[: pm.nnz[p]].view(np.uint16),
                              ref["rscale"][p].view(np.uint16)), "rscale differs"


def oracle_y(mat: dict, x: np.ndarray):
    y = O.gemv(mat["trits"], mat["scales"], mat["masks"], mat["offset"], mat["offset_mode"], x, mat["group"])
    b = O.bound(mat["trits"], mat["scales"], mat["masks"], mat["offset"], mat["offset_mode"], x, mat["group"])
    return y, b


def check_y(y_dev, y_ref: np.ndarray, b: np.ndarray, what: str = ""):
    """The acceptance bound |y - y_ref| <= 2e-3 * B, element by element."""
    y = y_dev.float().cpu().numpy().astype(np.float64)
    ok = O.accept(y, y_ref, b)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        detail = [(tuple(i), y[tuple(i)], y_ref[tuple(i)], b[tuple(i)]) for i in idx]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside the bound, e.g. {detail}")
    err = np.abs(y - y_ref)
    rel = np.max(err / np.where(b > 0, b, 1))
    return float(rel)


def small_matrix(n, k, group, planes, frac, seed, offset_mode=O.OFF_NONE, scale_law="uniform"):
    rng = np.random.default_rng(seed)
    mat = synth.make_matrix(n, k, group, planes, frac, rng=rng, scale_law=scale_law,
                            offset_mode=offset_mode)
    return mat, rng
