"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Packing must be byte-identical to the oracle's encoding; products must meet
|y - y_ref| <= 2e-3 * sum_k (|off| + sum_p m_p |s_p T_p|) |x| per element
(the tolerance the project fixes for FP32 accumulation on FP16 inputs), with
y == 0 exactly where that bound is 0.
"""
import ctypes

import numpy as np
import pytest

import oracle as O
from ternary_weight_only_tern_amd import lib as L
from ternary_weight_only_tern_amd import synth

from gpu_util import (assert_bytes_equal, b3_route, check_y, oracle_pack, oracle_y, say, small_matrix,
                       to_dev, upload_pack)

pytestmark = pytest.mark.gpu

FMTS = [O.FMT_2BIT, O.FMT_B3]
# formats with the base-3 route forced onto the matrix-core stream kernel as
# well as the default routing (small launches take the lane-per-row decode)
FMT_ROUTES = [(O.FMT_2BIT, "auto"), (O.FMT_B3, "auto"), (O.FMT_B3, "stream")]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.load()
    yield


def _ydt(f32):
    return L.TERN_F32 if f32 else L.TERN_F16


# ----------------------------------------------------------------- packing
SMALL_SHAPES = [  # n, k, group, planes, frac, offset_mode
    (128, 256, 64, 1, 0.0, O.OFF_NONE),
    (65, 640, 64, 2, 0.3, O.OFF_GROUP),
    (130, 1280, 128, 3, 0.2, O.OFF_ROW),
    (7, 2560, 128, 2, 0.1, O.OFF_NONE),
    (64, 128, 128, 2, 1.0, O.OFF_NONE),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_pack_bytes_small(shape, fmt):
    n, k, g, planes, frac, off = shape
    say("pack", shape, fmt)
    mat, _ = small_matrix(n, k, g, planes, frac, seed=n + k, offset_mode=off)
    pm = upload_pack(mat, fmt)
    assert_bytes_equal(pm, oracle_pack(mat, fmt))


@pytest.mark.parametrize("wl,proj,fmt", [("single_gemv", 0, O.FMT_2BIT), ("qwen3_4b_layer", 0, O.FMT_2BIT),
                                         ("qwen3_4b_layer", 6, O.FMT_B3), ("qwen3_8b_stack", 4, O.FMT_B3),
                                         ("qwen3_8b_stack", 6, O.FMT_B3), ("down_proj_stress", 0, O.FMT_2BIT),
                                         ("down_proj_stress", 0, O.FMT_B3)])
def test_pack_bytes_workloads(wl, proj, fmt):
    say("pack workload", wl, proj, fmt)
    mat = synth.workload_matrix(wl, proj)
    pm = upload_pack(mat, fmt)
    assert_bytes_equal(pm, oracle_pack(mat, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_unpack_roundtrip_and_corruption(fmt):
    import torch
    say("unpack", fmt)
    mat, _ = small_matrix(96, 1280, 128, 3, 0.25, seed=3, offset_mode=O.OFF_ROW)
    pm = upload_pack(mat, fmt)
    back = L.tern_unpack(pm).cpu().numpy()
    assert np.array_equal(back, mat["trits"])
    # invalid plane-0 code
    saved = pm.plane0.clone()
    if fmt == O.FMT_2BIT:
        pm.plane0[5] = 0x02          # offset-0 trit with code 10
    else:
        pm.plane0[5] = 250           # base-3 byte above 242
    with pytest.raises(L.TernError) as e:
        L.tern_unpack(pm)
    assert e.value.status == L.TERN_E_CORRUPT
    pm.plane0.copy_(saved)
    if fmt == O.FMT_B3:
        pm.plane0[25] = 121 - 81      # last byte of group 0 with a -1 padding trit
        with pytest.raises(L.TernError) as e:
            L.tern_unpack(pm)
        assert e.value.status == L.TERN_E_CORRUPT
        pm.plane0.copy_(saved)
    # corrupt residual block code and rowptr
    sb = pm.blocks[0].clone()
    pm.blocks[0][0] = 0x02
    with pytest.raises(L.TernError) as e:
        L.tern_unpack(pm)
    assert e.value.status == L.TERN_E_CORRUPT
    pm.blocks[0].copy_(sb)
    pm.rowptr[1][3] += 1
    with pytest.raises(L.TernError) as e:
        L.tern_unpack(pm)
    assert e.value.status == L.TERN_E_CORRUPT
    pm.rowptr[1][3] -= 1
    assert np.array_equal(L.tern_unpack(pm).cpu().numpy(), mat["trits"])
    torch.cuda.synchronize()


def test_pack_rejects_invalid_input():
    say("pack invalid")
    mat, _ = small_matrix(64, 256, 64, 2, 0.25, seed=4)
    bad = dict(mat)
    bad["trits"] = mat["trits"].copy()
    bad["trits"][0, 3, 7] = 2
    with pytest.raises(L.TernError) as e:
        upload_pack(bad, O.FMT_2BIT)
    assert e.value.status == L.TERN_E_INVAL
    bad["trits"] = mat["trits"].copy()
    rows, groups = np.nonzero(~mat["masks"][0])
    bad["trits"][1, rows[0], groups[0] * 64 + 5] = 1     # residual trit outside the mask
    with pytest.raises(L.TernError) as e:
        upload_pack(bad, O.FMT_B3)
    assert e.value.status == L.TERN_E_INVAL


# ----------------------------------------------------------------- decode products
def _gemv_case(mat, fmt, m, x_law="normal", f32=False, seed=0, batched=False):
    import torch
    rng = np.random.default_rng(seed)
    x = synth.draw_x(rng, m, mat["k"], x_law)
    pm = upload_pack(mat, fmt)
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    y = L.tern_gemv(pm, xd, _ydt(f32))
    torch.cuda.synchronize()
    y_ref, b = oracle_y(mat, x)
    return check_y(y, y_ref, b, f"gemv n={mat['n']} k={mat['k']} fmt={fmt} m={m}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SMALL_SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
def test_gemv_small(shape, fmt, m):
    n, k, g, planes, frac, off = shape
    say("gemv small", shape, fmt, m)
    mat, _ = small_matrix(n, k, g, planes, frac, seed=7 * n + k, offset_mode=off, scale_law="lognormal")
    _gemv_case(mat, fmt, m, x_law="student_t3", seed=m)


@pytest.mark.parametrize("shape", SMALL_SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_gemv_small_b3_stream(shape, m):
    """The small shapes through the base-3 matrix-core stream kernel (the
    default routing sends launches this small to the lane-per-row decode)."""
    n, k, g, planes, frac, off = shape
    say("gemv small b3 stream", shape, m)
    mat, _ = small_matrix(n, k, g, planes, frac, seed=7 * n + k, offset_mode=off, scale_law="lognormal")
    with b3_route("stream"):
        _gemv_case(mat, O.FMT_B3, m, x_law="student_t3", seed=m)


@pytest.mark.parametrize("route", ["stream", "auto"])
@pytest.mark.parametrize("m", [1, 3, 4])
@pytest.mark.parametrize("planes,off", [(3, O.OFF_ROW), (2, O.OFF_GROUP), (3, O.OFF_NONE)])
def test_b3_residual_split_units(planes, off, m, route):
    """Base-3 at m <= 4 with dense residual planes on few rows: the residual
    pass cuts each plane's entries of a row block into many ranges (units
    that sum their own rows, the block's last unit adding them in slot
    order).  Single products (tern_gemv: counters cleared inside the launch
    sequence) and a plan of both (counters cleared at creation), each run
    twice (the counters are left clear by the first run); runs are
    bit-identical."""
    import torch
    say("b3 residual split units", planes, off, m, route)
    with b3_route(route):
        _residual_split_case(planes, off, m)


def _residual_split_case(planes, off, m):
    import torch
    mats = [small_matrix(300, 2560, 128, planes, 1.0, seed=90 + planes, offset_mode=off)[0],
            small_matrix(130, 1280, 128, planes, 0.6, seed=91 + planes, offset_mode=off)[0]]
    rng = np.random.default_rng(m)
    xs = [synth.draw_x(rng, m, mat["k"], "student_t3") for mat in mats]
    pms = [upload_pack(mat, O.FMT_B3) for mat in mats]
    xds = [to_dev(x.view(np.uint16)).view(torch.float16) for x in xs]
    refs = [oracle_y(mat, x) for mat, x in zip(mats, xs)]
    first = []
    for rep in range(2):
        for i, (pm, xd) in enumerate(zip(pms, xds)):
            y = L.tern_gemv(pm, xd, L.TERN_F32)
            torch.cuda.synchronize()
            check_y(y, *refs[i], f"single product {i} run {rep}")
            if rep == 0:
                first.append(y.clone())
            else:
                assert torch.equal(y, first[i]), "runs differ"
    ys = [torch.empty((m, pm.n), dtype=torch.float32, device="cuda") for pm in pms]
    plan = L.Plan(pms, xds, ys, y_dtype=L.TERN_F32)
    prev = None
    for rep in range(2):
        plan.run()
        torch.cuda.synchronize()
        for i, y in enumerate(ys):
            check_y(y, *refs[i], f"plan product {i} run {rep}")
        if prev is not None:
            assert all(torch.equal(a, b) for a, b in zip(prev, ys)), "plan runs differ"
        prev = [y.clone() for y in ys]


@pytest.mark.parametrize("m", [9, 17, 32, 33, 63])
def test_gemv_m_chunks(m):
    say("gemv chunks", m)
    mat, _ = small_matrix(100, 1024, 128, 2, 0.1, seed=m)
    _gemv_case(mat, O.FMT_2BIT, m, f32=True, seed=m)
    _gemv_case(mat, O.FMT_B3, m, seed=m)


def test_gemv_single():
    say("gemv single")
    mat = synth.workload_matrix("single_gemv")
    _gemv_case(mat, O.FMT_2BIT, 1, seed=0)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_qwen3_4b_layer(fmt):
    for proj in range(7):
        say("gemv qwen3-4b layer", proj, fmt)
        mat = synth.workload_matrix("qwen3_4b_layer", proj)
        rel = _gemv_case(mat, fmt, 1, seed=proj)
        say("  max |err|/B", rel)


@pytest.mark.parametrize("fmt,m,f32", [(O.FMT_2BIT, 1, False), (O.FMT_2BIT, 8, True),
                                       (O.FMT_B3, 1, True), (O.FMT_B3, 8, False)])
def test_gemv_down_proj_stress(fmt, m, f32):
    say("gemv down-proj stress", fmt, m, f32)
    mat = synth.workload_matrix("down_proj_stress")
    _gemv_case(mat, fmt, m, x_law="student_t3", f32=f32, seed=5)


@pytest.mark.parametrize("m", [1, 4, 16])
def test_gemv_qwen3_8b_layer(m):
    for proj in range(7):
        say("gemv qwen3-8b layer", proj, m)
        mat = synth.workload_matrix("qwen3_8b_layer", proj)
        _gemv_case(mat, O.FMT_B3, m, seed=10 * m + proj)


@pytest.mark.parametrize("route", ["auto", "stream"])
def test_gemv_zero_and_sign_invariants(route):
    with b3_route(route):
        _invariants_case()


def _invariants_case():
    import torch
    say("gemv invariants")
    mat, rng = small_matrix(200, 1280, 128, 3, 0.2, seed=12, offset_mode=O.OFF_ROW)
    x = synth.draw_x(rng, 2, 1280, "normal")
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    for fmt in FMTS:
        pm = upload_pack(mat, fmt)
        y1 = L.tern_gemv(pm, xd, L.TERN_F32)
        y2 = L.tern_gemv(pm, xd, L.TERN_F32)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), "run-to-run results differ"
        neg = dict(mat, trits=-mat["trits"], offset=-mat["offset"])
        yn = L.tern_gemv(upload_pack(neg, fmt), xd, L.TERN_F32)
        assert torch.equal(yn, -y1), "sign flip is not exact"
        zero = dict(mat, trits=np.zeros_like(mat["trits"]), offset=None, offset_mode=O.OFF_NONE)
        yz = L.tern_gemv(upload_pack(zero, fmt), xd, L.TERN_F16)
        assert not yz.any(), "all-zero trits must give exactly zero"


def test_gemv_degenerate_shapes():
    import torch
    say("gemv degenerate")
    for (n, k) in [(1, 64), (0, 128), (5, 0)]:
        mat, rng = small_matrix(n, k, 64, 1, 0.0, seed=n + k)
        pm = upload_pack(mat, O.FMT_2BIT)
        x = synth.draw_x(rng, 2, k, "normal")
        xd = to_dev(x.view(np.uint16)).view(torch.float16) if k else torch.zeros((2, 64), dtype=torch.float16, device="cuda")
        y = torch.full((2, max(n, 1)), 7.0, dtype=torch.float32, device="cuda")
        L.tern_gemv(pm, xd, L.TERN_F32, out=y)
        torch.cuda.synchronize()
        if n == 0:
            assert (y == 7.0).all()
        elif k == 0:
            assert not y.any()
        else:
            y_ref, b = oracle_y(mat, x)
            check_y(y, y_ref, b, "n=1")


@pytest.mark.parametrize("fmt,route", FMT_ROUTES)
def test_batched_and_plan_match_oracle(fmt, route):
    with b3_route(route):
        _batched_and_plan_case(fmt)


def _batched_and_plan_case(fmt):
    """The 4B-class layer through one grouped launch and through a plan (whose
    2-bit residual entries come from a plan-time index and are added in entry
    order after the K parts are combined, so its rounding may differ from the
    batched call): both within the bound; a plan is bitwise reproducible."""
    import torch
    say("batched", fmt)
    mats, pms, xs, ys, refs = [], [], [], [], []
    for proj in range(7):
        mat = synth.workload_matrix("qwen3_4b_layer", proj)
        x = synth.workload_x("qwen3_4b_layer", 1, proj)
        mats.append(mat)
        pms.append(upload_pack(mat, fmt))
        xs.append(to_dev(x.view(np.uint16)).view(torch.float16))
        ys.append(torch.empty((1, mat["n"]), dtype=torch.float16, device="cuda"))
        refs.append(oracle_y(mat, x))
    L.tern_gemv_batched(pms, xs, ys)
    torch.cuda.synchronize()
    for y, (y_ref, b) in zip(ys, refs):
        check_y(y, y_ref, b, "batched")
    plan = L.Plan(pms, xs, ys)
    first = None
    for _ in range(3):
        for y in ys:
            y.zero_()
        plan.run()
        torch.cuda.synchronize()
        if first is None:
            first = [y.clone() for y in ys]
            for y, (y_ref, b) in zip(ys, refs):
                check_y(y, y_ref, b, "plan")
        else:
            for y, f in zip(ys, first):
                assert torch.equal(y, f), "plan runs differ"


@pytest.mark.parametrize("n,k,frac,m", [(40, 1024, 1.0, 1), (200, 4096, 0.5, 1), (33, 9728, 0.1, 2),
                                         (130, 2560, 0.1, 8)])
def test_plan_residual_index_edges(n, k, frac, m):
    """Plans on ragged row counts, tiles whose entries exceed the plan index's
    capacity (every group residual), K shared by 2 and 4 wavefronts, and
    several activation rows, against the oracle."""
    import torch
    rng = np.random.default_rng(n * 7 + k)
    mat = synth.make_matrix(n, k, 128, 2, frac, rng=rng)
    x = synth.draw_x(rng, m, k, "normal")
    pm = upload_pack(mat, O.FMT_2BIT)
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    say("plan edges", n, k, frac, m)
    plan = L.Plan([pm], [xd], [y])
    plan.run()
    torch.cuda.synchronize()
    y_ref, b = oracle_y(mat, x)
    check_y(y, y_ref, b, f"plan n={n} k={k} frac={frac} m={m}")


# ----------------------------------------------------------------- MFMA product
def _gemm_case(mat, fmt, m, x_law="normal", f32=False, seed=0):
    import torch
    rng = np.random.default_rng(seed)
    x = synth.draw_x(rng, m, mat["k"], x_law)
    pm = upload_pack(mat, fmt)
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    y = L.tern_gemm(pm, xd, _ydt(f32))
    torch.cuda.synchronize()
    y_ref, b = oracle_y(mat, x)
    return check_y(y, y_ref, b, f"gemm n={mat['n']} k={mat['k']} fmt={fmt} m={m}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SMALL_SHAPES)
@pytest.mark.parametrize("m", [1, 64, 130, 257])
def test_gemm_small(shape, fmt, m):
    n, k, g, planes, frac, off = shape
    say("gemm small", shape, fmt, m)
    mat, _ = small_matrix(n, k, g, planes, frac, seed=11 * n + k, offset_mode=off, scale_law="lognormal")
    _gemm_case(mat, fmt, m, x_law="student_t3", seed=m, f32=(m == 130))


@pytest.mark.parametrize("m", [64, 512])
def test_gemm_qwen3_8b_layer(m):
    for proj in range(7):
        say("gemm qwen3-8b layer", proj, m)
        mat = synth.workload_matrix("qwen3_8b_layer", proj)
        _gemm_case(mat, O.FMT_B3, m, seed=100 * m + proj)


def test_gemm_down_proj_stress():
    say("gemm down-proj stress")
    mat = synth.workload_matrix("down_proj_stress")
    _gemm_case(mat, O.FMT_2BIT, 8, x_law="student_t3", f32=True, seed=55)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,f32", [(64, False), (200, True), (300, False)])
def test_grouped_gemm_matches_oracle(fmt, m, f32):
    """Products with different K, row counts, residual planes and offset modes
    in one matrix-core launch (batched call and plan): every output within the
    bound of the oracle; plan runs bitwise reproducible."""
    import torch
    say("grouped gemm", fmt, m, f32)
    shapes = [(130, 1280, 128, 3, 0.2, O.OFF_ROW), (7, 2560, 128, 2, 0.1, O.OFF_NONE),
              (64, 128, 128, 2, 1.0, O.OFF_NONE), (300, 4096, 128, 1, 0.0, O.OFF_GROUP)]
    mats, pms, xs, ys, refs = [], [], [], [], []
    rng = np.random.default_rng(1000 + m)
    for i, (n, k, g, planes, frac, off) in enumerate(shapes):
        mat, _ = small_matrix(n, k, g, planes, frac, seed=7 * i + m, offset_mode=off, scale_law="lognormal")
        x = synth.draw_x(rng, m, k, "student_t3")
        mats.append(mat)
        pms.append(upload_pack(mat, fmt))
        xs.append(to_dev(x.view(np.uint16)).view(torch.float16))
        ys.append(torch.empty((m, n), dtype=torch.float32 if f32 else torch.float16, device="cuda"))
        refs.append(oracle_y(mat, x))
    L.tern_gemv_batched(pms, xs, ys, _ydt(f32))
    torch.cuda.synchronize()
    for y, (y_ref, b) in zip(ys, refs):
        check_y(y, y_ref, b, f"grouped gemm m={m}")
    plan = L.Plan(pms, xs, ys, _ydt(f32))
    first = None
    for _ in range(2):
        for y in ys:
            y.zero_()
        plan.run()
        torch.cuda.synchronize()
        if first is None:
            first = [y.clone() for y in ys]
            for y, (y_ref, b) in zip(ys, refs):
                check_y(y, y_ref, b, f"grouped gemm plan m={m}")
        else:
            for y, f in zip(ys, first):
                assert torch.equal(y, f), "plan runs differ"


SMALL_BATCHES = {
    128: [(130, 1280, 128, 3, 0.2, O.OFF_ROW), (7, 2560, 128, 2, 0.1, O.OFF_NONE),
          (64, 128, 128, 2, 1.0, O.OFF_NONE), (300, 4096, 128, 1, 0.0, O.OFF_GROUP)],
    64: [(65, 640, 64, 2, 0.3, O.OFF_GROUP), (128, 64, 64, 1, 0.0, O.OFF_NONE),
         (33, 3200, 64, 2, 0.5, O.OFF_ROW), (200, 1024, 64, 3, 0.15, O.OFF_NONE)],
}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("group", [128, 64])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 9, 16, 17, 32, 33, 40])
def test_small_m_batches_match_oracle(fmt, group, m):
    """Batched calls and plans at m <= 63 (the decode kernels up to 2 rows
    for base-3 and 5 (group 128) or 4 (group 64) for 2-bit; the 16-row
    matrix-core product with K split into step ranges and a grouped reduce
    up to 32; the 128-row tiles above):
    single-step, odd-step and split products, ragged rows, 1-3 planes, every
    offset mode, against the oracle."""
    import torch
    say("small m batch", fmt, group, m)
    mats, pms, xs, ys, refs = [], [], [], [], []
    rng = np.random.default_rng(2000 + 7 * m + group)
    f32 = m in (9, 40)
    for i, (n, k, g, planes, frac, off) in enumerate(SMALL_BATCHES[group]):
        mat, _ = small_matrix(n, k, g, planes, frac, seed=31 * i + m + group, offset_mode=off, scale_law="lognormal")
        x = synth.draw_x(rng, m, k, "student_t3")
        mats.append(mat)
        pms.append(upload_pack(mat, fmt))
        xs.append(to_dev(x.view(np.uint16)).view(torch.float16))
        ys.append(torch.empty((m, n), dtype=torch.float32 if f32 else torch.float16, device="cuda"))
        refs.append(oracle_y(mat, x))
    L.tern_gemv_batched(pms, xs, ys, _ydt(f32))
    torch.cuda.synchronize()
    for y, (y_ref, b) in zip(ys, refs):
        check_y(y, y_ref, b, f"small batch m={m}")
    plan = L.Plan(pms, xs, ys, _ydt(f32))
    first = None
    for _ in range(2):
        for y in ys:
            y.zero_()
        plan.run()
        torch.cuda.synchronize()
        if first is None:
            first = [y.clone() for y in ys]
            for y, (y_ref, b) in zip(ys, refs):
                check_y(y, y_ref, b, f"small plan m={m}")
        else:
            for y, f in zip(ys, first):
                assert torch.equal(y, f), "plan runs differ"


LONG_K_BATCH = [(96, 9728, 2, 0.2, O.OFF_ROW), (50, 5120, 1, 0.0, O.OFF_GROUP),
                (130, 12288, 3, 0.1, O.OFF_NONE), (70, 14336, 2, 0.3, O.OFF_ROW), (64, 1024, 2, 0.5, O.OFF_NONE)]


@pytest.mark.parametrize("group", [128, 64])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5])
def test_decode_batch_k_parts_match_oracle(group, m):
    """2-bit batched calls and plans on the matrix-core decode kernel with
    products longer than one workgroup stages at m activation rows: those
    are cut into K parts whose FP32 partials a grouped reduce sums, beside
    products that are not; ragged rows, 1-3 planes, offsets, against the
    oracle, and plans bitwise reproducible."""
    import torch
    say("decode batch k parts", group, m)
    mats, pms, xs, ys, refs = [], [], [], [], []
    rng = np.random.default_rng(4000 + 3 * m + group)
    for i, (n, k, planes, frac, off) in enumerate(LONG_K_BATCH):
        mat, _ = small_matrix(n, k, group, planes, frac, seed=53 * i + m + group, offset_mode=off, scale_law="lognormal")
        x = synth.draw_x(rng, m, k, "student_t3")
        pms.append(upload_pack(mat, O.FMT_2BIT))
        xs.append(to_dev(x.view(np.uint16)).view(torch.float16))
        ys.append(torch.empty((m, n), dtype=torch.float16, device="cuda"))
        refs.append(oracle_y(mat, x))
    L.tern_gemv_batched(pms, xs, ys)
    torch.cuda.synchronize()
    for i, (y, (y_ref, b)) in enumerate(zip(ys, refs)):
        check_y(y, y_ref, b, f"k-part batch m={m} i={i}")
    plan = L.Plan(pms, xs, ys)
    first = None
    for _ in range(2):
        for y in ys:
            y.zero_()
        plan.run()
        torch.cuda.synchronize()
        if first is None:
            first = [y.clone() for y in ys]
            for i, (y, (y_ref, b)) in enumerate(zip(ys, refs)):
                check_y(y, y_ref, b, f"k-part plan m={m} i={i}")
        else:
            for y, f in zip(ys, first):
                assert torch.equal(y, f), "plan runs differ"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 2])
def test_single_product_batches_fill_the_gpu(fmt, m):
    """A batch or plan of one product cuts it into enough K parts to fill
    the GPU (FP32 partials, grouped reduce): the down-projection stress
    matrix (three planes, row offsets, log-normal scales, Student-t x) and a
    7-row matrix whose parts are single blocks, against the oracle."""
    import torch
    say("single product fill", fmt, m)
    cases = [(synth.workload_matrix("down_proj_stress"), "student_t3"),
             (small_matrix(7, 2560, 128, 2, 0.3, seed=77 + m, offset_mode=O.OFF_GROUP)[0], "normal")]
    rng = np.random.default_rng(500 + m + 10 * fmt)
    for ci, (mat, law) in enumerate(cases):
        x = synth.draw_x(rng, m, mat["k"], law)
        pm = upload_pack(mat, fmt)
        xd = to_dev(x.view(np.uint16)).view(torch.float16)
        y_ref, b = oracle_y(mat, x)
        y = torch.empty((m, mat["n"]), dtype=torch.float16, device="cuda")
        L.tern_gemv_batched([pm], [xd], [y])
        torch.cuda.synchronize()
        check_y(y, y_ref, b, f"single batched case={ci} m={m}")
        y.zero_()
        plan = L.Plan([pm], [xd], [y])
        plan.run()
        torch.cuda.synchronize()
        check_y(y, y_ref, b, f"single plan case={ci} m={m}")


@pytest.mark.parametrize("group", [128, 64])
@pytest.mark.parametrize("m", [1, 3, 5])
def test_dense_residual_lists_in_windows(group, m):
    """Residual planes listed from the masks (no plan index) with every
    group masked: a wavefront's rows hold several windows of entries, two
    residual planes, plus a sparse matrix in the same batch; tern_gemv,
    batched call and plan, against the oracle."""
    import torch
    say("dense residual windows", group, m)
    rng = np.random.default_rng(900 + m + group)
    cases = [small_matrix(48, 3072, group, 3, 1.0, seed=91 + m, offset_mode=O.OFF_ROW)[0],
             small_matrix(100, 2048, group, 2, 0.05, seed=92 + m, offset_mode=O.OFF_NONE)[0]]
    pms, xs, ys, refs = [], [], [], []
    for mat in cases:
        x = synth.draw_x(rng, m, mat["k"], "normal")
        pm = upload_pack(mat, O.FMT_2BIT)
        xd = to_dev(x.view(np.uint16)).view(torch.float16)
        y_ref, b = oracle_y(mat, x)
        y = L.tern_gemv(pm, xd, L.TERN_F32)
        torch.cuda.synchronize()
        check_y(y, y_ref, b, f"gemv dense residual m={m}")
        pms.append(pm)
        xs.append(xd)
        ys.append(torch.empty((m, mat["n"]), dtype=torch.float16, device="cuda"))
        refs.append((y_ref, b))
    L.tern_gemv_batched(pms, xs, ys)
    torch.cuda.synchronize()
    for i, (y, (y_ref, b)) in enumerate(zip(ys, refs)):
        check_y(y, y_ref, b, f"batched dense residual m={m} i={i}")
    plan = L.Plan(pms, xs, ys)
    for y in ys:
        y.zero_()
    plan.run()
    torch.cuda.synchronize()
    for i, (y, (y_ref, b)) in enumerate(zip(ys, refs)):
        check_y(y, y_ref, b, f"plan dense residual m={m} i={i}")


@pytest.mark.parametrize("fmt,route", FMT_ROUTES)
def test_plan_graph_replays_match_eager(fmt, route):
    with b3_route(route):
        _graph_replays_case(fmt)


def _graph_replays_case(fmt):
    """A plan captured into a HIP graph: a single product cut into K parts
    (its row blocks' arrival counters must be left clear by every run) and
    a seven-product layer, replayed several times with eager launches and
    synchronizations in between; every replay equals the eager result
    bitwise and meets the oracle's bound."""
    import torch
    say("plan graph replays", fmt)
    stream = torch.cuda.Stream()
    cases = []
    mat = synth.workload_matrix("down_proj_stress")
    x = synth.workload_x("down_proj_stress", 1, 0)
    cases.append(([mat], [x]))
    mats = [synth.workload_matrix("qwen3_4b_layer", proj) for proj in range(7)]
    xs = [synth.workload_x("qwen3_4b_layer", 1, proj) for proj in range(7)]
    cases.append((mats, xs))
    for ci, (ms, xh) in enumerate(cases):
        pms = [upload_pack(mt, fmt) for mt in ms]
        xd = [to_dev(x_.view(np.uint16)).view(torch.float16) for x_ in xh]
        ys = [torch.empty((1, mt["n"]), dtype=torch.float16, device="cuda") for mt in ms]
        plan = L.Plan(pms, xd, ys)
        with torch.cuda.stream(stream):
            plan.run(stream.cuda_stream)
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        for mt, x_, y in zip(ms, xh, eager):
            y_ref, b = oracle_y(mt, x_)
            check_y(y, y_ref, b, f"eager plan case={ci}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            plan.run(stream.cuda_stream)
        torch.cuda.synchronize()
        for rep in range(3):
            for y in ys:
                y.zero_()
            with torch.cuda.stream(stream):
                g.replay()
            torch.cuda.synchronize()
            for i, (y, e) in enumerate(zip(ys, eager)):
                assert torch.equal(y, e), f"graph replay {rep} differs (case {ci}, product {i})"
            plan.run()  # an eager run between replays
            torch.cuda.synchronize()
            for y, e in zip(ys, eager):
                assert torch.equal(y, e), f"eager run after replay {rep} differs (case {ci})"


def test_read_probe_runs_and_checks_arguments():
    """The measurement probe reads a buffer without touching the sink (its
    XOR is not the sentinel for a buffer of ones) and rejects sizes that are
    not a multiple of 16."""
    import torch
    say("read probe")
    buf = torch.ones(1 << 20, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    L.tern_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.sum().item()) == 0
    lib = L.load()
    st = lib.tern_read_probe(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(24), ctypes.c_void_p(sink.data_ptr()), None)
    assert st == L.TERN_E_INVAL


@pytest.mark.parametrize("m", [64, 512])
def test_grouped_qwen3_8b_layer_matches_oracle(m):
    """The 8B-class layer (base-3, seven projections) through one plan at the
    sizes the benchmark times: one grouped matrix-core launch whose long-K
    product may be cut into K parts with FP32 partials and a grouped reduce;
    every output within the bound."""
    import torch
    say("grouped qwen3-8b layer", m)
    mats, pms, xs, ys, refs = [], [], [], [], []
    for proj in range(7):
        mat = synth.workload_matrix("qwen3_8b_layer", proj)
        x = synth.workload_x("qwen3_8b_layer", m, proj)
        pms.append(upload_pack(mat, O.FMT_B3))
        xs.append(to_dev(x.view(np.uint16)).view(torch.float16))
        ys.append(torch.empty((m, mat["n"]), dtype=torch.float16, device="cuda"))
        refs.append(oracle_y(mat, x))
    plan = L.Plan(pms, xs, ys)
    plan.run()
    torch.cuda.synchronize()
    for proj, (y, (y_ref, b)) in enumerate(zip(ys, refs)):
        check_y(y, y_ref, b, f"grouped layer m={m} proj={proj}")


@pytest.mark.parametrize("fmt", FMTS)
def test_calls_on_a_caller_stream_match_current_stream(fmt):
    """tern_gemv, tern_gemv_batched and tern_unpack through the binding on a
    stream of the caller's, with the workspaces the binding allocates: the
    same bits as on torch's current stream (the zero fill of such a
    workspace is queued on torch's stream and finished before a call on
    another stream starts), and the product within the oracle's bound."""
    import torch
    say("calls on a caller stream", fmt)
    mat, rng = small_matrix(300, 2560, 128, 2, 0.2, seed=77, offset_mode=O.OFF_ROW)
    x = synth.draw_x(rng, 3, 2560, "normal")
    pm = upload_pack(mat, fmt)
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    y0 = L.tern_gemv(pm, xd)
    yb0 = [torch.empty_like(y0)]
    L.tern_gemv_batched([pm], [xd], yb0)
    t0 = L.tern_unpack(pm)
    y1, yb1, t1 = torch.empty_like(y0), [torch.empty_like(y0)], torch.empty_like(t0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    L.tern_gemv(pm, xd, out=y1, stream=s.cuda_stream)
    L.tern_gemv_batched([pm], [xd], yb1, stream=s.cuda_stream)
    L.tern_unpack(pm, out=t1, stream=s.cuda_stream)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1), "tern_gemv differs on the caller's stream"
    assert torch.equal(yb0[0], yb1[0]), "tern_gemv_batched differs on the caller's stream"
    assert torch.equal(t0, t1), "tern_unpack differs on the caller's stream"
    y_ref, b = oracle_y(mat, x)
    check_y(y1, y_ref, b, f"caller stream fmt={fmt}")


@pytest.mark.parametrize("m", [2, 4])
def test_b3_layer_plan_two_stage_parts_match_oracle(m):
    """The 8B-class layer (base-3, seven projections) through one plan at
    m = 2 and 4, as the benchmark runs it: the matrix-core stream kernel
    after the residual pass.  The layer holds more 64-row stages than the
    launch has wavefronts, so its products are cut into K parts of two
    stages whose FP32 partials the row block's last part sums; every output
    within the bound, and two runs bitwise equal."""
    import torch
    say("b3 layer plan, two-stage K parts", m)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mats, pms, xs, ys, refs = [], [], [], [], []
    stages = 0
    for proj in range(7):
        mat = synth.workload_matrix("qwen3_8b_layer", proj)
        x = synth.workload_x("qwen3_8b_layer", m, proj)
        stages += -(-mat["n"] // 64) * -(-mat["k"] // 1024)
        pms.append(upload_pack(mat, O.FMT_B3))
        xs.append(to_dev(x.view(np.uint16)).view(torch.float16))
        ys.append(torch.empty((m, mat["n"]), dtype=torch.float16, device="cuda"))
        refs.append(oracle_y(mat, x))
    assert stages > 7 * cus, (stages, cus)
    plan = L.Plan(pms, xs, ys)
    first = None
    for _ in range(2):
        for y in ys:
            y.zero_()
        plan.run()
        torch.cuda.synchronize()
        if first is None:
            first = [y.clone() for y in ys]
            for proj, (y, (y_ref, b)) in enumerate(zip(ys, refs)):
                check_y(y, y_ref, b, f"b3 layer plan m={m} proj={proj}")
        else:
            for y, f in zip(ys, first):
                assert torch.equal(y, f), "plan runs differ"


@pytest.mark.timeout(600)
def test_qwen3_8b_stack_plan_matches_oracle():
    """The 8B-class stack at M=1 as the benchmark builds and runs it: 36
    distinct seeded layers x 7 base-3 projections in one plan, q/k/v and
    gate/up reading one activation vector each.  Layers 0, 17 and 35 are
    checked against the oracle's outputs (every projection, every row); in
    the other 33 layers 32 seeded rows of every projection are checked one
    by one (the oracle's definition restricted to those rows); every output
    of every layer is finite."""
    import torch
    import bench
    say("qwen3-8b stack plan: drawing and packing 36 layers")
    mats, xs, ys = bench.build_stack8b()
    plan = L.Plan(mats, xs, ys)
    plan.run()
    torch.cuda.synchronize()
    nproj = len(synth.QWEN3_8B_LAYER)
    for y in ys:
        assert torch.isfinite(y.float()).all()
    for layer in (0, 17, 35):
        for proj in range(nproj):
            say("  oracle layer", layer, "proj", proj)
            mat = synth.workload_matrix("qwen3_8b_stack", proj, layer)
            x = synth.workload_x("qwen3_8b_stack", 1, synth.LAYER_INPUT[proj], layer)
            assert np.array_equal(xs[layer * nproj + proj].cpu().numpy().view(np.uint16), x.view(np.uint16))
            y_ref, b = oracle_y(mat, x)
            check_y(ys[layer * nproj + proj], y_ref, b, f"stack layer {layer} proj {proj}")
            del mat
    from concurrent.futures import ThreadPoolExecutor

    def sampled(layer):
        rng = np.random.default_rng([4, layer])
        out = []
        for proj in range(nproj):
            mat = synth.workload_matrix("qwen3_8b_stack", proj, layer)
            x = synth.workload_x("qwen3_8b_stack", 1, synth.LAYER_INPUT[proj], layer)
            rows = np.sort(rng.choice(mat["n"], 32, replace=False))
            sub = dict(mat, trits=mat["trits"][:, rows], scales=mat["scales"][:, rows],
                       masks=[mk[rows] for mk in mat["masks"]])
            out.append((proj, rows, *oracle_y(sub, x)))
            del mat, sub
        return layer, out

    rest = [layer for layer in range(len(ys) // nproj) if layer not in (0, 17, 35)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        for layer, out in ex.map(sampled, rest):
            say("  sampled rows, layer", layer)
            for proj, rows, y_ref, b in out:
                y = ys[layer * nproj + proj][:, torch.from_numpy(rows).cuda()]
                check_y(y, y_ref, b, f"stack layer {layer} proj {proj} (sampled rows)")


@pytest.mark.parametrize("fmt,route", FMT_ROUTES)
def test_plan_recreated_after_repack(fmt, route):
    with b3_route(route):
        _recreate_case(fmt)


def _recreate_case(fmt):
    """A plan keeps tables derived from the packed matrices (the residual
    index built from masks, row pointers and residual scales), so after the
    buffers are packed again with other contents a new plan is created: it
    must match the oracle for the new contents, as the first plan did for
    the old ones."""
    import torch
    say("plan re-created after re-pack", fmt)
    n, k, g = 300, 1280, 128
    mat_a, _ = small_matrix(n, k, g, 2, 0.2, seed=71, offset_mode=O.OFF_GROUP)
    mat_b, _ = small_matrix(n, k, g, 2, 0.2, seed=72, offset_mode=O.OFF_GROUP)
    assert [int(m.sum()) for m in mat_a["masks"]] == [int(m.sum()) for m in mat_b["masks"]]
    assert not np.array_equal(mat_a["masks"][0], mat_b["masks"][0])
    pm = upload_pack(mat_a, fmt)
    x = synth.draw_x(np.random.default_rng(5), 1, k, "normal")
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    y = torch.empty((1, n), dtype=torch.float16, device="cuda")
    plan = L.Plan([pm], [xd], [y])
    plan.run()
    torch.cuda.synchronize()
    check_y(y, *oracle_y(mat_a, x), "plan on the first packing")
    # pack the second matrix into the same buffers, then a new plan
    masks = to_dev(np.stack(mat_b["mask_bits"]).view(np.int32))
    L.tern_pack(pm, to_dev(mat_b["trits"]), to_dev(mat_b["scales"]), masks, to_dev(mat_b["offset"]))
    torch.cuda.synchronize()
    del plan
    plan = L.Plan([pm], [xd], [y])
    plan.run()
    torch.cuda.synchronize()
    check_y(y, *oracle_y(mat_b, x), "new plan after re-packing")
