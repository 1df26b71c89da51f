"""GPU parity of the activation rotation (tern_rotate) against the oracle in
oracle/rotate_oracle.py: orthogonal blocks of 64 and 128, ragged row counts,
within the bound; identity blocks copy x bit for bit; in place equals out of
place."""
import numpy as np
import pytest

import oracle as O
import oracle.rotate_oracle as Rt
from ternary_weight_only_tern_amd import lib as L
from ternary_weight_only_tern_amd import synth
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _dev16(a):
    import torch
    return to_dev(np.ascontiguousarray(a).view(np.uint16)).view(torch.float16)


@pytest.mark.parametrize("m,k,block,law", [(1, 4096, 128, "normal"), (5, 2560, 128, "student_t3"),
                                           (17, 1024, 64, "normal"), (33, 384, 64, "student_t3"),
                                           (16, 9728, 128, "normal")])
def test_rotate_matches_oracle(m, k, block, law):
    import torch
    say("rotate", m, k, block, law)
    rng = np.random.default_rng(m * 7 + k + block)
    R = synth.draw_rotation(rng, k // block, block)
    x = synth.draw_x(rng, m, k, law)
    y = L.tern_rotate(_dev16(R), _dev16(x))
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    ref = Rt.rotate(R, x)
    b = Rt.rotate_bound(R, x)
    ok = np.isfinite(got) & (np.abs(got - ref) <= 2e-3 * b)
    assert ok.all(), f"{int((~ok).sum())} outputs outside the bound; worst {np.max(np.abs(got - ref) / np.maximum(b, 1e-30))}"


def test_rotate_identity_and_in_place():
    import torch
    say("rotate identity / in place")
    rng = np.random.default_rng(9)
    k, block = 512, 128
    x = synth.draw_x(rng, 3, k, "student_t3")
    eye = np.stack([np.eye(block, dtype=np.float16)] * (k // block))
    y = L.tern_rotate(_dev16(eye), _dev16(x))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint16), x.view(np.uint16))
    R = synth.draw_rotation(rng, k // block, block)
    Rd = _dev16(R)
    xd = _dev16(x)
    out = L.tern_rotate(Rd, xd)
    L.tern_rotate(Rd, xd, out=xd)
    torch.cuda.synchronize()
    assert torch.equal(out, xd)


def test_rotate_batched_equals_single_launches():
    """A layer's three inputs (K = 2560, 4096, 9728) and a ragged fourth in one
    launch equal separate tern_rotate calls bit for bit, at M = 1 and 20."""
    import torch
    say("rotate batched")
    rng = np.random.default_rng(21)
    for m in (1, 20):
        Rs, xs = [], []
        for k in (2560, 4096, 9728, 384):
            Rs.append(_dev16(synth.draw_rotation(rng, k // 128, 128)))
            xs.append(_dev16(synth.draw_x(rng, m, k, "normal")))
        outs = L.tern_rotate_batched(Rs, xs)
        singles = [L.tern_rotate(R, x) for R, x in zip(Rs, xs)]
        torch.cuda.synchronize()
        for o, s_ in zip(outs, singles):
            assert torch.equal(o, s_)


def test_rotate_batched_eight_inputs_empty_input_and_graph_replays():
    """The most inputs one launch takes (8, block 64, one of them with K = 0,
    which the call skips) at a ragged M = 19 equals separate launches bit for
    bit; the same call captured into a graph and replayed after the inputs
    change (eager work and synchronisations between replays) equals the eager
    call on every replay."""
    import torch
    say("rotate batched: 8 inputs, K = 0, graph replays")
    rng = np.random.default_rng(33)
    m, block = 19, 64
    ks = (64, 128, 320, 0, 1024, 2560, 192, 4096)
    Rs = [_dev16(synth.draw_rotation(rng, k // block, block)) if k else
          torch.empty((0, block, block), dtype=torch.float16, device="cuda") for k in ks]
    xs = [_dev16(synth.draw_x(rng, m, k, "student_t3")) if k else
          torch.empty((m, 0), dtype=torch.float16, device="cuda") for k in ks]
    outs = L.tern_rotate_batched(Rs, xs)
    singles = [L.tern_rotate(R, x) if x.shape[1] else torch.empty_like(x) for R, x in zip(Rs, xs)]
    torch.cuda.synchronize()
    for o, s_ in zip(outs, singles):
        assert torch.equal(o, s_)
    for o, R, x in zip(outs, Rs, xs):  # one of them against the oracle as well
        if x.shape[1] == 2560:
            got = o.cpu().numpy().astype(np.float64)
            Rh, xh = R.cpu().numpy(), x.cpu().numpy()
            assert (np.abs(got - Rt.rotate(Rh, xh)) <= 2e-3 * Rt.rotate_bound(Rh, xh)).all()

    gouts = [torch.empty_like(x) for x in xs]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        L.tern_rotate_batched(Rs, xs, gouts, stream.cuda_stream)  # warm the call once outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            L.tern_rotate_batched(Rs, xs, gouts, stream.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in xs:
            if x.shape[1]:
                x.copy_(_dev16(synth.draw_x(rng, m, x.shape[1], "normal")))
        want = L.tern_rotate_batched(Rs, xs)
        torch.cuda.synchronize()
        for o in gouts:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for g, w_ in zip(gouts, want):
            assert torch.equal(g, w_), f"replay {rep} differs from the eager call"


@pytest.mark.parametrize("fmt,m,route,block", [(O.FMT_B3, 1, "stream", 128), (O.FMT_B3, 4, "stream", 64),
                                               (O.FMT_B3, 1, "auto", 128), (O.FMT_2BIT, 1, "auto", 128),
                                               (O.FMT_2BIT, 8, "auto", 64), (O.FMT_B3, 64, "auto", 128)])
def test_rotated_plan_matches_oracle(fmt, m, route, block):
    """Rotate-then-product through one plan (tern_plan_create_rotated): on the
    base-3 stream kernel the rotation runs inside the activation preparation;
    on the other routes rotation launches precede the product.  Two products
    share one x and its rotation, one takes another rotation, one takes its x
    unrotated.  Checked against the oracle's rotation followed by its product:
    |y - y_ref| <= 2e-3 * B(|xr|) + 2.004e-3 * B(sum_j |R||x|), the product's
    bound on the exact rotated x plus the rotation's own bound carried through
    the weights; run twice, bit-identical."""
    import torch
    from gpu_util import b3_route, check_y, oracle_y, small_matrix, upload_pack
    say("rotated plan", fmt, m, route, block)
    rng = np.random.default_rng(m + block)
    mats = [small_matrix(300, 2560, 128, 2, 0.3, seed=41, offset_mode=O.OFF_GROUP)[0],
            small_matrix(130, 2560, 128, 2, 0.1, seed=42)[0],
            small_matrix(200, 1280, 128, 3, 0.2, seed=43, offset_mode=O.OFF_ROW)[0],
            small_matrix(64, 1024, 128, 1, 0.0, seed=44)[0]]
    xa = synth.draw_x(rng, m, 2560, "normal")
    xc = synth.draw_x(rng, m, 1280, "student_t3")
    xd = synth.draw_x(rng, m, 1024, "normal")
    R1 = synth.draw_rotation(rng, 2560 // block, block)
    R2 = synth.draw_rotation(rng, 1280 // block, block)
    xs_h = [xa, xa, xc, xd]
    rots_h = [R1, R1, R2, None]
    with b3_route(route):
        pms = [upload_pack(mt, fmt) for mt in mats]
        xa_d, xc_d, xd_d = _dev16(xa), _dev16(xc), _dev16(xd)
        xs = [xa_d, xa_d, xc_d, xd_d]
        R1d, R2d = _dev16(R1), _dev16(R2)
        rots = [R1d, R1d, R2d, None]
        ys = [torch.empty((m, mt["n"]), dtype=torch.float32, device="cuda") for mt in mats]
        plan = L.Plan(pms, xs, ys, y_dtype=L.TERN_F32, rots=rots, rot_block=block)
        say("launches per run:", plan.launches())
        plan.run()
        torch.cuda.synchronize()
        first = [y.clone() for y in ys]
        plan.run()
        torch.cuda.synchronize()
    for i, (mt, x, R) in enumerate(zip(mats, xs_h, rots_h)):
        assert torch.equal(ys[i], first[i]), "runs differ"
        if R is None:
            y_ref, b = oracle_y(mt, x)
        else:
            xr = Rt.rotate(R, x)
            y_ref, b1 = oracle_y(mt, xr)
            _, b2 = oracle_y(mt, Rt.rotate_bound(R, x))
            b = b1 + 1.002 * b2
        check_y(ys[i], y_ref, b, f"rotated plan product {i}")


@pytest.mark.parametrize("m", [1, 3])
def test_rotated_stream_plan_group64_block128(m):
    """Base-3 stream route at group 64 with 128 x 128 rotation blocks: the
    preparation works in spans of 128 positions, so an unrotated product with
    k = 960 (7.5 spans) ends inside its last span; two rotated products (k =
    1024 and 1536) and the unrotated one, against the oracle as above."""
    import torch
    from gpu_util import b3_route, small_matrix, upload_pack
    say("rotated stream plan, group 64, block 128, m =", m)
    rng = np.random.default_rng(90 + m)
    mats = [small_matrix(130, 1024, 64, 2, 0.2, seed=91, offset_mode=O.OFF_GROUP)[0],
            small_matrix(100, 960, 64, 1, 0.0, seed=92, offset_mode=O.OFF_ROW)[0],
            small_matrix(70, 1536, 64, 3, 0.1, seed=93)[0]]
    xs_h = [synth.draw_x(rng, m, mt["k"], "student_t3") for mt in mats]
    rots_h = [synth.draw_rotation(rng, 1024 // 128, 128), None, synth.draw_rotation(rng, 1536 // 128, 128)]
    with b3_route("stream"):
        pms = [upload_pack(mt, O.FMT_B3) for mt in mats]
        xs = [_dev16(x) for x in xs_h]
        rots = [None if R is None else _dev16(R) for R in rots_h]
        ys = [torch.empty((m, mt["n"]), dtype=torch.float32, device="cuda") for mt in mats]
        plan = L.Plan(pms, xs, ys, y_dtype=L.TERN_F32, rots=rots, rot_block=128)
        plan.run()
        torch.cuda.synchronize()
        first = [y.clone() for y in ys]
        plan.run()
        torch.cuda.synchronize()
    for y, f in zip(ys, first):
        assert torch.equal(y, f), "runs differ"
    _check_rotated(ys, mats, xs_h, rots_h, "rotated stream plan")


def test_rotated_plan_rejects_mixed_rotations():
    """Products that read one x with different rotations are refused."""
    import torch
    from gpu_util import small_matrix, upload_pack
    say("rotated plan: mixed rotations")
    rng = np.random.default_rng(3)
    mats = [small_matrix(64, 1024, 128, 1, 0.0, seed=s)[0] for s in (1, 2)]
    pms = [upload_pack(mt, O.FMT_2BIT) for mt in mats]
    x = _dev16(synth.draw_x(rng, 1, 1024, "normal"))
    R1, R2 = (_dev16(synth.draw_rotation(rng, 8, 128)) for _ in range(2))
    ys = [torch.empty((1, 64), dtype=torch.float16, device="cuda") for _ in range(2)]
    with pytest.raises(L.TernError):
        L.Plan(pms, [x, x], ys, rots=[R1, R2])


# the folded rotation's counters at the start of a rotated plan's workspace:
# 65 lines of 256 bytes (shares and groups counted, give-up word; 64 copies
# of the ready flag with their groups' counts)
ROT_SYNC_BYTES = (65 + 16) * 256  # flag lines and the share sub-counts


def _rotated_layer(rng, group, block, ks, m, fmt):
    """Products with rotated inputs: for each k in ks a product of that depth
    (some with residual planes and offsets), one distinct x and R per k,
    plus a product that shares the first x and R and one unrotated
    product."""
    from gpu_util import small_matrix, upload_pack
    mats, xs_h, rots_h = [], [], []
    for i, k in enumerate(ks):
        mt = small_matrix(96 + 40 * i, k, group, 1 + i % 3, 0.2, seed=60 + i,
                          offset_mode=(O.OFF_NONE, O.OFF_ROW, O.OFF_GROUP)[i % 3])[0]
        mats.append(mt)
        xs_h.append(synth.draw_x(rng, m, k, ("normal", "student_t3")[i % 2]))
        rots_h.append(synth.draw_rotation(rng, k // block, block))
    mats.append(small_matrix(70, ks[0], group, 2, 0.1, seed=70)[0])
    xs_h.append(xs_h[0])
    rots_h.append(rots_h[0])
    mats.append(small_matrix(64, ks[-1], group, 1, 0.0, seed=71)[0])
    xs_h.append(synth.draw_x(rng, m, ks[-1], "normal"))
    rots_h.append(None)
    pms = [upload_pack(mt, fmt) for mt in mats]
    return mats, xs_h, rots_h, pms


def _check_rotated(ys, mats, xs_h, rots_h, what):
    from gpu_util import check_y, oracle_y
    for i, (mt, x, R) in enumerate(zip(mats, xs_h, rots_h)):
        if R is None:
            y_ref, b = oracle_y(mt, x)
        else:
            y_ref, b1 = oracle_y(mt, Rt.rotate(R, x))
            _, b2 = oracle_y(mt, Rt.rotate_bound(R, x))
            b = b1 + 1.002 * b2
        check_y(ys[i], y_ref, b, f"{what}: product {i}")


@pytest.mark.parametrize("group,m,block,ks", [(128, 1, 128, (2560, 4096, 9728)), (128, 2, 64, (1408, 2560)),
                                              (128, 5, 128, (1024, 3072)), (64, 4, 64, (1344, 640, 2048)),
                                              (64, 1, 128, (512, 1536))])
def test_rotated_plan_folded_into_decode_launch(group, m, block, ks):
    """2-bit plans on the decode route rotate inside the product's own launch
    (tern_plan_launches == 1): the launch's first workgroups rotate, the
    others wait for the rotated activations.  Against the oracle's rotation
    followed by its product (bound as above), with a ragged last share (k =
    1344 = 21 * 64 at block 64), several inputs, one x shared by two
    products and one unrotated product; five eager runs bit-identical; the
    plan captured in a graph and replayed after the inputs change (eager
    work between replays) equals the eager run every time; the wait never
    gave up (the workspace's give-up word stays zero)."""
    import torch
    say("folded rotation", group, m, block, ks)
    rng = np.random.default_rng(group + m + block + len(ks))
    mats, xs_h, rots_h, pms = _rotated_layer(rng, group, block, ks, m, O.FMT_2BIT)
    xd = {}
    xs = [xd.setdefault(id(x), _dev16(x)) for x in xs_h]
    rd = {}
    rots = [None if R is None else rd.setdefault(id(R), _dev16(R)) for R in rots_h]
    ys = [torch.empty((m, mt["n"]), dtype=torch.float32, device="cuda") for mt in mats]
    plan = L.Plan(pms, xs, ys, y_dtype=L.TERN_F32, rots=rots, rot_block=block)
    assert plan.launches() == 1, f"{plan.launches()} launches: the rotation is not folded"
    first = None
    for rep in range(5):
        plan.run()
        torch.cuda.synchronize()
        if first is None:
            first = [y.clone() for y in ys]
        for y, f in zip(ys, first):
            assert torch.equal(y, f), f"run {rep} differs"
    _check_rotated(ys, mats, xs_h, rots_h, "folded rotation")
    sync = plan.ws[:ROT_SYNC_BYTES].cpu().numpy().view(np.uint32)
    assert not sync.any(), f"rotation counters left set at words {np.flatnonzero(sync)[:8].tolist()}"

    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        plan.run(stream.cuda_stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            plan.run(stream.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        new_h = {}
        for key, x in xd.items():
            fresh = synth.draw_x(rng, m, x.shape[1], "normal")
            x.copy_(_dev16(fresh))
            new_h[key] = fresh
        plan.run()
        torch.cuda.synchronize()
        want = [y.clone() for y in ys]
        for y in ys:
            y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (y, w_) in enumerate(zip(ys, want)):
            assert torch.equal(y, w_), f"replay {rep}: product {i} differs from the eager run"
    _check_rotated(ys, mats, [new_h[id(x)] for x in xs_h], rots_h, "folded rotation after replays")
    sync = plan.ws[:ROT_SYNC_BYTES].cpu().numpy().view(np.uint32)
    assert not sync.any(), f"rotation counters left set at words {np.flatnonzero(sync)[:8].tolist()}"
