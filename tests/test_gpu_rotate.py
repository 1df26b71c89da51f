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
