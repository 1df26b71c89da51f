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
