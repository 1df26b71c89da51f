"""Pins of the rotation oracle (oracle/rotate_oracle.py): the orientation on a
hand-worked block, identity and permutation blocks, the dense block-diagonal
product (scipy), norm preservation and the inverse for orthogonal blocks."""
import numpy as np
import scipy.linalg

import oracle.rotate_oracle as Rt
from ternary_weight_only_tern_amd import synth


def test_hand_worked_block_orientation():
    # R = [[0, -1], [1, 0]] (a quarter turn) applied as R x: [1, 2] -> [-2, 1]
    R = np.array([[[0.0, -1.0], [1.0, 0.0]]])
    assert Rt.rotate(R, np.array([[1.0, 2.0]])).tolist() == [[-2.0, 1.0]]


def test_identity_and_permutation_blocks():
    rng = np.random.default_rng(1)
    x = synth.draw_x(rng, 3, 256, "normal")
    eye = np.stack([np.eye(128)] * 2)
    assert np.array_equal(Rt.rotate(eye, x), x.astype(np.float64))
    perm = rng.permutation(128)
    P = np.stack([np.eye(128)[perm]] * 2)
    y = Rt.rotate(P, x)
    assert np.array_equal(y[:, :128], x[:, :128][:, perm].astype(np.float64))
    assert np.array_equal(y[:, 128:], x[:, 128:][:, perm].astype(np.float64))


def test_matches_dense_block_diagonal_product():
    rng = np.random.default_rng(2)
    R = synth.draw_rotation(rng, 3, 64)
    x = synth.draw_x(rng, 4, 192, "student_t3")
    D = scipy.linalg.block_diag(*[r.astype(np.float64) for r in R])
    assert np.allclose(Rt.rotate(R, x), x.astype(np.float64) @ D.T, rtol=1e-12, atol=1e-12)


def test_orthogonal_blocks_preserve_norms_and_invert():
    rng = np.random.default_rng(3)
    Q = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(2)])
    x = rng.standard_normal((5, 256))
    y = Rt.rotate(Q, x)
    for b in range(2):
        seg = slice(128 * b, 128 * (b + 1))
        assert np.allclose(np.linalg.norm(y[:, seg], axis=1), np.linalg.norm(x[:, seg], axis=1), rtol=1e-12)
    back = Rt.rotate(np.transpose(Q, (0, 2, 1)), y)
    assert np.allclose(back, x, rtol=0, atol=1e-12)


def test_bound_dominates_and_is_zero_only_for_zero_inputs():
    rng = np.random.default_rng(4)
    R = synth.draw_rotation(rng, 2, 128)
    x = synth.draw_x(rng, 2, 256, "normal")
    assert np.all(Rt.rotate_bound(R, x) >= np.abs(Rt.rotate(R, x)))
    assert not Rt.rotate_bound(R, np.zeros((1, 256))).any()
