"""Pins of the quantizer oracle (oracle/quant_oracle.py, fp64) against what
the method and the mathematics fix: a hand-worked group, the threshold rule by
hand, exact recovery of representable weights, the least-squares step against
numpy's solver, the normal equations, the sign rule by brute force, monotone
error over the refinement, scale and sign equivariance and the degenerate
groups.  Then the validity checks that the GPU tests apply to the kernel's
output (tests/quant_checks.py): they accept the oracle's own output and the
kernel's FP32 transcription, and reject planted mistakes."""
import numpy as np
import pytest

import oracle.quant_oracle as Q
import quant_checks as C
import quant_fp32_reference as R
from ternary_weight_only_tern_amd import synth


def test_fp32_reference_tree_sum_pairs_halves_first():
    # the kernel's FP32 transcription sums a group as a halving tree:
    # G = 4: (v0 + v2) + (v1 + v3), in float32
    Q = R
    v = np.array([1e8, 1.0, -1e8, 1.0], dtype=np.float32)
    assert Q.tree_sum(v) == np.float32(2.0)  # (1e8 - 1e8) + (1 + 1)
    # a left-to-right sum would lose the ones: ((1e8 + 1) - 1e8) + 1 = 1
    w = np.array([1e8, -1e8, 1.0, 1.0], dtype=np.float32)
    # (1e8 + 1) + (-1e8 + 1) in float32: both halves round to -+1e8, so 0
    assert Q.tree_sum(w) == np.float32(0.0)
    x = np.random.default_rng(0).standard_normal((5, 64)).astype(np.float32)
    ref = x.copy()
    while ref.shape[1] > 1:
        h = ref.shape[1] // 2
        ref = ref[:, :h] + ref[:, h:]
    assert np.array_equal(Q.tree_sum(x), ref[:, 0])


def test_hand_worked_group():
    # w = [3, -3, 0.5, -0.5]: mean 0, mean|r| = 1.75, threshold 1.225 ->
    # support {0, 1}, signs (+, -), first scale 3; the fit keeps mu = 0, s0 = 3
    w = np.array([[3.0, -3.0, 0.5, -0.5]], dtype=np.float32)
    t0, t1, mu, s0, s1 = Q.quantize_groups(w, np.array([False]))
    assert t0.tolist() == [[1, -1, 0, 0]] and not t1.any()
    assert mu[0] == 0.0 and s0[0] == 3.0 and s1[0] == 0.0


def _representable(rng, R, G, mu, s0, s1):
    """Groups w = mu + s0 t0 + s1 t1 with balanced signs (mean(t0) = mean(t1) = 0)."""
    t0 = np.zeros((R, G), np.int8)
    t1 = np.zeros((R, G), np.int8)
    for r in range(R):
        idx = rng.permutation(G)
        n0 = G // 2          # plane-0 support, half + and half -
        t0[r, idx[: n0 // 2]] = 1
        t0[r, idx[n0 // 2: n0]] = -1
        n1 = G // 4          # plane-1 support overlapping plane 0 only
        sub = idx[: n0]
        pick = rng.permutation(sub)[:n1]
        t1[r, pick[: n1 // 2]] = 1
        t1[r, pick[n1 // 2:]] = -1
    w = mu + s0 * t0.astype(np.float64) + s1 * t1.astype(np.float64)
    return w.astype(np.float32), t0, t1


@pytest.mark.parametrize("G", [64, 128])
def test_exact_recovery_of_representable_groups(G):
    rng = np.random.default_rng(G)
    w, t0, t1 = _representable(rng, 6, G, 0.125, 1.0, 0.25)
    q0, q1, mu, s0, s1 = Q.quantize_groups(w, np.ones(6, bool))
    assert np.array_equal(q0, t0) and np.array_equal(q1, t1)
    assert np.allclose(mu, 0.125, rtol=0, atol=1e-12)
    assert np.allclose(s0, 1.0, rtol=1e-12) and np.allclose(s1, 0.25, rtol=1e-12)
    # without the mask the second plane is not used
    q0u, q1u, _, _, s1u = Q.quantize_groups(w, np.zeros(6, bool))
    assert not q1u.any() and not s1u.any()


def test_fit_matches_numpy_least_squares():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((40, 128)) * 0.02).astype(np.float32)
    masked = rng.random(40) < 0.5
    t0, t1, mu, s0, s1 = Q.quantize_groups(w, masked)
    for r in range(40):
        cols = [np.ones(128), t0[r].astype(np.float64)]
        if masked[r] and t1[r].any():
            cols.append(t1[r].astype(np.float64))
        A = np.stack(cols, axis=1)
        sol = np.linalg.lstsq(A, w[r].astype(np.float64), rcond=None)[0]
        got = [mu[r], s0[r]] + ([s1[r]] if len(cols) == 3 else [])
        assert np.allclose(got, sol, rtol=1e-10, atol=1e-13), (r, got, sol)
        if len(cols) == 2:
            assert s1[r] == 0.0


def test_normal_equations_hold():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((64, 128)).astype(np.float32)
    masked = np.arange(64) % 3 == 0
    t0, t1, mu, s0, s1 = Q.quantize_groups(w, masked)
    res = w.astype(np.float64) - (mu[:, None] + s0[:, None] * t0 + s1[:, None] * t1)
    scale = np.abs(w).sum(axis=1)
    assert np.all(np.abs(res.sum(axis=1)) <= 1e-12 * scale)
    assert np.all(np.abs((res * t0).sum(axis=1)) <= 1e-12 * scale)
    assert np.all(np.abs((res * t1).sum(axis=1)) <= 1e-12 * scale)


def test_refinement_never_increases_the_error():
    rng = np.random.default_rng(5)
    w = synth.draw_x(rng, 32, 128, "student_t3").astype(np.float32)  # heavy-tailed groups
    masked = np.arange(32) % 2 == 0
    errs = []
    for it in range(0, 16):
        t0, t1, mu, s0, s1 = Q.quantize_groups(w, masked, iters=it)
        errs.append(Q.group_error(w, t0, t1, mu, s0, s1))
    errs = np.stack(errs)
    assert np.all(errs[1:] <= errs[:-1] * (1 + 1e-12) + 1e-15)
    assert np.all(errs[-1] <= errs[0])
    # supports never change
    t0a, t1a, *_ = Q.quantize_groups(w, masked, iters=0)
    t0b, t1b, *_ = Q.quantize_groups(w, masked, iters=15)
    assert np.array_equal(t0a != 0, t0b != 0) and np.array_equal(t1a != 0, t1b != 0)


def test_scale_and_sign_equivariance():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((16, 128)).astype(np.float32)
    masked = np.arange(16) % 2 == 1
    a = Q.quantize_groups(w, masked)
    b = Q.quantize_groups(2.0 * w.astype(np.float64), masked)
    c = Q.quantize_groups(-w, masked)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for x, y in zip(a[2:], b[2:]):
        assert np.array_equal(2.0 * x, y)
    assert np.array_equal(a[0], -c[0]) and np.array_equal(a[1], -c[1])
    assert np.array_equal(a[2], -c[2]) and np.array_equal(a[3], c[3]) and np.array_equal(a[4], c[4])


def test_degenerate_groups():
    w = np.stack([np.full(128, 0.375, np.float32), np.zeros(128, np.float32)])
    t0, t1, mu, s0, s1 = Q.quantize_groups(w, np.array([True, True]))
    assert not t0.any() and not t1.any()
    assert mu.tolist() == [0.375, 0.0] and not s0.any() and not s1.any()


def test_matrix_entry_point_layout():
    rng = np.random.default_rng(7)
    n, k, G = 5, 384, 128
    w = rng.standard_normal((n, k)).astype(np.float16)
    _, mb = synth.draw_mask(rng, n, k // G, 0.4)
    trits, scales, offset = Q.quantize(w, mb, G)
    assert trits.shape == (2, n, k) and scales.shape == (2, n, k // G) and offset.shape == (n, k // G)
    assert scales.dtype == np.float16 and offset.dtype == np.float16
    for r in range(n):
        for g in range(k // G):
            on = bool((mb[r, g // 32] >> (g % 32)) & 1)
            seg = slice(g * G, (g + 1) * G)
            t0, t1, mu, s0, s1 = Q.quantize_groups(w[r:r + 1, seg].astype(np.float64), np.array([on]))
            assert np.array_equal(trits[0, r, seg], t0[0]) and np.array_equal(trits[1, r, seg], t1[0])
            assert scales[0, r, g] == np.float16(s0[0]) and scales[1, r, g] == np.float16(s1[0])
            assert offset[r, g] == np.float16(mu[0])
            if not on:
                assert not trits[1, r, seg].any() and scales[1, r, g] == 0


def test_threshold_rule_by_hand():
    # w = [4, 0, 0, 0, 0, 0, 0, -4]: mean 0, mean|r| = 1, threshold 0.7 ->
    # plane 0 on {0, 7} with signs (+, -), alpha = 4; the residual is 0
    # everywhere, so plane 1 (masked) is empty (0 > 0 is false)
    w = np.array([[4.0, 0, 0, 0, 0, 0, 0, -4.0]])
    t0, t1 = Q.initial_supports(w, np.array([True]))
    assert t0.tolist() == [[1, 0, 0, 0, 0, 0, 0, -1]] and not t1.any()
    # w = [3, 1, 0, 0]: mean 1, r = [2, 0, -1, -1], mean|r| = 1, threshold 0.7
    # -> plane 0 on {0, 2, 3} (+, -, -), alpha = 4/3; residual
    # [2/3, 0, 1/3, 1/3], mean 1/3, threshold 7/30 -> plane 1 on {0, 2, 3}
    w = np.array([[3.0, 1.0, 0.0, 0.0]])
    t0, t1 = Q.initial_supports(w, np.array([True]))
    assert t0.tolist() == [[1, 0, -1, -1]] and t1.tolist() == [[1, 0, 1, 1]]
    t0u, t1u = Q.initial_supports(w, np.array([False]))
    assert t0u.tolist() == [[1, 0, -1, -1]] and not t1u.any()


def test_sign_rule_by_brute_force():
    # for a given fit, each refined sign is the one of {-1, +1} with the
    # smaller squared error, element by element (plane 0 first)
    rng = np.random.default_rng(12)
    w = rng.standard_normal((50, 16))
    t0 = rng.integers(-1, 2, size=(50, 16)).astype(np.int8)
    t1 = (rng.integers(-1, 2, size=(50, 16)) * (rng.random((50, 16)) < 0.3)).astype(np.int8)
    mu, s0, s1 = rng.standard_normal(50), rng.standard_normal(50), rng.standard_normal(50)
    n0, n1 = Q.refine_signs(w, t0, t1, mu, s0, s1)
    for r in range(50):
        for j in range(16):
            if t0[r, j]:
                e = lambda t: (w[r, j] - mu[r] - s0[r] * t - s1[r] * t1[r, j]) ** 2
                assert e(n0[r, j]) <= e(-n0[r, j])
            else:
                assert n0[r, j] == 0
            if t1[r, j]:
                e = lambda t: (w[r, j] - mu[r] - s0[r] * n0[r, j] - s1[r] * t) ** 2
                assert e(n1[r, j]) <= e(-n1[r, j])
            else:
                assert n1[r, j] == 0


CHECK_CASES = [(37, 512, 128, 0.3, "normal"), (64, 1024, 128, None, "normal"), (5, 256, 64, 1.0, "student_t3"),
               (130, 640, 64, 0.1, "normal")]


@pytest.mark.parametrize("n,k,group,frac,law", CHECK_CASES)
def test_checks_accept_oracle_and_fp32_transcription(n, k, group, frac, law):
    rng = np.random.default_rng(n * 31 + k + group)
    w = synth.draw_x(rng, n, k, law)
    mb = synth.draw_mask(rng, n, k // group, frac)[1] if frac is not None else None
    C.check_quantization(w, mb, group, *Q.quantize(w, mb, group))
    C.check_quantization(w, mb, group, *R.quantize(w, mb, group))


def test_checks_reject_planted_mistakes():
    rng = np.random.default_rng(21)
    n, k, group = 24, 512, 128
    w = synth.draw_x(rng, n, k, "normal")
    mb = synth.draw_mask(rng, n, k // group, 0.5)[1]
    trits, scales, offset = Q.quantize(w, mb, group)
    masked = Q.masked_groups(mb, n, k // group)
    g = int(np.argwhere(masked[3])[0, 0])  # a masked group of row 3
    seg = slice(g * group, (g + 1) * group)

    def bad(tr, sc, of):
        with pytest.raises(AssertionError):
            C.check_quantization(w, mb, group, tr, sc, of)

    t = trits.copy()
    j = int(np.argwhere(t[0, 3, seg] != 0)[0, 0])
    t[0, 3, g * group + j] *= -1                     # a flipped plane-0 sign
    bad(t, scales, offset)
    t = trits.copy()
    j = int(np.argwhere(t[0, 3, seg] != 0)[0, 0])
    t[0, 3, g * group + j] = 0                       # a dropped support element
    bad(t, scales, offset)
    t = trits.copy()
    j = int(np.argwhere(t[1, 3, seg] != 0)[0, 0])
    t[1, 3, g * group + j] *= -1                     # a flipped plane-1 sign
    bad(t, scales, offset)
    s = scales.copy()
    s[0, 3, g] = np.float16(float(s[0, 3, g]) * 1.01)  # a scale 1 % off
    bad(trits, s, offset)
    o = offset.copy()
    o[3, g] = np.float16(float(o[3, g]) + 0.01 * abs(float(scales[0, 3, g])))  # an offset off by 1 % of a scale
    bad(trits, scales, o)
    t = trits.copy()
    um = int(np.argwhere(~masked[5])[0, 0])
    t[1, 5, um * group] = 1                          # plane 1 outside the mask
    bad(t, scales, offset)
