"""Validity checks of a quantization against the fp64 reading of the
quantizer (oracle/quant_oracle.py), for outputs computed in another precision
(the GPU kernel computes in FP32).  Where several outputs are correct (a
threshold or a sign decided within rounding), the checks accept either and
count the cases.

check_quantization(w, mask_bits, group, trits, scales, offset) verifies:
  (i)   supports: plane 0 is the threshold rule |r| > 0.7 mean|r| of fp64,
        except at elements within a relative margin of the threshold; plane 1
        likewise on the residual of the output's own plane-0 support, and only
        on masked groups;
  (ii)  fit: the offset and scales equal the fp64 least-squares fit over the
        output's own trits, to half an FP16 unit in the last place plus an
        FP32 solve margin;
  (iii) signs: every non-zero trit has the error-minimizing sign given that
        fit, except at near-ties (with no refinement iteration: the sign the
        threshold rule gives);
  (iv)  error: the per-group squared error of the output is at most
        (1 + 1e-3) times that of the fp64 oracle's own quantization (both with
        FP16-rounded values), plus a tiny absolute term.
It returns the counts of the accepted near-threshold and near-tie cases.
"""
from __future__ import annotations

import numpy as np

import oracle.quant_oracle as Q

D = np.float64
THR_MARGIN = 1e-4      # relative distance to a threshold within which either side is correct
TIE_MARGIN = 1e-4      # relative size of s * e below which either sign is correct
FIT_MARGIN = 2e-4      # FP32 solve error, relative to the group's largest fitted magnitude


def _half_ulp16(v: np.ndarray) -> np.ndarray:
    """Half a unit in the last place of FP16 at |v| (subnormal floor 2^-25)."""
    a = np.abs(np.asarray(v, D))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.maximum(2.0 ** (e - 11), 2.0 ** -25)


def check_quantization(w, mask_bits, group, trits, scales, offset, iters=15):
    w = np.asarray(w)
    n, k = w.shape
    ng = k // group
    G = group
    W = w.astype(D).reshape(n * ng, G)
    masked = Q.masked_groups(mask_bits, n, ng).reshape(-1)
    t0 = np.asarray(trits[0]).reshape(n * ng, G).astype(np.int8)
    t1 = np.asarray(trits[1]).reshape(n * ng, G).astype(np.int8)
    mu = np.asarray(offset, np.float16).reshape(-1).astype(D)
    s0 = np.asarray(scales[0], np.float16).reshape(-1).astype(D)
    s1 = np.asarray(scales[1], np.float16).reshape(-1).astype(D)
    assert set(np.unique(t0)).issubset({-1, 0, 1}) and set(np.unique(t1)).issubset({-1, 0, 1})

    # (i) supports
    r = W - W.mean(axis=1, keepdims=True)
    a = np.abs(r)
    thr = 0.7 * a.mean(axis=1, keepdims=True)
    sup0 = t0 != 0
    near0 = np.abs(a - thr) <= THR_MARGIN * thr + 1e-30
    bad0 = (sup0 != (a > thr)) & ~near0
    assert not bad0.any(), f"plane-0 support off the threshold rule at {np.argwhere(bad0)[:5].tolist()}"
    t0i = np.where(sup0, np.where(r < 0, -1, 1), 0)
    cnt = sup0.sum(axis=1)
    alpha = np.where(cnt > 0, np.where(sup0, a, 0.0).sum(axis=1) / np.maximum(cnt, 1), 0.0)
    a2 = np.abs(r - alpha[:, None] * t0i)
    thr2 = 0.7 * a2.mean(axis=1, keepdims=True)
    sup1 = t1 != 0
    near1 = np.abs(a2 - thr2) <= THR_MARGIN * thr2 + 1e-30
    bad1 = (sup1 != ((a2 > thr2) & masked[:, None])) & ~(near1 & masked[:, None])
    assert not bad1.any(), f"plane-1 support off the threshold rule at {np.argwhere(bad1)[:5].tolist()}"
    assert not (sup1 & ~masked[:, None]).any() and not (s1[~masked] != 0).any(), "plane 1 outside the mask"

    # (ii) fit over the output's own trits
    fm, f0, f1 = Q.fit(W, t0, t1, masked)
    mag = np.maximum.reduce([np.abs(fm), np.abs(f0), np.abs(f1)])
    for name, got, ref in (("offset", mu, fm), ("s0", s0, f0), ("s1", s1, f1)):
        tol = _half_ulp16(ref) + FIT_MARGIN * mag + 1e-30
        bad = np.abs(got - ref) > tol
        assert not bad.any(), f"{name} off the least-squares fit at groups {np.argwhere(bad)[:5].ravel().tolist()}"

    # (iii) signs: with no refinement (iters == 0) they are the threshold
    # rule's (the sign of r, then of the residual); otherwise error-minimizing
    # given that fit (plane 0, then plane 1 with plane 0 as output)
    if iters == 0:
        i0, i1 = Q.initial_supports(W, masked)
        assert np.array_equal(np.where(sup0, t0, 0), np.where(sup0, i0, 0)), "plane-0 signs off the threshold rule"
        on1 = sup1 & (i1 != 0)
        assert np.array_equal(np.where(on1, t1, 0), np.where(on1, i1, 0)), "plane-1 signs off the threshold rule"
    e0 = W - fm[:, None] - f1[:, None] * t1
    g0 = f0[:, None] * e0
    tie0 = np.abs(g0) <= TIE_MARGIN * (f0[:, None] ** 2 + np.abs(g0).max(axis=1, keepdims=True) * 1e-3) + 1e-30
    bad_s0 = sup0 & (t0 != np.where(g0 < 0, -1, 1)) & ~tie0 & (iters > 0)
    assert not bad_s0.any(), f"plane-0 sign not error-minimizing at {np.argwhere(bad_s0)[:5].tolist()}"
    e1 = W - fm[:, None] - f0[:, None] * t0
    g1 = f1[:, None] * e1
    tie1 = np.abs(g1) <= TIE_MARGIN * (f1[:, None] ** 2 + np.abs(g1).max(axis=1, keepdims=True) * 1e-3) + 1e-30
    bad_s1 = sup1 & (t1 != np.where(g1 < 0, -1, 1)) & ~tie1 & (iters > 0)
    assert not bad_s1.any(), f"plane-1 sign not error-minimizing at {np.argwhere(bad_s1)[:5].tolist()}"

    # (iv) error against the fp64 oracle's own quantization (both FP16-rounded)
    o0, o1, om, os0, os1 = Q.quantize_groups(W, masked, iters)
    r16 = lambda v: np.asarray(v, D).astype(np.float16).astype(D)
    err = Q.group_error(W, t0, t1, mu, s0, s1)
    ref = Q.group_error(W, o0, o1, r16(om), r16(os0), r16(os1))
    scale = (W ** 2).sum(axis=1)
    bad_e = err > ref * (1 + 1e-3) + 1e-9 * scale + 1e-30
    assert not bad_e.any(), (f"group error above the fp64 oracle's at {np.argwhere(bad_e)[:5].ravel().tolist()}: "
                             f"{err[bad_e][:3]} vs {ref[bad_e][:3]}")
    return dict(near_threshold=int((near0 & (sup0 != (a > thr))).sum()
                                   + (near1 & (sup1 != ((a2 > thr2) & masked[:, None]))).sum()),
                near_ties=int((sup0 & tie0 & (t0 != np.where(g0 < 0, -1, 1))).sum()
                              + (sup1 & tie1 & (t1 != np.where(g1 < 0, -1, 1))).sum()),
                same_trits_as_oracle=float(np.mean((t0 == o0).all(axis=1) & (t1 == o1).all(axis=1))))
