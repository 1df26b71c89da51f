"""CPU oracle for the quantizer front-end (float weights -> trit planes).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only ``tests/`` and ``bench.py``'s CPU leg use it.  It shares no code
with the HIP library; the two meet only on seeded inputs from
``ternary_weight_only_tern_amd.synth``.

What is computed, and where the pages define it
------------------------------------------------
"Post-Training Ternarization of Qwen3-4B" (arXiv 2609.01962v1 summary) §4.3
describes E2M-ATQ, order-2 asymmetric residual ternarization: each group of
weights is approximated by an offset plus two ternary planes with scales, and
15 refinement iterations follow while the ternary supports stay fixed.  §4.4
(and the 8B page's representation section) gives the second plane only to
salience-selected groups: here a caller-supplied mask per (row, group), the
same bitmap the packed format stores.  §4.5 fixes the group size at 128.

The pages give neither the initial threshold rule nor the content of a
refinement iteration.  The readings taken (listed in the design notes):

* Initial supports: the ternary-weight-network threshold (Li and Liu,
  "Ternary Weight Networks", 2016).  With r = w - mean(w), a trit is non-zero
  where |r| > 0.7 * mean(|r|), with the sign of r; the first scale is the
  mean |r| over that support.  The second plane (masked groups only) applies
  the same rule to the first plane's residual r - alpha * t0.
* One refinement iteration, supports fixed: (a) the least-squares fit of
  (mu, s0, s1) to w over the basis (1, t0, t1); a singular basis drops s1,
  then s0; (b) the squared-error-minimizing sign of every non-zero trit given
  that fit and the other plane, plane 0 first, then plane 1 with the new
  plane 0.  The sign minimizing (e - s t)^2 over t in {-1, +1} is the sign of
  s * e; a tie (s * e == 0) takes +1.  After the iterations a last fit (a)
  gives the stored values.
* Outputs: trits, offset mu and scales s0, s1 rounded to FP16 (round to
  nearest even); s1 = 0 and t1 = 0 on unmasked groups.

Precision.  Everything is fp64.  The basis columns are integers, so the
normal matrix and its determinant are exact and "singular" means det == 0;
the least-squares solution is that of the normal equations, solved with
numpy's batched linear solver.  The GPU kernel computes in FP32, so near a
threshold or a sign tie the two may take different decisions; the GPU tests
check the kernel's output against the rules above with explicit margins
instead of bit for bit.
"""
from __future__ import annotations

import numpy as np

D = np.float64


def masked_groups(mask_bits, n: int, ng: int) -> np.ndarray:
    """bool [n][ng]: bit g % 32 of word g // 32 of row n (None: all False)."""
    if mask_bits is None:
        return np.zeros((n, ng), dtype=bool)
    mb = np.asarray(mask_bits, dtype=np.uint32)
    g = np.arange(ng)
    return ((mb[:, g // 32] >> (g % 32).astype(np.uint32)) & 1).astype(bool)


def _sign(x: np.ndarray) -> np.ndarray:
    """+1 where x >= 0, -1 where x < 0 (int8)."""
    return np.where(x < 0, np.int8(-1), np.int8(1)).astype(np.int8)


def initial_supports(w: np.ndarray, masked: np.ndarray):
    """The threshold rule on groups w [R,G] (fp64): returns t0, t1 (int8)."""
    w = np.asarray(w, dtype=D)
    r = w - w.mean(axis=1, keepdims=True)
    a = np.abs(r)
    on0 = a > 0.7 * a.mean(axis=1, keepdims=True)
    t0 = np.where(on0, _sign(r), np.int8(0)).astype(np.int8)
    n0 = on0.sum(axis=1)
    alpha = np.where(n0 > 0, np.where(on0, a, 0.0).sum(axis=1) / np.maximum(n0, 1), 0.0)
    r2 = r - alpha[:, None] * t0
    a2 = np.abs(r2)
    on1 = (a2 > 0.7 * a2.mean(axis=1, keepdims=True)) & np.asarray(masked, bool)[:, None]
    t1 = np.where(on1, _sign(r2), np.int8(0)).astype(np.int8)
    return t0, t1


def fit(w: np.ndarray, t0: np.ndarray, t1: np.ndarray, masked: np.ndarray):
    """Least-squares (mu, s0, s1) of w [R,G] over the basis (1, t0, t1)
    (t1's column only on masked groups with a non-empty second plane; a
    singular basis drops s1, then s0).  fp64 [R] arrays."""
    w = np.asarray(w, dtype=D)
    R, G = w.shape
    f0, f1 = t0.astype(D), t1.astype(D)
    # normal equations A x = b of the basis (1, t0, t1); A holds exact integers
    p0, p1, c01 = f0.sum(axis=1), f1.sum(axis=1), (f0 * f1).sum(axis=1)
    n0, n1 = (f0 * f0).sum(axis=1), (f1 * f1).sum(axis=1)
    A = np.stack([np.stack([np.full(R, float(G)), p0, p1], axis=1),
                  np.stack([p0, n0, c01], axis=1),
                  np.stack([p1, c01, n1], axis=1)], axis=1)      # [R,3,3]
    b = np.stack([w.sum(axis=1), (w * f0).sum(axis=1), (w * f1).sum(axis=1)], axis=1)
    mu, s0, s1 = w.mean(axis=1), np.zeros(R), np.zeros(R)
    det3 = np.linalg.det(A)
    det2 = A[:, 0, 0] * A[:, 1, 1] - A[:, 0, 1] * A[:, 1, 0]
    use3 = np.asarray(masked, bool) & (A[:, 2, 2] > 0) & (np.rint(det3) != 0)
    use2 = ~use3 & (A[:, 1, 1] > 0) & (det2 != 0)
    if use3.any():
        x = np.linalg.solve(A[use3], b[use3][..., None])[..., 0]
        mu[use3], s0[use3], s1[use3] = x[:, 0], x[:, 1], x[:, 2]
    if use2.any():
        x = np.linalg.solve(A[use2][:, :2, :2], b[use2][:, :2, None])[..., 0]
        mu[use2], s0[use2] = x[:, 0], x[:, 1]
    return mu, s0, s1


def refine_signs(w, t0, t1, mu, s0, s1):
    """The error-minimizing sign of every non-zero trit, plane 0 then plane 1."""
    w = np.asarray(w, dtype=D)
    e0 = w - mu[:, None] - s1[:, None] * t1
    t0 = np.where(t0 != 0, _sign(s0[:, None] * e0), np.int8(0)).astype(np.int8)
    e1 = w - mu[:, None] - s0[:, None] * t0
    t1 = np.where(t1 != 0, _sign(s1[:, None] * e1), np.int8(0)).astype(np.int8)
    return t0, t1


def quantize_groups(w: np.ndarray, masked: np.ndarray, iters: int = 15):
    """Quantize groups w [R,G] (any float dtype) with the second-plane flags
    masked [R].  Returns (t0, t1) int8 [R,G] and (mu, s0, s1) fp64 [R] before
    FP16 rounding."""
    w = np.asarray(w, dtype=D)
    masked = np.asarray(masked, dtype=bool)
    t0, t1 = initial_supports(w, masked)
    for _ in range(iters):
        mu, s0, s1 = fit(w, t0, t1, masked)
        t0, t1 = refine_signs(w, t0, t1, mu, s0, s1)
    mu, s0, s1 = fit(w, t0, t1, masked)
    return t0, t1, mu, s0, s1


def quantize(w: np.ndarray, mask_bits, group: int, iters: int = 15):
    """Quantize a weight matrix w [n][k] (fp16) with group size `group` and
    the residual-plane mask (u32 bitmap [n][ceil(k/group/32)], or None).

    Returns trits int8 [2][n][k], scales fp16 [2][n][k/group] and offsets
    fp16 [n][k/group] (the inputs of packing with per-group offsets).
    """
    w = np.asarray(w)
    n, k = w.shape
    ng = k // group
    masked = masked_groups(mask_bits, n, ng)
    t0, t1, mu, s0, s1 = quantize_groups(w.astype(D).reshape(n * ng, group), masked.reshape(-1), iters)
    trits = np.stack([t0.reshape(n, k), t1.reshape(n, k)])
    scales = np.stack([s0.reshape(n, ng), s1.reshape(n, ng)]).astype(np.float16)
    offset = mu.reshape(n, ng).astype(np.float16)
    return trits, scales, offset


def group_error(w, t0, t1, mu, s0, s1) -> np.ndarray:
    """Squared reconstruction error per group, in fp64."""
    w = np.asarray(w, dtype=D)
    rec = (np.asarray(mu, D)[:, None] + np.asarray(s0, D)[:, None] * t0 + np.asarray(s1, D)[:, None] * t1)
    return ((w - rec) ** 2).sum(axis=1)
