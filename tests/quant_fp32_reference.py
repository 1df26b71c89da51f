"""FP32 transcription of the quantizer kernel's own operation order (test
infrastructure; regression reference only, not the oracle).

The quantizer's parity rests on ``oracle/quant_oracle.py``, a plain fp64
reading of the method, and on validity checks of the GPU output against it
(``tests/test_gpu_quant.py``).  This module instead repeats, in numpy float32,
the fixed summation tree (halve the group, add the halves elementwise: element
i is paired with i + G/2 first), the Cramer's-rule order and the constants of
the kernel, with no fused multiply-adds, so that one test can flag any change
of the kernel's arithmetic bit for bit.  Agreement with it says the kernel is
unchanged, not that it is right.
"""
from __future__ import annotations

import numpy as np

F = np.float32


def tree_sum(v: np.ndarray) -> np.ndarray:
    """Sum over the last axis (a power of two) as the fixed halving tree."""
    v = np.asarray(v, dtype=F)
    while v.shape[-1] > 1:
        h = v.shape[-1] // 2
        v = (v[..., :h] + v[..., h:]).astype(F)
    return v[..., 0]


def _sign(x: np.ndarray) -> np.ndarray:
    """+1 where x >= 0, -1 where x < 0 (as int8)."""
    return np.where(x < F(0), np.int8(-1), np.int8(1)).astype(np.int8)


def _fit(w, t0, t1, masked, sw, n0, n1):
    with np.errstate(divide="ignore", invalid="ignore"):
        return _fit_body(w, t0, t1, masked, sw, n0, n1)


def _fit_body(w, t0, t1, masked, sw, n0, n1):
    """Least-squares (mu, s0, s1) of w over (1, t0, t1) per group (float32).

    w [R,G] float32; t0/t1 [R,G] int8; masked [R] bool; sw, n0, n1 [R]
    float32 (sum of w, support sizes).  Returns three float32 [R] arrays.
    """
    G = w.shape[-1]
    f0 = t0.astype(F)
    f1 = t1.astype(F)
    p0 = tree_sum(f0)
    p1 = tree_sum(f1)
    c01 = tree_sum((f0 * f1).astype(F))
    sw0 = tree_sum((w * f0).astype(F))
    sw1 = tree_sum((w * f1).astype(F))
    g = F(G)
    # 3 x 3: [[g, p0, p1], [p0, n0, c01], [p1, c01, n1]] [mu a b] = [sw sw0 sw1]
    m00 = (n0 * n1 - c01 * c01).astype(F)
    m01 = (p1 * c01 - p0 * n1).astype(F)
    m02 = (p0 * c01 - p1 * n0).astype(F)
    det3 = (g * m00 + p0 * m01 + p1 * m02).astype(F)
    mu3 = ((sw * m00 + sw0 * m01 + sw1 * m02) / det3).astype(F)
    # a = det([[g, sw, p1], [p0, sw0, c01], [p1, sw1, n1]]) / det3
    da = (g * (sw0 * n1 - c01 * sw1) - sw * (p0 * n1 - c01 * p1) + p1 * (p0 * sw1 - sw0 * p1)).astype(F)
    # b = det([[g, p0, sw], [p0, n0, sw0], [p1, c01, sw1]]) / det3
    db = (g * (n0 * sw1 - sw0 * c01) - p0 * (p0 * sw1 - sw0 * p1) + sw * (p0 * c01 - n0 * p1)).astype(F)
    a3 = (da / det3).astype(F)
    b3 = (db / det3).astype(F)
    # 2 x 2: [[g, p0], [p0, n0]] [mu a] = [sw sw0]
    det2 = (g * n0 - p0 * p0).astype(F)
    mu2 = ((sw * n0 - p0 * sw0) / det2).astype(F)
    a2 = ((g * sw0 - p0 * sw) / det2).astype(F)
    # 1 x 1
    mu1 = (sw / g).astype(F)
    use3 = masked & (n1 > 0) & (det3 != 0)
    use2 = ~use3 & (n0 > 0) & (det2 != 0)
    mu = np.where(use3, mu3, np.where(use2, mu2, mu1)).astype(F)
    a = np.where(use3, a3, np.where(use2, a2, F(0))).astype(F)
    b = np.where(use3, b3, F(0)).astype(F)
    return mu, a, b


def quantize_groups(w: np.ndarray, masked: np.ndarray, iters: int = 15):
    """Quantize groups: w [R,G] (fp16 or float32 values), masked [R] bool.

    Returns (t0, t1) int8 [R,G] and (mu, s0, s1) float32 [R] before FP16
    rounding.
    """
    w = np.asarray(w, dtype=F)
    masked = np.asarray(masked, dtype=bool)
    R, G = w.shape
    inv = F(1.0 / G)
    # initial supports (ternary-weight-network threshold)
    sw = tree_sum(w)
    mu0 = (sw * inv).astype(F)
    r = (w - mu0[:, None]).astype(F)
    a = np.abs(r)
    thr = ((tree_sum(a) * inv).astype(F) * F(0.7)).astype(F)
    on0 = a > thr[:, None]
    t0 = np.where(on0, _sign(r), np.int8(0)).astype(np.int8)
    n0 = tree_sum(on0.astype(F))
    s_on = tree_sum(np.where(on0, a, F(0)).astype(F))
    with np.errstate(divide="ignore", invalid="ignore"):
        alpha = np.where(n0 > 0, (s_on / np.maximum(n0, F(1))).astype(F), F(0)).astype(F)
    r2 = (r - (alpha[:, None] * t0.astype(F)).astype(F)).astype(F)
    a2 = np.abs(r2)
    thr2 = ((tree_sum(a2) * inv).astype(F) * F(0.7)).astype(F)
    on1 = (a2 > thr2[:, None]) & masked[:, None]
    t1 = np.where(on1, _sign(r2), np.int8(0)).astype(np.int8)
    n1 = tree_sum(on1.astype(F))
    # refinement with the supports fixed
    for _ in range(iters):
        mu, s0, s1 = _fit(w, t0, t1, masked, sw, n0, n1)
        e0 = (w - mu[:, None] - (s1[:, None] * t1.astype(F)).astype(F)).astype(F)
        t0 = np.where(on0, _sign((s0[:, None] * e0).astype(F)), np.int8(0)).astype(np.int8)
        e1 = (w - mu[:, None] - (s0[:, None] * t0.astype(F)).astype(F)).astype(F)
        t1 = np.where(on1, _sign((s1[:, None] * e1).astype(F)), np.int8(0)).astype(np.int8)
    mu, s0, s1 = _fit(w, t0, t1, masked, sw, n0, n1)
    return t0, t1, mu, s0, s1


def quantize(w: np.ndarray, mask_bits, group: int, iters: int = 15):
    """Quantize a weight matrix w [n][k] (fp16) with group size `group` and
    the residual-plane mask (u32 bitmap [n][ceil(k/group/32)], bit g % 32 of
    word g // 32, or None for no second plane).

    Returns trits int8 [2][n][k], scales fp16 [2][n][k/group] and offsets
    fp16 [n][k/group] (the inputs of packing with per-group offsets).
    """
    w = np.asarray(w)
    n, k = w.shape
    ng = k // group
    if mask_bits is None:
        masked = np.zeros((n, ng), dtype=bool)
    else:
        mb = np.asarray(mask_bits, dtype=np.uint32)
        g = np.arange(ng)
        masked = ((mb[:, g // 32] >> (g % 32).astype(np.uint32)) & 1).astype(bool)
    wg = w.astype(F).reshape(n * ng, group)
    t0, t1, mu, s0, s1 = quantize_groups(wg, masked.reshape(-1), iters)
    trits = np.stack([t0.reshape(n, k), t1.reshape(n, k)])
    scales = np.stack([s0.reshape(n, ng), s1.reshape(n, ng)]).astype(np.float16)
    offset = mu.reshape(n, ng).astype(np.float16)
    return trits, scales, offset


def group_error(w, t0, t1, mu, s0, s1) -> np.ndarray:
    """Squared reconstruction error per group, in fp64 (for the pins)."""
    w = np.asarray(w, dtype=np.float64)
    rec = (np.asarray(mu, np.float64)[:, None] + np.asarray(s0, np.float64)[:, None] * t0
           + np.asarray(s1, np.float64)[:, None] * t1)
    return ((w - rec) ** 2).sum(axis=1)
