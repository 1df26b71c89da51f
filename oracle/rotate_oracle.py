"""CPU oracle for the activation-side rotation (x -> R x, block diagonal).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only ``tests/`` and ``bench.py``'s CPU leg use it.  It shares no code
with the HIP library.

What is computed, and where the pages define it
------------------------------------------------
"Post-Training Ternarization of Qwen3-4B" (arXiv 2609.01962v1 summary) §4.2:
the weights are quantized after an orthogonal change of basis, so at run
time the activations are rotated by the matching transform before they meet
the ternary product (an orthogonal map leaves norms unchanged in exact
arithmetic).  The pages do not give the structure, so the reading
here is the plainest one that fits: a block-diagonal R with B x B blocks
(B = 64 or 128, aligned with the weight groups), given by the caller:
    xr[m, b*B + i] = sum_j R[b][i][j] * x[m, b*B + j].
fp16 inputs are converted exactly to fp64 and the sum is fp64; the GPU
result (FP32 accumulation, FP16 output) must satisfy
    |xr - xr_ref| <= 2e-3 * sum_j |R[b][i][j]| |x[m, b*B + j]|
the same form of bound as the products.
"""
from __future__ import annotations

import numpy as np


def rotate(R: np.ndarray, x: np.ndarray) -> np.ndarray:
    """R [nb][B][B], x [m][nb*B] (any float dtype) -> fp64 [m][nb*B]."""
    R = np.asarray(R, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    nb, B, _ = R.shape
    m = x.shape[0]
    out = np.empty((m, nb * B), dtype=np.float64)
    for b in range(nb):
        seg = slice(b * B, (b + 1) * B)
        out[:, seg] = x[:, seg] @ R[b].T
    return out


def rotate_bound(R: np.ndarray, x: np.ndarray) -> np.ndarray:
    """sum_j |R[b][i][j]| |x[m, b*B + j]| per output element, fp64."""
    return rotate(np.abs(np.asarray(R, dtype=np.float64)), np.abs(np.asarray(x, dtype=np.float64)))
