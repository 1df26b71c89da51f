"""Seeded synthetic inputs for packed ternary linear layers.

This module only *draws* inputs: trit planes, FP16 scales, salience masks,
offsets and FP16 activations, with the shapes and value laws of the layers
the pages study (Qwen3-4B- and Qwen3-8B-class decoder projections: 36 layers,
q/k/v/o and gate/up/down; arXiv 2609.09240, model section; 2609.01962 §3.1).
It holds none of the method's arithmetic (no packing, no products) and is
the only code shared between the CPU oracle and the GPU path.

Laws (the pages fix only the group size 128 and FP16 scales/activations):
  trits   iid, P(-1) = P(+1) = 0.33, P(0) = 0.34 (100-bin uniform integer draw)
  scales  fp16 ~ U(0.01, 0.1), or log-normal exp(N(0, 1)) for the stress layer
  masks   exactly round(f * N * K/G) groups per matrix, uniform without
          replacement; residual trits are drawn inside the mask only
  x       fp16 ~ N(0, 1), or Student-t(3) clipped to +-65504 for the stress layer
  offset  fp16 ~ N(0, 1) per output row (stress layer only)
Values are drawn in fp64 and rounded to fp16 (round-to-nearest-even).
Every matrix has its own stream: PCG64(SeedSequence([seed, stream, layer,
proj])), where `stream` is the workload's fixed stream id; its activations use
SeedSequence([seed, stream, layer, proj, 1]).
"""
from __future__ import annotations

import numpy as np

FMT_2BIT = 0
FMT_B3 = 1
OFF_NONE = 0
OFF_ROW = 1
OFF_GROUP = 2

# (name, K, N) for the seven projections of a decoder layer.
QWEN3_4B_LAYER = [("q", 2560, 4096), ("k", 2560, 1024), ("v", 2560, 1024),
                  ("o", 4096, 2560), ("gate", 2560, 9728), ("up", 2560, 9728),
                  ("down", 9728, 2560)]
QWEN3_8B_LAYER = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024),
                  ("o", 4096, 4096), ("gate", 4096, 12288), ("up", 4096, 12288),
                  ("down", 12288, 4096)]
NUM_LAYERS = 36
# For each projection of a decoder layer, the projection whose input it
# reads: q/k/v take the same normed hidden state, gate/up the same normed
# post-attention state (one activation vector each per layer and token).
LAYER_INPUT = (0, 0, 0, 3, 4, 4, 6)

WORKLOADS = {
    "single_gemv": dict(stream=1, name="single-gemv K256 N128 G64 2-bit", shapes=[("w", 256, 128)], group=64,
            planes=1, res_frac=0.0, fmt=FMT_2BIT, m=[1], scale_law="uniform",
            x_law="normal", offset_mode=OFF_NONE),
    "qwen3_4b_layer": dict(stream=2, name="qwen3-4b-class layer M=1", shapes=QWEN3_4B_LAYER, group=128,
            planes=2, res_frac=0.10, fmt=FMT_2BIT, m=[1], scale_law="uniform",
            x_law="normal", offset_mode=OFF_NONE),
    "qwen3_8b_stack": dict(stream=3, name="qwen3-8b-class 36x7 stack M=1 base-3", shapes=QWEN3_8B_LAYER, group=128,
            planes=2, res_frac=0.08, fmt=FMT_B3, m=[1], scale_law="uniform",
            x_law="normal", offset_mode=OFF_NONE, layers=NUM_LAYERS),
    "qwen3_8b_layer": dict(stream=4, name="qwen3-8b-class layer batched base-3", shapes=QWEN3_8B_LAYER, group=128,
            planes=2, res_frac=0.08, fmt=FMT_B3, m=[1, 4, 16, 64, 512], scale_law="uniform",
            x_law="normal", offset_mode=OFF_NONE),
    "down_proj_stress": dict(stream=5, name="down-proj stress K12288 N4096", shapes=[("down", 12288, 4096)], group=128,
            planes=3, res_frac=0.20, fmt=FMT_2BIT, m=[1, 8], scale_law="lognormal",
            x_law="student_t3", offset_mode=OFF_ROW, shared_mask=True),
}


def rng_for(seed: int, stream: int, layer: int, proj: int, extra=None) -> np.random.Generator:
    key = [seed, stream, layer, proj] + ([] if extra is None else [extra])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def draw_trits(rng: np.random.Generator, shape) -> np.ndarray:
    u = rng.integers(0, 100, size=shape, dtype=np.uint8)
    return (u >= 67).astype(np.int8) - (u < 33).astype(np.int8)


def draw_scales(rng: np.random.Generator, shape, law: str) -> np.ndarray:
    if law == "uniform":
        return rng.uniform(0.01, 0.1, size=shape).astype(np.float16)
    if law == "lognormal":
        return np.exp(rng.standard_normal(size=shape)).astype(np.float16)
    raise ValueError(law)


def draw_x(rng: np.random.Generator, m: int, k: int, law: str) -> np.ndarray:
    if law == "normal":
        return rng.standard_normal(size=(m, k)).astype(np.float16)
    if law == "student_t3":
        return np.clip(rng.standard_t(3, size=(m, k)), -65504.0, 65504.0).astype(np.float16)
    raise ValueError(law)


def draw_mask(rng: np.random.Generator, n: int, ngroups: int, frac: float):
    """Exactly round(frac*n*ngroups) groups; returns (bool [N][ng], bitmap u32 [N][W])."""
    count = int(round(frac * n * ngroups))
    flat = np.zeros(n * ngroups, dtype=bool)
    if count:
        flat[rng.choice(n * ngroups, size=count, replace=False)] = True
    sel = flat.reshape(n, ngroups)
    words = (ngroups + 31) // 32
    bits = np.zeros((n, words), dtype=np.uint32)
    for g in range(ngroups):
        bits[:, g // 32] |= sel[:, g].astype(np.uint32) << np.uint32(g % 32)
    return sel, bits


def make_matrix(n: int, k: int, group: int, planes: int, res_frac: float, *,
                rng: np.random.Generator, scale_law: str = "uniform",
                offset_mode: int = OFF_NONE, shared_mask: bool = False) -> dict:
    """One synthetic quantized matrix in unpacked form.

    Returns dict(trits int8 [P][N][K], scales fp16 [P][N][K/G],
    masks bool [P-1][N][K/G], mask_bits u32 [P-1][N][W], offset, offset_mode,
    n, k, group, planes).  Draw order: plane-0 trits, plane-0 scales, then per
    residual plane: mask (unless shared with the previous one), trits inside
    the mask, scales; then the offset.
    """
    ng = k // group
    trits = np.zeros((planes, n, k), dtype=np.int8)
    scales = np.zeros((planes, n, ng), dtype=np.float16)
    trits[0] = draw_trits(rng, (n, k))
    scales[0] = draw_scales(rng, (n, ng), scale_law)
    masks, mask_bits = [], []
    for p in range(1, planes):
        if shared_mask and masks:
            sel, bits = masks[-1], mask_bits[-1]
        else:
            sel, bits = draw_mask(rng, n, ng, res_frac)
        masks.append(sel)
        mask_bits.append(bits)
        rows, groups = np.nonzero(sel)
        tp = trits[p].reshape(n, ng, group)
        tp[rows, groups] = draw_trits(rng, (rows.size, group))
        scales[p] = draw_scales(rng, (n, ng), scale_law)
    if offset_mode == OFF_ROW:
        offset = rng.standard_normal(size=n).astype(np.float16)
    elif offset_mode == OFF_GROUP:
        offset = rng.standard_normal(size=(n, ng)).astype(np.float16)
    else:
        offset = None
    return dict(trits=trits, scales=scales, masks=masks, mask_bits=mask_bits,
                offset=offset, offset_mode=offset_mode, n=n, k=k, group=group,
                planes=planes)


def workload_matrix(wl: str, proj: int = 0, layer: int = 0, seed: int = 0) -> dict:
    """Matrix `proj` of layer `layer` of the named workload."""
    c = WORKLOADS[wl]
    _, k, n = c["shapes"][proj]
    mat = make_matrix(n, k, c["group"], c["planes"], c["res_frac"],
                      rng=rng_for(seed, c["stream"], layer, proj), scale_law=c["scale_law"],
                      offset_mode=c["offset_mode"], shared_mask=c.get("shared_mask", False))
    mat["fmt"] = c["fmt"]
    mat["name"] = c["shapes"][proj][0]
    return mat


def workload_x(wl: str, m: int, proj: int = 0, layer: int = 0, seed: int = 0) -> np.ndarray:
    """Activations [m][k] for matrix `proj` of layer `layer` of the named workload."""
    c = WORKLOADS[wl]
    _, k, _ = c["shapes"][proj]
    return draw_x(rng_for(seed, c["stream"], layer, proj, 1), m, k, c["x_law"])


def draw_rotation(rng: np.random.Generator, nb: int, block: int) -> np.ndarray:
    """nb random orthogonal block x block matrices (QR of a Gaussian draw, the
    usual Haar construction), rounded to fp16: [nb][block][block]."""
    out = np.empty((nb, block, block), dtype=np.float16)
    for b in range(nb):
        q, r = np.linalg.qr(rng.standard_normal((block, block)))
        q = q * np.sign(np.diag(r))[None, :]
        out[b] = q.astype(np.float16)
    return out
