"""GPU parity of the quantizer front-end (tern_quantize) against the fp64
oracle in oracle/quant_oracle.py.  The kernel computes in FP32, so its output
is checked for validity against the oracle's rules (tests/quant_checks.py):
supports by the threshold rule outside a margin, scales and offset equal to
the least-squares fit of its own trits to FP16 rounding, error-minimizing
signs outside ties, and a group error within 1e-3 of the oracle's.  A
separate regression test compares it bit for bit with the FP32 transcription
of its own operation order (tests/quant_fp32_reference.py), which flags any
change of the kernel's arithmetic.  Finally the output is packed and
multiplied and the product checked against the oracle's product of the same
planes."""
import numpy as np
import pytest

import oracle as O
import quant_checks as C
import quant_fp32_reference as R
from ternary_weight_only_tern_amd import lib as L
from ternary_weight_only_tern_amd import synth
from gpu_util import check_y, say, to_dev

pytestmark = pytest.mark.gpu


def _weights(rng, n, k, group, law):
    w = synth.draw_x(rng, n, k, law)  # fp16 [n][k]
    if n >= 3:
        w[0, :group] = np.float16(0.375)        # a constant group
        w[1, group:2 * group] = np.float16(0.0)  # an all-zero group (k >= 2 groups)
        t = rng.integers(-1, 2, size=group)
        w[2, :group] = (np.float16(0.25) + np.float16(1.5) * t).astype(np.float16)  # representable
    return w


def _run(w, mask_bits, group, iters=15):
    import torch
    wd = to_dev(w.view(np.uint16))
    md = to_dev(mask_bits.view(np.int32)) if mask_bits is not None else None
    trits, scales, offset = L.tern_quantize(wd, md, group, iters)
    torch.cuda.synchronize()
    return trits.cpu().numpy(), scales.cpu().numpy(), offset.cpu().numpy()


CASES = [  # n, k, group, mask fraction (None: no mask), weight law, iterations
    (37, 512, 128, 0.3, "normal", 15),
    (64, 1024, 128, None, "normal", 15),
    (5, 256, 64, 1.0, "student_t3", 15),
    (130, 640, 64, 0.1, "normal", 15),
    (9, 384, 128, 0.5, "student_t3", 0),
    (9, 384, 128, 0.5, "normal", 3),
]


@pytest.mark.parametrize("n,k,group,frac,law,iters", CASES)
def test_quantize_is_valid_against_fp64_oracle(n, k, group, frac, law, iters):
    say("quantize (validity)", n, k, group, frac, law, iters)
    rng = np.random.default_rng(n * 31 + k + group)
    w = _weights(rng, n, k, group, law)
    mb = synth.draw_mask(rng, n, k // group, frac)[1] if frac is not None else None
    trits, scales, offset = _run(w, mb, group, iters)
    info = C.check_quantization(w, mb, group, trits, scales, offset, iters)
    say("  accepted near-threshold / near-tie cases", info)


@pytest.mark.parametrize("n,k,group,frac,law,iters", CASES)
def test_quantize_regression_fp32_transcription(n, k, group, frac, law, iters):
    """Bit-exact with the FP32 transcription of the kernel's operation order
    (a regression check of the kernel's arithmetic, not the parity claim)."""
    say("quantize (regression)", n, k, group, frac, law, iters)
    rng = np.random.default_rng(n * 31 + k + group)
    w = _weights(rng, n, k, group, law)
    mb = synth.draw_mask(rng, n, k // group, frac)[1] if frac is not None else None
    trits, scales, offset = _run(w, mb, group, iters)
    rt, rs, ro = R.quantize(w, mb, group, iters)
    assert np.array_equal(trits, rt), f"trits differ at {np.argwhere(trits != rt)[:5].tolist()}"
    assert np.array_equal(scales.view(np.uint16), rs.view(np.uint16)), "scales differ"
    assert np.array_equal(offset.view(np.uint16), ro.view(np.uint16)), "offsets differ"


def test_quantize_empty_and_degenerate_shapes():
    import torch
    say("quantize empty")
    w = torch.zeros((0, 256), dtype=torch.float16, device="cuda")
    trits, scales, offset = L.tern_quantize(w, None, 128)
    assert trits.shape == (2, 0, 256) and scales.shape == (2, 0, 2) and offset.shape == (0, 2)
    # one row, one group, every weight equal: no trits, offset = the weight
    w1 = np.full((1, 128), np.float16(-2.5))
    t, s, o = _run(w1, None, 128)
    assert not t.any() and not s.any() and o[0, 0] == np.float16(-2.5)


@pytest.mark.parametrize("fmt", [O.FMT_2BIT, O.FMT_B3])
def test_quantized_layer_packs_and_multiplies(fmt):
    """Quantize a 4B-class projection's shape (q, 2560 -> 4096) with a 10 %
    salience mask; the output is valid against the fp64 oracle (checked on its
    first 512 rows, to bound the CPU time), packs (two planes, per-group
    offsets) and multiplies within the bound of the oracle's product of the
    same planes, scales and offsets."""
    import torch
    say("quantize -> pack -> gemv", fmt)
    rng = np.random.default_rng(11 + fmt)
    n, k, group = 4096, 2560, 128
    w = synth.draw_x(rng, n, k, "normal")
    sel, mb = synth.draw_mask(rng, n, k // group, 0.10)
    wd = to_dev(w.view(np.uint16))
    trits, scales, offset = L.tern_quantize(wd, to_dev(mb.view(np.int32)), group)
    nnz = [int(sel.sum())]
    pm = L.PackedMatrix(n, k, group, 2, fmt, O.OFF_GROUP, nnz)
    L.tern_pack(pm, trits, scales, to_dev(mb[None].view(np.int32)), offset)
    x = synth.draw_x(rng, 1, k, "normal")
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    y = L.tern_gemv(pm, xd, L.TERN_F32)
    torch.cuda.synchronize()
    gt, gs, go = trits.cpu().numpy(), scales.cpu().numpy(), offset.cpu().numpy()
    C.check_quantization(w[:512], mb[:512], group, gt[:, :512], gs[:, :512], go[:512])
    y_ref = O.gemv(gt, [gs[0], gs[1]], [sel], go, O.OFF_GROUP, x, group)
    b = O.bound(gt, [gs[0], gs[1]], [sel], go, O.OFF_GROUP, x, group)
    check_y(y, y_ref, b, "quantized layer")
