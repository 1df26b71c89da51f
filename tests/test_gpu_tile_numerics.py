"""The tile paths' error budget at its edge: the 16-row product (M=8,
gemm_small_kernel) and the large tiles (M=64, tern_gemm and a plan) on
products whose decoded weights are all the same and all round the same way.

Every trit of every plane is +1 on every group (three planes, masks full), a
row offset, x > 0, K = 12288: every term of every output has the same sign,
so nothing cancels.  The offset and scales are FP16 values for which each
rounding of an FP16 multiply-add chain 2*off + 2*s0, + 2*s1, + 2*s2 goes up
by half a unit in the last place (2.2 * 2^-11 of the decoded weight in all),
while their one rounding from FP32 goes up by 0.44 * 2^-11
(test_adversarial_values_round_the_same_way pins both on the CPU).  The
products take the decode that rounds once (an offset with residual planes,
or two residual planes) or, with one plane and no offset, the FP16 chain
that rounds at most once; all must meet |y - y_ref| <= 2e-3 * B.  The
large-magnitude cases scale the values by 2^14 (|off| + sum|s| = 37,144,
whose doubled value would overflow FP16), with FP32 outputs."""
import numpy as np
import pytest

import oracle as O
from ternary_weight_only_tern_amd import lib as L
from gpu_util import check_y, oracle_y, say, to_dev, upload_pack

# offset, s0, s1, s2 (FP16 values)
ADV = (0.56201171875, 0.755859375, 0.6884765625, 0.2607421875)
K = 12288
G = 128
N = 256


def _r16(v):
    return np.float64(np.float16(v))


def _ulp16(v):
    return 2.0 ** (np.floor(np.log2(abs(v))) - 10)


def test_adversarial_values_round_the_same_way():
    """The FP16 chain 2*off + 2*s0 -> + 2*s1 -> + 2*s2 rounds up by half an
    ulp at every step; one rounding of off + s0 + s1 + s2 goes up by 0.44 *
    2^-11 relative; scaled by 2^14 the values stay exact in FP16."""
    off, s0, s1, s2 = ADV
    steps, acc = [], 2 * off
    for s in (s0, s1, s2):
        exact = 2 * s + acc
        acc = _r16(exact)
        steps.append((acc - exact) / _ulp16(exact))
    assert all(abs(r - 0.5) < 1e-12 for r in steps)
    w = off + s0 + s1 + s2
    assert (acc / 2 - w) / w > 2.1 * 2 ** -11
    assert 0 < (_r16(w) - w) / w < 0.5 * 2 ** -11
    for v in ADV:
        assert _r16(v * 2 ** 14) == v * 2 ** 14


def _matrix(planes, offset_mode, scale):
    """All trits +1 on every plane and group, masks full, the ADV values
    times `scale` as offset (per row or per group) and scales."""
    ng = K // G
    trits = np.ones((planes, N, K), np.int8)
    scales = np.zeros((planes, N, ng), np.float16)
    for p in range(planes):
        scales[p] = np.float16(ADV[1 + p] * scale)
    masks = [np.ones((N, ng), bool) for _ in range(planes - 1)]
    words = (ng + 31) // 32
    bits = np.zeros((N, words), np.uint32)
    for g in range(ng):
        bits[:, g // 32] |= np.uint32(1) << np.uint32(g % 32)
    mask_bits = [bits.copy() for _ in range(planes - 1)]
    if offset_mode == O.OFF_ROW:
        offset = np.full(N, np.float16(ADV[0] * scale))
    elif offset_mode == O.OFF_GROUP:
        offset = np.full((N, ng), np.float16(ADV[0] * scale))
    else:
        offset = None
    return dict(trits=trits, scales=scales, masks=masks, mask_bits=mask_bits, offset=offset,
                offset_mode=offset_mode, n=N, k=K, group=G, planes=planes)


CASES = [  # planes, offset mode, scale, FP32 output
    (3, O.OFF_ROW, 1.0, False),
    (2, O.OFF_GROUP, 1.0, False),
    (3, O.OFF_NONE, 1.0, False),
    (2, O.OFF_NONE, 1.0, False),
    (3, O.OFF_ROW, 2.0 ** 14, True),
    (2, O.OFF_NONE, 2.0 ** 14, True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", [O.FMT_2BIT, O.FMT_B3])
@pytest.mark.parametrize("planes,off,scale,f32", CASES)
@pytest.mark.parametrize("m", [8, 64])
def test_tile_paths_at_the_edge_of_the_bound(planes, off, scale, f32, fmt, m):
    import torch
    say("tile edge", planes, off, scale, f32, fmt, m)
    mat = _matrix(planes, off, scale)
    x = np.full((m, K), np.float16(0.75))
    x[:, ::7] = np.float16(1.25)  # positive, not all equal
    pm = upload_pack(mat, fmt)
    xd = to_dev(x.view(np.uint16)).view(torch.float16)
    ydt = L.TERN_F32 if f32 else L.TERN_F16
    y_ref, b = oracle_y(mat, x)
    if m < 64:
        y = L.tern_gemv(pm, xd, ydt)  # m = 8: the 16-row product in both formats
    else:
        y = L.tern_gemm(pm, xd, ydt)
    torch.cuda.synchronize()
    rel = check_y(y, y_ref, b, f"tile edge m={m}")
    say("  max |y - y_ref| / B", rel)
    # the same through a plan (the grouped launch)
    yp = torch.empty((m, N), dtype=torch.float32 if f32 else torch.float16, device="cuda")
    plan = L.Plan([pm], [xd], [yp], y_dtype=ydt)
    plan.run()
    torch.cuda.synchronize()
    check_y(yp, y_ref, b, f"tile edge plan m={m}")
