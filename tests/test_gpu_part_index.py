"""2-bit plans whose products are cut into K parts or carry two residual
planes: the plan indexes every residual plane per K part, and items stage
their entries from that index (or, past the staging capacity, take the mask
path).  Against the oracle's bound, two runs bit-identical, on single
products (which a plan cuts into K parts to fill the GPU) and a batch."""
import numpy as np
import pytest

import oracle as O
from ternary_weight_only_tern_amd import lib as L
from ternary_weight_only_tern_amd import synth
from gpu_util import check_y, oracle_y, say, small_matrix, to_dev, upload_pack

pytestmark = pytest.mark.gpu


def _dev16(a):
    import torch
    return to_dev(np.ascontiguousarray(a).view(np.uint16)).view(torch.float16)


# (n, k, group, planes, residual fraction, offsets, m): K-split single
# products with one and two residual planes, whole rows with two, a dense
# residual (every group, both planes: past the staging capacity), group 64
CASES = [
    (4096, 12288, 128, 3, 0.20, O.OFF_ROW, 1),
    (1024, 8192, 128, 2, 0.10, O.OFF_NONE, 1),
    (700, 3072, 128, 3, 0.30, O.OFF_GROUP, 3),
    (256, 4096, 128, 3, 1.00, O.OFF_ROW, 1),
    (600, 6144, 64, 3, 0.25, O.OFF_NONE, 2),
    (300, 2048, 64, 2, 0.50, O.OFF_GROUP, 4),
]


@pytest.mark.parametrize("n,k,group,planes,frac,off,m", CASES)
def test_single_product_plan_with_part_index(n, k, group, planes, frac, off, m):
    import torch
    say("part index", n, k, group, planes, frac, off, m)
    mat, rng = small_matrix(n, k, group, planes, frac, seed=n + k + planes, offset_mode=off, scale_law="lognormal")
    pm = upload_pack(mat, O.FMT_2BIT)
    x_h = synth.draw_x(rng, m, k, "student_t3")
    x = _dev16(x_h)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    plan = L.Plan([pm], [x], [y], y_dtype=L.TERN_F32)
    plan.run()
    torch.cuda.synchronize()
    first = y.clone()
    plan.run()
    torch.cuda.synchronize()
    assert torch.equal(y, first), "runs differ"
    y_ref, b = oracle_y(mat, x_h)
    check_y(y, y_ref, b, "single-product plan")


def test_batch_plan_with_part_index():
    """A layer-like batch mixing products with and without an index per K
    part (two residual planes, one, none) at M=1 and M=5."""
    import torch
    say("part index batch")
    specs = [(512, 4096, 3, 0.2, O.OFF_ROW), (1024, 2048, 2, 0.1, O.OFF_NONE), (256, 6144, 1, 0.0, O.OFF_GROUP),
             (384, 8192, 3, 0.15, O.OFF_NONE)]
    mats = [small_matrix(n, k, 128, p, f, seed=80 + i, offset_mode=o)[0] for i, (n, k, p, f, o) in enumerate(specs)]
    pms = [upload_pack(mt, O.FMT_2BIT) for mt in mats]
    rng = np.random.default_rng(81)
    for m in (1, 5):
        xs_h = [synth.draw_x(rng, m, mt["k"], "normal") for mt in mats]
        xs = [_dev16(x) for x in xs_h]
        ys = [torch.empty((m, mt["n"]), dtype=torch.float32, device="cuda") for mt in mats]
        plan = L.Plan(pms, xs, ys, y_dtype=L.TERN_F32)
        plan.run()
        torch.cuda.synchronize()
        for i, (mt, x_h, y) in enumerate(zip(mats, xs_h, ys)):
            y_ref, b = oracle_y(mt, x_h)
            check_y(y, y_ref, b, f"batch product {i} at m={m}")
