"""tern_gemv and tern_gemv_noalloc captured into HIP graphs.  Every route a
single product takes at m <= 63 (the decode kernels with their K-part
reduce, the 16-row matrix-core product, whose tiles and reduce table are
written on the device, and the matrix-core tiles) takes no table from host
memory, so a captured call replays correctly: each replay, after the
activations change and with eager calls and synchronisations in between,
equals the eager call bitwise and meets the oracle's bound."""
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


@pytest.mark.parametrize("fmt,m,noalloc", [(O.FMT_2BIT, 8, False), (O.FMT_B3, 8, False), (O.FMT_2BIT, 20, True),
                                           (O.FMT_B3, 32, True), (O.FMT_2BIT, 1, False), (O.FMT_B3, 3, True),
                                           (O.FMT_2BIT, 40, False)])
def test_gemv_captured_replays(fmt, m, noalloc):
    import torch
    say("captured tern_gemv", fmt, m, "noalloc" if noalloc else "")
    mat, rng = small_matrix(300, 3840, 128, 3, 0.2, seed=500 + m, offset_mode=O.OFF_ROW, scale_law="lognormal")
    pm = upload_pack(mat, fmt)
    x_h = synth.draw_x(rng, m, 3840, "student_t3")
    x = _dev16(x_h)
    y = torch.empty((m, 300), dtype=torch.float32, device="cuda")
    ws = L._workspace(pm.desc(), m)
    stream = torch.cuda.Stream()

    def call(s):
        if noalloc:
            L.tern_gemv_noalloc(pm, x, y, y_dtype=L.TERN_F32, stream=s)
        else:
            L.tern_gemv(pm, x, y_dtype=L.TERN_F32, out=y, stream=s, ws=ws)

    with torch.cuda.stream(stream):
        call(stream.cuda_stream)
    torch.cuda.synchronize()
    y_ref, b = oracle_y(mat, x_h)
    check_y(y, y_ref, b, "eager call")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call(stream.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        x_h = synth.draw_x(rng, m, 3840, "normal")
        x.copy_(_dev16(x_h))
        call(None)  # eager, on the current stream
        torch.cuda.synchronize()
        want = y.clone()
        y.fill_(float("nan"))
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {rep} differs from the eager call"
        y_ref, b = oracle_y(mat, x_h)
        check_y(y, y_ref, b, f"replay {rep}")
