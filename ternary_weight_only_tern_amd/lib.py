"""ctypes binding of libtern (include/tern.h), with the same names.

Argument marshalling only: torch supplies device memory and streams, every
step of packing and of the products runs in the HIP kernels behind the C ABI.
There is no CPU fallback: importing this module on a machine without the
built library raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_int32, c_size_t, c_uint32, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtern.so")

TERN_OK = 0
TERN_E_INVAL = -1
TERN_E_ALIGN = -2
TERN_E_UNSUPPORTED = -3
TERN_E_CORRUPT = -4
TERN_E_WORKSPACE = -5
TERN_E_HIP = -6

TERN_FMT_2BIT = 0
TERN_FMT_B3 = 1
TERN_OFF_NONE = 0
TERN_OFF_ROW = 1
TERN_OFF_GROUP = 2
TERN_F16 = 0
TERN_F32 = 1

(TERN_BUF_PLANE0, TERN_BUF_SCALE0, TERN_BUF_OFFSET, TERN_BUF_MASK, TERN_BUF_ROWPTR,
 TERN_BUF_BLOCKS1, TERN_BUF_BLOCKS2, TERN_BUF_RSCALE1, TERN_BUF_RSCALE2, TERN_NBUF) = range(10)

SYMBOLS = ["tern_row_stride", "tern_check", "tern_packed_sizes", "tern_workspace_bytes",
           "tern_pack", "tern_unpack", "tern_gemv", "tern_gemm", "tern_batch_workspace_bytes",
           "tern_gemv_batched", "tern_plan_create", "tern_plan_run", "tern_plan_run_events", "tern_plan_launches", "tern_plan_destroy", "tern_b3_min_stages", "tern_gemv_noalloc",
           "tern_rotated_workspace_bytes", "tern_plan_create_rotated",
           "tern_bits", "tern_quantize", "tern_rotate", "tern_rotate_batched", "tern_read_probe", "tern_status_str", "tern_last_error"]


class tern_matrix(ctypes.Structure):
    _fields_ = [("n", c_int32), ("k", c_int32), ("group", c_int32), ("planes", c_int32),
                ("format", c_int32), ("offset_mode", c_int32),
                ("plane0", c_void_p), ("scale0", c_void_p),
                ("mask", c_void_p * 2), ("rowptr", c_void_p * 2), ("blocks", c_void_p * 2),
                ("rscale", c_void_p * 2), ("offset", c_void_p), ("nnz", c_uint32 * 2)]


class TernError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_str(status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libtern.so (built in-tree by ternary_weight_only_tern_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m ternary_weight_only_tern_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER(tern_matrix)
    sig = {
        "tern_row_stride": (c_size_t, [c_int32, c_int32, c_int32]),
        "tern_check": (c_int32, [P]),
        "tern_packed_sizes": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, POINTER(c_uint32), c_int32, POINTER(c_size_t)]),
        "tern_workspace_bytes": (c_size_t, [P, c_int32]),
        "tern_pack": (c_int32, [c_void_p, c_void_p, P, c_void_p, c_size_t, c_void_p]),
        "tern_unpack": (c_int32, [P, c_void_p, c_void_p, c_size_t, c_void_p]),
        "tern_gemv": (c_int32, [P, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]),
        "tern_gemm": (c_int32, [P, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]),
        "tern_batch_workspace_bytes": (c_size_t, [P, c_int32, c_int32]),
        "tern_gemv_batched": (c_int32, [P, POINTER(c_void_p), POINTER(c_void_p), c_int32, c_int32, c_int32, c_void_p, c_size_t, c_void_p]),
        "tern_plan_create": (c_int32, [P, POINTER(c_void_p), POINTER(c_void_p), c_int32, c_int32, c_int32, c_void_p, c_size_t, POINTER(c_void_p)]),
        "tern_plan_run": (c_int32, [c_void_p, c_void_p]),
        "tern_plan_run_events": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p]),
        "tern_plan_launches": (c_int32, [c_void_p]),
        "tern_b3_min_stages": (ctypes.c_int64, [ctypes.c_int64]),
        "tern_rotated_workspace_bytes": (c_size_t, [c_void_p, c_int32, c_int32]),
        "tern_plan_create_rotated": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32,
                                              c_int32, c_void_p, c_size_t, c_void_p]),
        "tern_gemv_noalloc": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p]),
        "tern_plan_destroy": (None, [c_void_p]),
        "tern_bits": (c_int32, [P, POINTER(c_double), POINTER(c_double), POINTER(c_double)]),
        "tern_quantize": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_void_p,
                                    c_void_p, c_void_p]),
        "tern_rotate": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
        "tern_rotate_batched": (c_int32, [c_int32, POINTER(c_void_p), c_int32, POINTER(c_void_p), POINTER(c_int32),
                                          c_int32, POINTER(c_void_p), c_void_p]),
        "tern_read_probe": (c_int32, [c_void_p, c_size_t, c_void_p, c_void_p]),
        "tern_status_str": (ctypes.c_char_p, [c_int32]),
        "tern_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().tern_status_str(status).decode()


def last_error() -> str:
    return load().tern_last_error().decode()


def check(status: int) -> None:
    if status != TERN_OK:
        raise TernError(status, last_error())


# ---------------------------------------------------------------- thin wrappers
def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def tern_row_stride(k: int, group: int, fmt: int) -> int:
    return load().tern_row_stride(k, group, fmt)


def tern_packed_sizes(n, k, group, fmt, planes, nnz, offset_mode) -> list:
    out = (c_size_t * TERN_NBUF)()
    nz = (c_uint32 * 2)(*(list(nnz) + [0, 0])[:2])
    check(load().tern_packed_sizes(n, k, group, fmt, planes, nz, offset_mode, out))
    return list(out)


class PackedMatrix:
    """Device buffers of one packed matrix (torch tensors) and its descriptor."""

    def __init__(self, n, k, group, planes, fmt, offset_mode, nnz, device="cuda"):
        import torch
        self.n, self.k, self.group, self.planes, self.fmt = n, k, group, planes, fmt
        self.offset_mode = offset_mode
        self.nnz = [int(v) for v in (list(nnz) + [0, 0])[:2]]
        sz = tern_packed_sizes(n, k, group, fmt, planes, self.nnz, offset_mode)
        u8 = dict(dtype=torch.uint8, device=device)
        ng = k // group if group else 0
        self.plane0 = torch.zeros(max(sz[TERN_BUF_PLANE0], 1), **u8)
        self.scale0 = torch.zeros((n, ng), dtype=torch.float16, device=device)
        self.mask, self.rowptr, self.blocks, self.rscale = [], [], [], []
        for p in range(planes - 1):
            self.mask.append(torch.zeros((n, (ng + 31) // 32), dtype=torch.int32, device=device))
            self.rowptr.append(torch.zeros(n + 1, dtype=torch.int32, device=device))
            self.blocks.append(torch.zeros(max(sz[TERN_BUF_BLOCKS1 + p], 1), **u8))
            self.rscale.append(torch.zeros(max(self.nnz[p], 1), dtype=torch.float16, device=device))
        shape = (n,) if offset_mode == TERN_OFF_ROW else (n, ng)
        self.offset = (torch.zeros(shape, dtype=torch.float16, device=device)
                       if offset_mode != TERN_OFF_NONE else None)

    def desc(self) -> tern_matrix:
        d = tern_matrix()
        d.n, d.k, d.group, d.planes = self.n, self.k, self.group, self.planes
        d.format, d.offset_mode = self.fmt, self.offset_mode
        d.plane0, d.scale0 = _ptr(self.plane0), _ptr(self.scale0)
        for p in range(self.planes - 1):
            d.mask[p] = _ptr(self.mask[p])
            d.rowptr[p] = _ptr(self.rowptr[p])
            d.blocks[p] = _ptr(self.blocks[p])
            d.rscale[p] = _ptr(self.rscale[p])
            d.nnz[p] = self.nnz[p]
        d.offset = _ptr(self.offset)
        return d

    def nbytes(self) -> int:
        """Bytes of the representation a product reads (every buffer)."""
        sz = tern_packed_sizes(self.n, self.k, self.group, self.fmt, self.planes, self.nnz,
                               self.offset_mode)
        extra = max(self.planes - 2, 0) * (sz[TERN_BUF_MASK] + sz[TERN_BUF_ROWPTR])
        return sum(sz) + extra


def _zeroed(nbytes: int, device, stream):
    """A zero-filled workspace for a call on `stream`.  The fill is queued on
    torch's current stream.  When the call goes to a stream of the caller's,
    which may be another one, that stream waits for the fill, and the
    allocator is told that the stream uses the buffer, so that it does not
    hand the memory out again (and fill it on torch's stream) before the
    call has finished there."""
    import torch
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
    if stream is not None:
        ext = torch.cuda.ExternalStream(stream, device=ws.device)
        ext.wait_stream(torch.cuda.current_stream(ws.device))
        ws.record_stream(ext)
    return ws


def _workspace(desc: tern_matrix, m: int, device="cuda", stream=None):
    return _zeroed(load().tern_workspace_bytes(ctypes.byref(desc), m), device, stream)


def tern_pack(pm: PackedMatrix, trits, scales, mask_bits, offset=None, stream=None, ws=None):
    """Fill pm from device trits [P][N][K] int8, scales [P][N][K/G] fp16 and
    mask_bits [P-1][N][W] int32 (copied into pm.mask); plane-0 scales and the
    offset are copied into pm as given."""
    pm.scale0.copy_(scales[0])
    for p in range(pm.planes - 1):
        pm.mask[p].copy_(mask_bits[p])
    if pm.offset is not None:
        pm.offset.copy_(offset)
    d = pm.desc()
    ws = ws if ws is not None else _workspace(d, 1, pm.plane0.device, stream)
    rs = scales[1:].contiguous() if pm.planes > 1 else None
    check(load().tern_pack(_ptr(trits), _ptr(rs), ctypes.byref(d), _ptr(ws), ws.numel(), _stream(stream)))
    return pm


def tern_unpack(pm: PackedMatrix, out=None, stream=None, ws=None):
    import torch
    d = pm.desc()
    if out is None:
        out = torch.empty((pm.planes, pm.n, pm.k), dtype=torch.int8, device=pm.plane0.device)
    ws = ws if ws is not None else _workspace(d, 1, pm.plane0.device, stream)
    check(load().tern_unpack(ctypes.byref(d), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def _product(fn, pm, x, y_dtype, out, stream, ws):
    import torch
    m = x.shape[0]
    if out is None:
        dt = torch.float32 if y_dtype == TERN_F32 else torch.float16
        out = torch.empty((m, pm.n), dtype=dt, device=x.device)
    d = pm.desc()
    ws = ws if ws is not None else _workspace(d, m, x.device, stream)
    check(fn(ctypes.byref(d), _ptr(x), m, _ptr(out), y_dtype, _ptr(ws), ws.numel(), _stream(stream)))
    return out


def tern_gemv(pm, x, y_dtype=TERN_F16, out=None, stream=None, ws=None):
    return _product(load().tern_gemv, pm, x, y_dtype, out, stream, ws)


def tern_gemv_noalloc(pm, x, out, y_dtype=TERN_F16, stream=None):
    """tern_gemv with the library's fixed per-GPU workspace: the caller
    passes the output tensor `out` ([m][n], fp16 or fp32 per y_dtype); no
    device memory is allocated."""
    d = pm.desc()
    check(load().tern_gemv_noalloc(ctypes.byref(d), _ptr(x), x.shape[0], _ptr(out), y_dtype, _stream(stream)))
    return out


def tern_gemm(pm, x, y_dtype=TERN_F16, out=None, stream=None, ws=None):
    return _product(load().tern_gemm, pm, x, y_dtype, out, stream, ws)


def _arrays(mats, xs, ys):
    n = len(mats)
    descs = (tern_matrix * max(n, 1))(*[m.desc() for m in mats])
    xp = (c_void_p * max(n, 1))(*[x.data_ptr() for x in xs])
    yp = (c_void_p * max(n, 1))(*[y.data_ptr() for y in ys])
    return descs, xp, yp


def tern_gemv_batched(mats, xs, ys, y_dtype=TERN_F16, stream=None, ws=None):
    m = xs[0].shape[0] if xs else 0
    descs, xp, yp = _arrays(mats, xs, ys)
    if ws is None:
        ws = _zeroed(load().tern_batch_workspace_bytes(descs, len(mats), m), xs[0].device, stream)
    check(load().tern_gemv_batched(descs, xp, yp, len(mats), m, y_dtype, _ptr(ws), ws.numel(), _stream(stream)))
    return ys


def _event(e):
    """The HIP event handle of a torch.cuda.Event (created on first record)."""
    if e is None:
        return None
    if not e.cuda_event:
        e.record()
    return e.cuda_event


class Plan:
    """tern_plan_create / tern_plan_run / tern_plan_destroy; with `rots` (a
    list of fp16 rotation-block tensors or None per product) and rot_block,
    tern_plan_create_rotated.  The plan's workspace is a torch tensor that
    lives as long as the Plan: keep the Plan until runs queued on a stream
    other than torch's current one have finished (torch's allocator may hand
    the memory out again as soon as the Plan is gone)."""

    def __init__(self, mats, xs, ys, y_dtype=TERN_F16, rots=None, rot_block=128):
        import torch
        self.m = xs[0].shape[0] if xs else 0
        descs, xp, yp = _arrays(mats, xs, ys)
        if rots is not None:
            nbytes = load().tern_rotated_workspace_bytes(descs, len(mats), self.m)
        else:
            nbytes = load().tern_batch_workspace_bytes(descs, len(mats), self.m)
        # tern_plan_create writes every table and clears its counters itself
        # (synchronously, on the null stream): no fill is queued here, and the
        # caller's queued work on its inputs is finished first
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=xs[0].device)
        if xs:
            torch.cuda.current_stream(xs[0].device).synchronize()
        self._keep = (mats, xs, ys, rots)
        handle = c_void_p()
        if rots is not None:
            rp = (c_void_p * max(len(rots), 1))(*[None if r is None else r.data_ptr() for r in rots])
            check(load().tern_plan_create_rotated(descs, xp, rp, rot_block, yp, len(mats), self.m, y_dtype,
                                                  _ptr(self.ws), self.ws.numel(), ctypes.byref(handle)))
        else:
            check(load().tern_plan_create(descs, xp, yp, len(mats), self.m, y_dtype, _ptr(self.ws),
                                          self.ws.numel(), ctypes.byref(handle)))
        self.handle = handle

    def run(self, stream=None):
        check(load().tern_plan_run(self.handle, _stream(stream)))

    def run_events(self, before, after, stream=None):
        """run() recording two torch.cuda.Event objects (created with
        enable_timing=True) around the main decode launch."""
        check(load().tern_plan_run_events(self.handle, _stream(stream), _event(before), _event(after)))

    def launches(self):
        """Kernel launches one run() makes (tern_plan_launches)."""
        return int(load().tern_plan_launches(self.handle))

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tern_plan_destroy(self.handle)
            self.handle = None


def tern_quantize(w, mask_bits=None, group=128, iters=15, stream=None):
    """Quantize fp16 weights w [n][k] (device tensor; torch.float16 or its
    uint16 bits) into (trits int8 [2][n][k], scales fp16 [2][n][k/group],
    offsets fp16 [n][k/group]); mask_bits: int32/uint32 device bitmap
    [n][ceil(k/group/32)] of the groups that get the second plane, or None."""
    import torch
    n, k = w.shape
    ng = k // group if group else 0
    trits = torch.empty((2, n, k), dtype=torch.int8, device=w.device)
    scales = torch.empty((2, n, ng), dtype=torch.float16, device=w.device)
    offset = torch.empty((n, ng), dtype=torch.float16, device=w.device)
    check(load().tern_quantize(_ptr(w), n, k, group, _ptr(mask_bits) if mask_bits is not None else None, iters,
                               _ptr(trits), _ptr(scales), _ptr(offset), _stream(stream)))
    return trits, scales, offset


def tern_rotate(R, x, out=None, stream=None):
    """out = x rotated by the block-diagonal R (device tensors: R fp16
    [k/block][block][block], x fp16 [m][k]); returns out (fp16 [m][k])."""
    import torch
    m, k = x.shape
    block = R.shape[-1]
    if out is None:
        out = torch.empty((m, k), dtype=torch.float16, device=x.device)
    check(load().tern_rotate(_ptr(R), block, _ptr(x), m, k, _ptr(out), _stream(stream)))
    return out


def tern_rotate_batched(Rs, xs, outs=None, stream=None):
    """Rotate several activation tensors in one launch (same block size and
    number of rows); returns the outputs."""
    import torch
    n = len(xs)
    m = xs[0].shape[0] if n else 0
    block = Rs[0].shape[-1] if n else 128
    if outs is None:
        outs = [torch.empty_like(x) for x in xs]
    rp = (c_void_p * max(n, 1))(*[r.data_ptr() for r in Rs])
    xp = (c_void_p * max(n, 1))(*[x.data_ptr() for x in xs])
    op = (c_void_p * max(n, 1))(*[o.data_ptr() for o in outs])
    kk = (c_int32 * max(n, 1))(*[x.shape[1] for x in xs])
    check(load().tern_rotate_batched(n, rp, block, xp, kk, m, op, _stream(stream)))
    return outs


def tern_read_probe(buf, sink, stream=None) -> None:
    """Plain streaming read of a whole device tensor (measurement aid)."""
    check(load().tern_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def tern_b3_min_stages(stages: int = -2) -> int:
    """Threshold (in 64-row stages per launch) from which base-3 products at
    m <= 4 take the matrix-core stream kernel: stages >= 0 sets it, -1
    restores the default, -2 queries; returns the value in effect before."""
    return int(load().tern_b3_min_stages(stages))


def tern_bits(pm: PackedMatrix) -> dict:
    d = pm.desc()
    info, plane, storage = c_double(), c_double(), c_double()
    check(load().tern_bits(ctypes.byref(d), ctypes.byref(info), ctypes.byref(plane), ctypes.byref(storage)))
    return dict(info=info.value, plane=plane.value, storage=storage.value)
