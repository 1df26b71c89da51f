"""CPU oracle for packed ternary (W1.58A16) linear weights.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library (no kernels,
headers, tables or pre/post-processing); the two meet only on seeded inputs
produced by ``ternary_weight_only_tern_amd.synth``, a module that holds none of
the method's arithmetic.

What is computed, and where the pages define it
------------------------------------------------
* Representation.  A quantized linear weight is a stack of trit planes
  ``T_p in {-1,0,+1}^{N x K}`` with one FP16 scale per (output row, group of G
  input columns), an optional asymmetric offset, and second/third planes that
  exist only on salience-selected groups.  Sources: "Post-Training
  Ternarization of Qwen3-4B" (arXiv 2609.01962v1 summary) §4.3 (E2M-ATQ: an
  offset plus ternary planes with scales; grid {mu-alpha, mu, mu+alpha}), §4.4
  (salience masks; 3.6 % of weights get a second plane), §4.5 (group size
  128); arXiv 2609.09240 (Qwen3-8B scale-up), representation section (one
  plane for most weights, a salience-selected second plane, per-group
  offsets/scales).  The displayed reconstruction equation is missing from the
  extracted text; the reading used here is additive planes sharing the group
  structure:  W[n,k] = off(n,g) + sum_p m_p[n,g] * s_p[n,g] * T_p[n,k],
  g = k // G, m_0 = 1.
* Product.  y[m,n] = sum_k W[n,k] x[m,k], evaluated group by group from the
  unpacked trits: "matrix multiplications become additions and subtractions"
  ("Can ternary LLMs hit 1.58 bits per weight", How It Works), and packed
  planes are consumed directly (2609.01962 §14, §15; 2609.09240, direct
  packed execution).  fp16 inputs are converted exactly to fp64; every
  product s*t*x is exact in fp64 and the only error is fp64 summation order.
* Packing.  The pages require a lossless, lattice-aware serialization of the
  planes, scales and offsets (2609.01962 §9.1, §15; 2609.09240 packing
  paragraph) but print no byte layout.  The layouts below are this library's
  own definition (the readings are listed in the design notes):

  2-bit plane.  code(t) = t mod 4 (2-bit two's complement: 0 -> 00, +1 -> 01,
  -1 -> 11; 10 is invalid).  Each 32-bit little-endian word holds 16
  consecutive trits of a row: the trit at offset o (0..15) occupies bits
  [b, b+1] with b = 16*(o % 2) + 2*(o // 2), i.e. even offsets in the low
  half-word, odd offsets in the high half-word, ascending.  Row stride K/4.

  Base-3 plane.  Each group of G trits is stored in ceil(G/5) bytes; byte j
  of a group holds the group's trits 5j..5j+4 as sum_i (t_{5j+i}+1) * 3**i
  (least-significant digit first); positions past the end of the group are
  zero trits (digit 1).  Groups follow each other along the row; the row is
  zero-padded to a multiple of 16 bytes.  Bytes 243..255 are invalid.

  Residual plane p >= 1.  A bitmap mask (uint32 words, bit g%32 of word g//32
  of row n set when group g of row n carries plane p), rowptr = exclusive
  prefix of per-row popcounts (N+1 uint32), blocks = the 2-bit encoding of the
  G trits of each masked group in (n, g) order (G/4 bytes each), rscale = the
  plane's FP16 scale of each masked group in the same order.  Trits outside
  the mask must be zero.
* Bits per weight.  Information content log2(3) bits per stored trit, counted
  over the planes actually present (2609.01962 §3.2 and §7.1: 1.641 effective
  bits per weight against the 1.585 single-plane ideal; 2609.09240,
  representation section, rate in terms of the fraction f2 of weights with a
  second plane).
* Acceptance bound.  |y - y_ref| <= 2e-3 * B with
  B[m,n] = sum_k (|off(n,g)| + sum_p m_p |s_p| |T_p[n,k]|) |x[m,k]|.

All functions take and return numpy arrays.  Floating point is fp64.
"""
from __future__ import annotations

import math

import numpy as np

FMT_2BIT = 0
FMT_B3 = 1
OFF_NONE = 0
OFF_ROW = 1
OFF_GROUP = 2


class PackError(ValueError):
    """Input to packing violates the representation (bad trit, trit outside mask)."""


class CorruptError(ValueError):
    """Packed bytes are not a valid encoding."""


# --------------------------------------------------------------------------
# sizes
# --------------------------------------------------------------------------
def b3_bytes_per_group(group: int) -> int:
    return (group + 4) // 5


def row_stride(k: int, group: int, fmt: int) -> int:
    """Bytes per packed plane-0 row."""
    if fmt == FMT_2BIT:
        return k // 4
    ng = k // group
    raw = ng * b3_bytes_per_group(group)
    return (raw + 15) // 16 * 16


def mask_words(k: int, group: int) -> int:
    return (k // group + 31) // 32


# --------------------------------------------------------------------------
# 2-bit encoding
# --------------------------------------------------------------------------
def _bitpos(o: int) -> int:
    """Bit position of the trit at offset o (0..15) inside its 32-bit word."""
    return 16 * (o % 2) + 2 * (o // 2)


def pack_2bit_row(trits: np.ndarray) -> np.ndarray:
    """One row (length multiple of 16) of trits -> bytes, plain loops."""
    trits = np.asarray(trits)
    assert trits.ndim == 1 and trits.size % 16 == 0
    out = bytearray()
    for w0 in range(0, trits.size, 16):
        word = 0
        for o in range(16):
            t = int(trits[w0 + o])
            if t not in (-1, 0, 1):
                raise PackError(f"trit {t} at column {w0 + o}")
            word |= (t & 3) << _bitpos(o)
        out += word.to_bytes(4, "little")
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def pack_2bit(trits: np.ndarray) -> np.ndarray:
    """[N][K] trits -> [N][K/4] bytes.  Vectorised form of pack_2bit_row."""
    t = np.asarray(trits)
    n, k = t.shape
    assert k % 16 == 0
    if not np.isin(t, (-1, 0, 1)).all():
        bad = np.argwhere(~np.isin(t, (-1, 0, 1)))[0]
        raise PackError(f"trit {t[tuple(bad)]} at {tuple(bad)}")
    codes = (t.astype(np.int64) & 3).astype(np.uint64).reshape(n, k // 16, 16)
    shifts = np.array([_bitpos(o) for o in range(16)], dtype=np.uint64)
    words = np.bitwise_or.reduce(codes << shifts, axis=2).astype("<u4")
    return words.view(np.uint8).reshape(n, k // 4)


def unpack_2bit(packed: np.ndarray, k: int) -> np.ndarray:
    """[N][K/4] bytes -> [N][K] int8 trits; raises CorruptError on code 10."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    n = p.shape[0]
    words = p.reshape(n, k // 4).view("<u4").astype(np.uint64)
    out = np.empty((n, k // 16, 16), dtype=np.int8)
    for o in range(16):
        code = (words >> np.uint64(_bitpos(o))) & np.uint64(3)
        if (code == 2).any():
            raise CorruptError("2-bit code 0b10 is not a trit")
        out[:, :, o] = np.where(code == 3, -1, code.astype(np.int8))
    return out.reshape(n, k)


# --------------------------------------------------------------------------
# base-3 encoding
# --------------------------------------------------------------------------
def pack_b3_group(trits: np.ndarray) -> bytes:
    """One group of trits -> ceil(G/5) bytes, plain loops."""
    out = bytearray()
    g = len(trits)
    for j in range(b3_bytes_per_group(g)):
        v = 0
        for i in range(5):
            pos = 5 * j + i
            t = int(trits[pos]) if pos < g else 0
            if t not in (-1, 0, 1):
                raise PackError(f"trit {t} at group offset {pos}")
            v += (t + 1) * 3 ** i
        out.append(v)
    return bytes(out)


def pack_b3(trits: np.ndarray, group: int) -> np.ndarray:
    """[N][K] trits -> [N][row_stride] bytes (group-aligned base-3)."""
    t = np.asarray(trits)
    n, k = t.shape
    if not np.isin(t, (-1, 0, 1)).all():
        bad = np.argwhere(~np.isin(t, (-1, 0, 1)))[0]
        raise PackError(f"trit {t[tuple(bad)]} at {tuple(bad)}")
    ng = k // group
    nb = b3_bytes_per_group(group)
    padded = np.zeros((n, ng, nb * 5), dtype=np.int64)
    padded[:, :, :group] = t.reshape(n, ng, group)
    digits = (padded + 1).reshape(n, ng, nb, 5)
    weights = np.array([1, 3, 9, 27, 81], dtype=np.int64)
    vals = (digits * weights).sum(axis=3).astype(np.uint8).reshape(n, ng * nb)
    out = np.zeros((n, row_stride(k, group, FMT_B3)), dtype=np.uint8)
    out[:, : ng * nb] = vals
    return out


def unpack_b3(packed: np.ndarray, k: int, group: int) -> np.ndarray:
    """[N][row_stride] bytes -> [N][K] trits.

    Raises CorruptError on a byte above 242 or a non-zero padding trit.
    Alignment bytes at the end of a row are not part of any group and are
    not inspected.
    """
    p = np.asarray(packed, dtype=np.uint8)
    n = p.shape[0]
    ng = k // group
    nb = b3_bytes_per_group(group)
    body = p[:, : ng * nb].astype(np.int64).reshape(n, ng, nb)
    if (body > 242).any():
        raise CorruptError("base-3 byte above 242")
    digits = np.empty((n, ng, nb, 5), dtype=np.int64)
    rem = body.copy()
    for i in range(5):
        digits[..., i] = rem % 3
        rem //= 3
    trits = (digits - 1).reshape(n, ng, nb * 5)
    if (trits[:, :, group:] != 0).any():
        raise CorruptError("non-zero padding trit in the last byte of a group")
    return trits[:, :, :group].reshape(n, k).astype(np.int8)


# --------------------------------------------------------------------------
# masks and residual planes
# --------------------------------------------------------------------------
def mask_bool(mask_bits: np.ndarray, ngroups: int) -> np.ndarray:
    """uint32 bitmap [N][W] -> bool [N][ngroups] (bit g%32 of word g//32)."""
    mb = np.asarray(mask_bits, dtype=np.uint32)
    n = mb.shape[0]
    out = np.zeros((n, ngroups), dtype=bool)
    for g in range(ngroups):
        out[:, g] = (mb[:, g // 32] >> np.uint32(g % 32)) & np.uint32(1) == 1
    return out


def pack_residual(trits_p: np.ndarray, scale_p: np.ndarray, mask_bits: np.ndarray,
                  group: int):
    """One residual plane -> (rowptr [N+1] u32, blocks [nnz][G/4] u8, rscale [nnz] f16)."""
    t = np.asarray(trits_p)
    n, k = t.shape
    ng = k // group
    m = mask_bool(mask_bits, ng)
    tg = t.reshape(n, ng, group)
    outside = (tg != 0) & ~m[:, :, None]
    if outside.any():
        bad = np.argwhere(outside)[0]
        raise PackError(f"non-zero residual trit outside the mask at row {bad[0]} group {bad[1]}")
    counts = m.sum(axis=1)
    rowptr = np.zeros(n + 1, dtype=np.uint32)
    rowptr[1:] = np.cumsum(counts)
    rows, groups = np.nonzero(m)  # row-major (n, g) order
    sel = tg[rows, groups]         # [nnz][G]
    if sel.shape[0]:
        blocks = pack_2bit(sel)
    else:
        blocks = np.zeros((0, group // 4), dtype=np.uint8)
    rscale = np.asarray(scale_p, dtype=np.float16)[rows, groups]
    return rowptr, blocks, rscale


def unpack_residual(rowptr, blocks, mask_bits, n: int, k: int, group: int) -> np.ndarray:
    """Inverse of pack_residual for the trits; zeros outside the mask.

    Raises CorruptError when rowptr disagrees with the mask popcounts.
    """
    ng = k // group
    m = mask_bool(mask_bits, ng)
    counts = m.sum(axis=1)
    expect = np.zeros(n + 1, dtype=np.int64)
    expect[1:] = np.cumsum(counts)
    if not np.array_equal(np.asarray(rowptr, dtype=np.int64), expect):
        raise CorruptError("rowptr does not match the mask popcounts")
    out = np.zeros((n, ng, group), dtype=np.int8)
    rows, groups = np.nonzero(m)
    if rows.size:
        out[rows, groups] = unpack_2bit(np.asarray(blocks).reshape(rows.size, group // 4), group)
    return out.reshape(n, k)


# --------------------------------------------------------------------------
# whole matrix
# --------------------------------------------------------------------------
def pack(trits, scales, mask_bits, offset, group: int, fmt: int):
    """Unpacked representation -> dict of packed arrays.

    trits [P][N][K] int8, scales [P][N][K/G] fp16 (dense; residual entries
    outside the mask are ignored), mask_bits [P-1][N][W] u32, offset fp16
    [N], [N][K/G] or None.
    """
    trits = np.asarray(trits)
    planes, n, k = trits.shape
    if fmt == FMT_2BIT:
        plane0 = pack_2bit(trits[0])
    else:
        plane0 = pack_b3(trits[0], group)
    out = dict(n=n, k=k, group=group, planes=planes, fmt=fmt, plane0=plane0,
               scale0=np.asarray(scales[0], dtype=np.float16).copy(),
               mask=[], rowptr=[], blocks=[], rscale=[],
               offset=None if offset is None else np.asarray(offset, dtype=np.float16).copy())
    for p in range(1, planes):
        rp, bl, rs = pack_residual(trits[p], scales[p], mask_bits[p - 1], group)
        out["mask"].append(np.asarray(mask_bits[p - 1], dtype=np.uint32).copy())
        out["rowptr"].append(rp)
        out["blocks"].append(bl)
        out["rscale"].append(rs)
    return out


def unpack(pk) -> tuple:
    """Packed dict -> (trits [P][N][K] int8, scale views).

    Returns (trits, residual_scale_dense) where residual_scale_dense[p-1] is
    an fp16 [N][K/G] array holding rscale at masked groups and 0 elsewhere.
    """
    n, k, group, planes = pk["n"], pk["k"], pk["group"], pk["planes"]
    ng = k // group
    trits = np.zeros((planes, n, k), dtype=np.int8)
    if pk["fmt"] == FMT_2BIT:
        trits[0] = unpack_2bit(pk["plane0"], k)
    else:
        trits[0] = unpack_b3(pk["plane0"], k, group)
    rdense = []
    for p in range(1, planes):
        trits[p] = unpack_residual(pk["rowptr"][p - 1], pk["blocks"][p - 1],
                                   pk["mask"][p - 1], n, k, group)
        m = mask_bool(pk["mask"][p - 1], ng)
        d = np.zeros((n, ng), dtype=np.float16)
        d[m] = pk["rscale"][p - 1]
        rdense.append(d)
    return trits, rdense


# --------------------------------------------------------------------------
# arithmetic (fp64)
# --------------------------------------------------------------------------
def _f64(a):
    return np.asarray(a).astype(np.float64)


def _offset_dense(offset, offset_mode: int, n: int, ng: int) -> np.ndarray:
    if offset_mode == OFF_NONE or offset is None:
        return np.zeros((n, ng))
    o = _f64(offset)
    if offset_mode == OFF_ROW:
        return np.repeat(o.reshape(n, 1), ng, axis=1)
    return o.reshape(n, ng)


def gemv(trits, scales, masks, offset, offset_mode: int, x, group: int) -> np.ndarray:
    """y[m,n] = sum_g [off(n,g) * xs[m,g] + sum_p m_p s_p (T_p[n,g-block] . x[m,g-block])].

    trits [P][N][K]; scales [P][N][K/G] (plane p's scale per group); masks
    bool [P-1][N][K/G] (or None when P == 1); x [M][K].  fp64 throughout.
    """
    t = _f64(trits)
    planes, n, k = t.shape
    ng = k // group
    xm = _f64(x)
    mrows = xm.shape[0]
    xg = xm.reshape(mrows, ng, group)
    y = np.zeros((mrows, n))
    off = _offset_dense(offset, offset_mode, n, ng)
    xs = xg.sum(axis=2)                       # [M][ng]
    y += xs @ off.T
    for p in range(planes):
        s = _f64(scales[p])                   # [N][ng]
        if p > 0:
            s = s * np.asarray(masks[p - 1], dtype=bool)
        tg = t[p].reshape(n, ng, group)
        for g in range(ng):
            dot = xg[:, g, :] @ tg[:, g, :].T  # [M][N]
            y += dot * s[:, g][None, :]
    return y


def dequant(trits, scales, masks, offset, offset_mode: int, group: int) -> np.ndarray:
    """Dense fp64 W[n,k] = off(n,g) + sum_p m_p s_p T_p[n,k]."""
    t = _f64(trits)
    planes, n, k = t.shape
    ng = k // group
    w = np.repeat(_offset_dense(offset, offset_mode, n, ng), group, axis=1)
    for p in range(planes):
        s = _f64(scales[p])
        if p > 0:
            s = s * np.asarray(masks[p - 1], dtype=bool)
        w += np.repeat(s, group, axis=1) * t[p]
    return w


def bound(trits, scales, masks, offset, offset_mode: int, x, group: int) -> np.ndarray:
    """B[m,n] = sum_k (|off| + sum_p m_p |s_p| |T_p[n,k]|) |x[m,k]|."""
    t = np.abs(_f64(trits))
    planes, n, k = t.shape
    ng = k // group
    a = np.repeat(np.abs(_offset_dense(offset, offset_mode, n, ng)), group, axis=1)
    for p in range(planes):
        s = np.abs(_f64(scales[p]))
        if p > 0:
            s = s * np.asarray(masks[p - 1], dtype=bool)
        a += np.repeat(s, group, axis=1) * t[p]
    return np.abs(_f64(x)) @ a.T


def gemv_packed(pk, x) -> np.ndarray:
    """The plain CPU unpack-and-dot: decode the packed bytes, then gemv()."""
    trits, rdense = unpack(pk)
    ng = pk["k"] // pk["group"]
    scales = [pk["scale0"]] + rdense
    masks = [mask_bool(mb, ng) for mb in pk["mask"]]
    mode = OFF_NONE if pk["offset"] is None else (OFF_ROW if pk["offset"].ndim == 1 else OFF_GROUP)
    return gemv(trits, scales, masks, pk["offset"], mode, x, pk["group"])


def accept(y, y_ref, b, rel: float = 2e-3) -> np.ndarray:
    """Elementwise acceptance: finite and |y - y_ref| <= rel * B (B = 0 -> y == 0)."""
    y = _f64(y)
    return np.isfinite(y) & (np.abs(y - y_ref) <= rel * b)


# --------------------------------------------------------------------------
# bits per weight
# --------------------------------------------------------------------------
def info_bits(f2: float, f3: float = 0.0) -> float:
    """Trit information per weight when fractions f2, f3 carry extra planes."""
    return math.log2(3.0) * (1.0 + f2 + f3)


def bits(pk) -> dict:
    """info / plane / storage bits per weight of a packed matrix."""
    n, k, group = pk["n"], pk["k"], pk["group"]
    weights = n * k
    stored_trits = weights + sum(len(r) * group for r in pk["rscale"])
    plane_bytes = pk["plane0"].size + sum(b.size for b in pk["blocks"])
    total = plane_bytes + pk["scale0"].size * 2
    for p in range(len(pk["blocks"])):
        total += pk["rscale"][p].size * 2 + pk["mask"][p].size * 4 + pk["rowptr"][p].size * 4
    if pk["offset"] is not None:
        total += pk["offset"].size * 2
    return dict(info=math.log2(3.0) * stored_trits / weights,
                plane=8.0 * plane_bytes / weights,
                storage=8.0 * total / weights,
                total_bytes=total)
