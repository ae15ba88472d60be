"""An independent array formulation of the box load / store, used only to
cross-check the CPU oracle.

The oracle walks box elements one at a time and computes byte addresses; this
module instead builds a strided numpy view of the whole tensor, copies the
intersection of the box with the tensor by slicing into a zero-filled box
array, and applies the swizzle as one fancy-index permutation.  The swizzle
here is written in the mask-then-shift form of CuTe's Swizzle<B,M,S>
(offset ^ ((offset & yyy_mask) >> S), yyy_mask = (2^B - 1) << (M+S)), not the
oracle's shift-then-mask form.
"""
from __future__ import annotations

import numpy as np

_DT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def perm(n: int, swz) -> np.ndarray:
    b, m, s = swz
    e = np.arange(n, dtype=np.int64)
    if b == 0:
        return e
    yyy = ((1 << b) - 1) << (m + s)
    return e ^ ((e & yyy) >> s)


def tensor_view(buf: np.ndarray, es, dims, strides) -> np.ndarray:
    """Outermost-first ndarray view of the tensor bytes in buf."""
    shape = tuple(reversed([int(x) for x in dims]))
    bstr = tuple(reversed([es] + [int(x) for x in strides]))
    return np.ndarray(shape, dtype=_DT[es], buffer=buf, offset=0, strides=bstr)


def _intersection(corner, dims, box):
    src, dst = [], []
    for c, n, b in zip(corner, dims, box):
        lo, hi = max(int(c), 0), min(int(c) + int(b), int(n))
        if lo >= hi:
            return None
        src.append(slice(lo, hi))
        dst.append(slice(lo - int(c), hi - int(c)))
    return tuple(reversed(src)), tuple(reversed(dst))


def load_tiles(buf, es, dims, strides, box, swz, corners) -> np.ndarray:
    view = tensor_view(buf, es, dims, strides)
    n_el = int(np.prod(box))
    p = perm(n_el, swz)
    out = np.zeros((len(corners), n_el), dtype=_DT[es])
    for t, c in enumerate(corners):
        z = np.zeros(tuple(reversed([int(x) for x in box])), dtype=_DT[es])
        inter = _intersection(c, dims, box)
        if inter is not None:
            z[inter[1]] = view[inter[0]]
        out[t, p] = z.reshape(-1)
    return out.view(np.uint8).reshape(-1)


def store_tiles(buf, es, dims, strides, box, swz, corners, packed) -> None:
    view = tensor_view(buf, es, dims, strides)
    n_el = int(np.prod(box))
    p = perm(n_el, swz)
    tiles = np.ascontiguousarray(packed).view(_DT[es]).reshape(len(corners), n_el)
    for t, c in enumerate(corners):
        z = tiles[t, p].reshape(tuple(reversed([int(x) for x in box])))
        inter = _intersection(c, dims, box)
        if inter is not None:
            view[inter[0]] = z[inter[1]]


def inbounds_mask(es, dims, box, corner) -> np.ndarray:
    """Boolean box (outermost first) of the elements inside the tensor."""
    m = np.ones(tuple(reversed([int(x) for x in box])), dtype=bool)
    for d, (c, n, b) in enumerate(zip(corner, dims, box)):
        g = int(c) + np.arange(int(b))
        ok = (g >= 0) & (g < int(n))
        shape = [1] * len(box)
        shape[len(box) - 1 - d] = int(b)
        m &= ok.reshape(shape)
    return m
