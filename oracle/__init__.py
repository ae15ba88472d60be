"""CPU oracle for the tiled bulk copy -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The product library never loads it and shares no code
with it: the oracle (``oracle.c``) has its own map struct, validator, swizzle
and address arithmetic, written from the pages' definitions and computed one
element at a time on one host thread.

The wrappers below only marshal numpy arrays into the C functions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# Test hook: TMAP_ORACLE_SRC names another copy of oracle.c, built into a
# liboracle.so beside it.  The mutation tests use it to run the pins against
# copies of the oracle with one mistake planted each.
_SRC = os.environ.get("TMAP_ORACLE_SRC") or os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(os.path.dirname(os.path.abspath(_SRC)), "liboracle.so")

MAX_RANK = 5

# Reject codes returned by validate(); 1..4 are the pages' rules.
REJECT_NAMES = {
    0: "ok", 1: "rank", 2: "box_max", 3: "stride_16", 4: "base_16", 5: "base_null",
    6: "elem_size", 7: "dim_range", 8: "box_zero", 9: "stride_range", 10: "elem_stride",
    11: "row_16", 12: "box_bytes", 13: "swizzle_range", 14: "swizzle_shift",
    15: "swizzle_tile", 16: "span",
}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain C11, -O2, one thread)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fPIC",
                               "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


class _CMap(ctypes.Structure):
    _fields_ = [("es", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("dims", ctypes.c_uint64 * MAX_RANK), ("stride", ctypes.c_uint64 * MAX_RANK),
                ("box", ctypes.c_uint32 * MAX_RANK),
                ("swz_b", ctypes.c_int32), ("swz_m", ctypes.c_int32), ("swz_s", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        u8p, i32p, u64p, u32p = P(ctypes.c_uint8), P(ctypes.c_int32), P(ctypes.c_uint64), P(ctypes.c_uint32)
        mp = P(_CMap)
        lib.oracle_validate.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64, u64p, u64p,
                                        u32p, u32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        lib.oracle_validate.restype = ctypes.c_int
        lib.oracle_swizzle.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        lib.oracle_swizzle.restype = ctypes.c_uint64
        lib.oracle_sweep_count.argtypes = [mp]
        lib.oracle_sweep_count.restype = ctypes.c_int64
        lib.oracle_sweep_coords.argtypes = [mp, ctypes.c_int64, i32p]
        lib.oracle_sweep_coords.restype = None
        lib.oracle_box_bytes.argtypes = [mp]
        lib.oracle_box_bytes.restype = ctypes.c_uint64
        lib.oracle_load_tiles.argtypes = [mp, u8p, ctypes.c_uint64, i32p, ctypes.c_int64, u8p]
        lib.oracle_load_tiles.restype = ctypes.c_int
        lib.oracle_store_tiles.argtypes = [mp, u8p, ctypes.c_uint64, i32p, ctypes.c_int64, u8p]
        lib.oracle_store_tiles.restype = ctypes.c_int
        lib.oracle_roundtrip.argtypes = [mp, u8p, ctypes.c_uint64, mp, u8p, ctypes.c_uint64,
                                         i32p, ctypes.c_int64, u8p]
        lib.oracle_roundtrip.restype = ctypes.c_int
        lib.oracle_roundtrip_add_f32.argtypes = [mp, u8p, ctypes.c_uint64, mp, u8p, ctypes.c_uint64,
                                                 i32p, ctypes.c_int64, ctypes.c_float, u8p]
        lib.oracle_roundtrip_add_f32.restype = ctypes.c_int
        lib.oracle_bulk_copy.argtypes = [u8p, u8p, ctypes.c_uint64]
        lib.oracle_bulk_copy.restype = None
        lib.oracle_inb_elems.argtypes = [mp, i32p, ctypes.c_int64]
        lib.oracle_inb_elems.restype = ctypes.c_uint64
        _lib = lib
    return _lib


@dataclass
class Map:
    """A tensor map as the oracle sees it: dims/box innermost first, byte
    strides for dims 1..rank-1 (dimension 0 is contiguous)."""
    es: int
    dims: Sequence[int]
    strides: Sequence[int]          # rank-1 byte strides
    box: Sequence[int]
    swizzle: Sequence[int] = (0, 0, 0)
    rank: int = field(init=False)

    def __post_init__(self):
        self.rank = len(self.dims)
        assert len(self.box) == self.rank and len(self.strides) == self.rank - 1

    def _c(self) -> _CMap:
        m = _CMap()
        m.es, m.rank = self.es, self.rank
        for d in range(MAX_RANK):
            m.dims[d] = int(self.dims[d]) if d < self.rank else 1
            m.box[d] = int(self.box[d]) if d < self.rank else 1
            m.stride[d] = (self.es if d == 0 else int(self.strides[d - 1])) if d < self.rank else 0
        m.swz_b, m.swz_m, m.swz_s = (int(x) for x in self.swizzle)
        return m


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def validate(es, rank, base, dims, strides, box, estrides=None, swizzle=(0, 0, 0)) -> int:
    """0 when the encode parameters are accepted, else a reject code."""
    lib = _load()
    d = (ctypes.c_uint64 * MAX_RANK)(*[int(x) for x in list(dims)[:MAX_RANK]])
    s = (ctypes.c_uint64 * MAX_RANK)(*[int(x) for x in list(strides)[:MAX_RANK]])
    b = (ctypes.c_uint32 * MAX_RANK)(*[int(x) for x in list(box)[:MAX_RANK]])
    e = None if estrides is None else (ctypes.c_uint32 * MAX_RANK)(*[int(x) for x in list(estrides)[:MAX_RANK]])
    return lib.oracle_validate(int(es), int(rank), int(base), d, s, b, e, *[int(x) for x in swizzle])


def swizzle(e: int, b: int, m: int, s: int) -> int:
    return int(_load().oracle_swizzle(int(e), int(b), int(m), int(s)))


def sweep_count(mp: Map) -> int:
    c = mp._c()
    return int(_load().oracle_sweep_count(ctypes.byref(c)))


def sweep_coords(mp: Map, t: int) -> list:
    c = mp._c()
    out = (ctypes.c_int32 * MAX_RANK)()
    _load().oracle_sweep_coords(ctypes.byref(c), int(t), out)
    return [out[d] for d in range(mp.rank)]


def box_bytes(mp: Map) -> int:
    c = mp._c()
    return int(_load().oracle_box_bytes(ctypes.byref(c)))


def _coords_arg(mp: Map, coords: Optional[np.ndarray], n: int):
    if coords is None:
        assert n == sweep_count(mp)
        return None
    coords = np.ascontiguousarray(coords, dtype=np.int32).reshape(n, mp.rank)
    return coords


def load_tiles(mp: Map, src: np.ndarray, coords: Optional[np.ndarray], n: int) -> np.ndarray:
    """Packed tile images (n * box_bytes bytes) of n boxes read from src (the
    tensor's bytes starting at its base)."""
    src = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    coords = _coords_arg(mp, coords, n)
    out = np.empty(n * box_bytes(mp), dtype=np.uint8)
    c = mp._c()
    rc = _load().oracle_load_tiles(ctypes.byref(c), _ptr(src, ctypes.c_uint8), src.size,
                                   _ptr(coords, ctypes.c_int32), n, _ptr(out, ctypes.c_uint8))
    if rc:
        raise ValueError("map reaches outside the source buffer")
    return out


def store_tiles(mp: Map, dst: np.ndarray, coords: Optional[np.ndarray], n: int, packed: np.ndarray) -> None:
    """Clipped store of n tile images into dst (modified in place)."""
    assert dst.dtype == np.uint8 and dst.flags["C_CONTIGUOUS"]
    packed = np.ascontiguousarray(packed).view(np.uint8).reshape(-1)
    assert packed.size >= n * box_bytes(mp)
    coords = _coords_arg(mp, coords, n)
    c = mp._c()
    rc = _load().oracle_store_tiles(ctypes.byref(c), _ptr(dst, ctypes.c_uint8), dst.size,
                                    _ptr(coords, ctypes.c_int32), n, _ptr(packed, ctypes.c_uint8))
    if rc:
        raise ValueError("map reaches outside the destination buffer")


def roundtrip(smap: Map, src: np.ndarray, dmap: Map, dst: np.ndarray,
              coords: Optional[np.ndarray], n: int) -> None:
    """Load each box from src and store it through dmap into dst (in place)."""
    src = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    assert dst.dtype == np.uint8 and dst.flags["C_CONTIGUOUS"]
    coords = _coords_arg(smap, coords, n)
    scratch = np.empty(box_bytes(smap), dtype=np.uint8)
    a, b = smap._c(), dmap._c()
    rc = _load().oracle_roundtrip(ctypes.byref(a), _ptr(src, ctypes.c_uint8), src.size,
                                  ctypes.byref(b), _ptr(dst, ctypes.c_uint8), dst.size,
                                  _ptr(coords, ctypes.c_int32), n, _ptr(scratch, ctypes.c_uint8))
    if rc:
        raise ValueError("map reaches outside a buffer")


def inb_elems(mp: Map, coords: Optional[np.ndarray], n: int) -> int:
    coords = _coords_arg(mp, coords, n)
    c = mp._c()
    return int(_load().oracle_inb_elems(ctypes.byref(c), _ptr(coords, ctypes.c_int32), n))


def roundtrip_add_f32(smap: Map, src: np.ndarray, dmap: Map, dst: np.ndarray,
                      coords: Optional[np.ndarray], n: int, addend: float) -> None:
    """Load each box, add `addend` (fp32) to every element of the tile, store
    it through dmap into dst (in place)."""
    src = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    assert dst.dtype == np.uint8 and dst.flags["C_CONTIGUOUS"]
    coords = _coords_arg(smap, coords, n)
    scratch = np.empty(box_bytes(smap), dtype=np.uint8)
    a, b = smap._c(), dmap._c()
    rc = _load().oracle_roundtrip_add_f32(ctypes.byref(a), _ptr(src, ctypes.c_uint8), src.size,
                                          ctypes.byref(b), _ptr(dst, ctypes.c_uint8), dst.size,
                                          _ptr(coords, ctypes.c_int32), n, float(addend),
                                          _ptr(scratch, ctypes.c_uint8))
    if rc:
        raise ValueError("maps need 4-byte elements and must stay inside their buffers")


def bulk_copy(dst: np.ndarray, src: np.ndarray, nbytes: int) -> None:
    """Copy nbytes from src to dst (uint8 arrays, dst modified in place)."""
    src = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    assert dst.dtype == np.uint8 and dst.flags["C_CONTIGUOUS"] and src.size >= nbytes and dst.size >= nbytes
    _load().oracle_bulk_copy(_ptr(dst, ctypes.c_uint8), _ptr(src, ctypes.c_uint8), int(nbytes))
