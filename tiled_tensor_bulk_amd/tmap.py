"""Python binding of libtmap (ctypes).  Argument marshalling only: every step
of the copy runs in the HIP library; torch supplies device memory and
streams.  Raises if libtmap.so has not been built -- there is no fallback.

Names match the C ABI in include/tmap.h.  Device pointers may be given as
ints or as torch tensors (their data_ptr()); streams as ints, torch streams
or None (torch's current stream when a GPU is present, else the default).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtmap.so")

SUCCESS, INVALID_VALUE, UNSUPPORTED_DEVICE, LAUNCH, TIMEOUT = 0, 1, 2, 3, 4
FLAG_CONTIGUOUS = 0x1
FLAG_NONTEMPORAL = 0x2
FLAG_THREAD_COPY = 0x4
FLAG_PRODUCER_WAVE = 0x8
FLAG_WAVE_PER_BOX = 0x40
FLAG_CACHED_PACKED = 0x80
FLAG_WHOLE_BOX = 0x10
FLAG_BAND = 0x20
FLAG_INJECT_BUDGET_MISMATCH = 0x100
FLAG_DEBUG_POISON = 0x200

DTYPES = {"u8": 0, "i8": 1, "u16": 2, "f16": 3, "bf16": 4, "u32": 5, "i32": 6, "f32": 7,
          "u64": 8, "f64": 9}


class TmapError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {detail}")


class tmap_t(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint64 * 16)]


class tmap_swizzle(ctypes.Structure):
    _fields_ = [("b", ctypes.c_uint8), ("m", ctypes.c_uint8), ("s", ctypes.c_uint8)]


class tmap_launch_opts(ctypes.Structure):
    _fields_ = [("stages", ctypes.c_uint32), ("grid_wgs", ctypes.c_uint32),
                ("flags", ctypes.c_uint32), ("spin_limit", ctypes.c_uint32),
                ("group", ctypes.c_uint32), ("regions", ctypes.c_uint32),
                ("band_rows", ctypes.c_uint32)]


class tmap_plan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_uint32), ("band_boxes", ctypes.c_uint32), ("band_rows", ctypes.c_uint32),
                ("stages", ctypes.c_uint32), ("slots", ctypes.c_uint32), ("group", ctypes.c_uint32),
                ("walkers", ctypes.c_uint32), ("workgroups", ctypes.c_uint32), ("regions", ctypes.c_uint32),
                ("lds_bytes", ctypes.c_uint32), ("units", ctypes.c_int64)]


DIRECTIONS = {"load": 0, "store": 1, "roundtrip": 2}
VARIANTS = {0: "ring", 1: "thread_copy", 2: "producer_wave", 3: "wave_per_box", 4: "band", 5: "corner", 6: "corner4"}


class tmap_info(ctypes.Structure):
    _fields_ = [("global_address", ctypes.c_uint64), ("dims", ctypes.c_uint64 * 5),
                ("strides", ctypes.c_uint64 * 5), ("box", ctypes.c_uint32 * 5),
                ("rank", ctypes.c_uint32), ("elem_size", ctypes.c_uint32), ("dtype", ctypes.c_uint32),
                ("swizzle", tmap_swizzle)]


_lib = None


def lib():
    """Load libtmap.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run: python -m tiled_tensor_bulk_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
        L.tmap_encode.argtypes = [P(tmap_t), ctypes.c_int, u32, vp, P(ctypes.c_uint64), P(ctypes.c_uint64),
                                  P(ctypes.c_uint32), P(ctypes.c_uint32), tmap_swizzle]
        L.tmap_encode.restype = ctypes.c_int
        for name in ("tmap_load_tiles", "tmap_store_tiles"):
            f = getattr(L, name)
            f.argtypes = [P(tmap_t), vp, i64, vp, P(tmap_launch_opts), vp]
            f.restype = ctypes.c_int
        L.tmap_roundtrip.argtypes = [P(tmap_t), P(tmap_t), vp, i64, P(tmap_launch_opts), vp]
        L.tmap_roundtrip.restype = ctypes.c_int
        L.tmap_roundtrip_noalloc.argtypes = [P(tmap_t), P(tmap_t), vp, i64, P(tmap_launch_opts), vp]
        L.tmap_roundtrip_noalloc.restype = ctypes.c_int
        L.tmap_roundtrip_add_f32.argtypes = [P(tmap_t), P(tmap_t), vp, i64, ctypes.c_float,
                                             P(tmap_launch_opts), vp]
        L.tmap_roundtrip_add_f32.restype = ctypes.c_int
        L.tmap_bulk_copy.argtypes = [vp, vp, ctypes.c_uint64, P(tmap_launch_opts), vp]
        L.tmap_bulk_copy.restype = ctypes.c_int
        L.tmap_box_bytes.argtypes = [P(tmap_t)]
        L.tmap_box_bytes.restype = ctypes.c_uint64
        L.tmap_sweep_tiles.argtypes = [P(tmap_t)]
        L.tmap_sweep_tiles.restype = ctypes.c_int64
        L.tmap_band_boxes.argtypes = [P(tmap_t), P(tmap_t), vp, P(tmap_launch_opts)]
        L.tmap_band_boxes.restype = u32
        L.tmap_inbounds_elems.argtypes = [P(tmap_t), vp, i64, P(ctypes.c_uint64)]
        L.tmap_inbounds_elems.restype = ctypes.c_int
        L.tmap_plan_launch.argtypes = [ctypes.c_int, P(tmap_t), P(tmap_t), vp, i64, P(tmap_launch_opts),
                                       P(tmap_plan)]
        L.tmap_plan_launch.restype = ctypes.c_int
        L.tmap_query.argtypes = [P(tmap_t), P(tmap_info)]
        L.tmap_query.restype = ctypes.c_int
        L.tmap_status_string.argtypes = [ctypes.c_int]
        L.tmap_status_string.restype = ctypes.c_char_p
        L.tmap_last_error_detail.argtypes = []
        L.tmap_last_error_detail.restype = ctypes.c_char_p
        L.tmap_sync_status.argtypes = [vp]
        L.tmap_sync_status.restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(st: int) -> str:
    try:
        return lib().tmap_status_string(st).decode()
    except Exception:
        return str(st)


def _check(st: int, where: str) -> None:
    if st != SUCCESS:
        raise TmapError(st, where, lib().tmap_last_error_detail().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> Optional[int]:
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except Exception:
            pass
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _is_tensor(x) -> bool:
    return hasattr(x, "data_ptr") and hasattr(x, "numel") and hasattr(x, "element_size")


def _check_buffer(x, need: int, what: str) -> None:
    """When x is a tensor (not a raw pointer), check that the kernels can
    touch `need` bytes of it: a device buffer too small would be written or
    read past its end on the GPU."""
    if not _is_tensor(x):
        return
    if not x.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    have = x.numel() * x.element_size()
    if have < need:
        raise ValueError(f"{what} holds {have} bytes, the copy needs {need}")


def _check_corners(coords, m: tmap_t, n_tiles: int) -> None:
    if coords is None or not _is_tensor(coords):
        return
    import torch
    if coords.dtype != torch.int32:
        raise ValueError("coords must be int32")
    _check_buffer(coords, 4 * int(n_tiles) * tmap_query(m)["rank"], "coords")


def _opts(stages=0, grid_wgs=0, flags=0, spin_limit=0, group=0, regions=0, band_rows=0):
    if not (stages or grid_wgs or flags or spin_limit or group or regions or band_rows):
        return None
    return ctypes.byref(tmap_launch_opts(stages, grid_wgs, flags, spin_limit, group, regions, band_rows))


# ------------------------------------------------------------------- C ABI names
def tmap_encode(dtype, rank: int, global_address, global_dim: Sequence[int],
                global_strides: Sequence[int], box_dim: Sequence[int],
                element_strides: Optional[Sequence[int]] = None, swizzle=(0, 0, 0)) -> tmap_t:
    """Validate and pack a tensor map; raises TmapError(INVALID_VALUE) on a rule violation."""
    m = tmap_t()
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    dims = (ctypes.c_uint64 * max(1, len(global_dim)))(*[int(v) for v in global_dim])
    strides = (ctypes.c_uint64 * max(1, len(global_strides)))(*[int(v) for v in global_strides])
    box = (ctypes.c_uint32 * max(1, len(box_dim)))(*[int(v) for v in box_dim])
    es = None if element_strides is None else (ctypes.c_uint32 * len(element_strides))(
        *[int(v) for v in element_strides])
    st = lib().tmap_encode(ctypes.byref(m), dt, int(rank), _ptr(global_address), dims, strides, box, es,
                           tmap_swizzle(*[int(v) for v in swizzle]))
    _check(st, "tmap_encode")
    return m


def tmap_load_tiles(src: tmap_t, coords, n_tiles: int, packed_out, stream=None, **opts) -> None:
    _check_corners(coords, src, n_tiles)
    _check_buffer(packed_out, int(n_tiles) * tmap_box_bytes(src), "packed_out")
    st = lib().tmap_load_tiles(ctypes.byref(src), _ptr(coords), int(n_tiles), _ptr(packed_out),
                               _opts(**opts), _stream(stream))
    _check(st, "tmap_load_tiles")


def tmap_store_tiles(dst: tmap_t, coords, n_tiles: int, packed_in, stream=None, **opts) -> None:
    _check_corners(coords, dst, n_tiles)
    _check_buffer(packed_in, int(n_tiles) * tmap_box_bytes(dst), "packed_in")
    st = lib().tmap_store_tiles(ctypes.byref(dst), _ptr(coords), int(n_tiles), _ptr(packed_in),
                                _opts(**opts), _stream(stream))
    _check(st, "tmap_store_tiles")


def tmap_roundtrip(src: tmap_t, dst: tmap_t, coords, n_tiles: int, stream=None, **opts) -> None:
    _check_corners(coords, src, n_tiles)
    st = lib().tmap_roundtrip(ctypes.byref(src), ctypes.byref(dst), _ptr(coords), int(n_tiles),
                              _opts(**opts), _stream(stream))
    _check(st, "tmap_roundtrip")


def tmap_roundtrip_noalloc(src: tmap_t, dst: tmap_t, coords, n_tiles: int, stream=None, **opts) -> None:
    """tmap_roundtrip without any device allocation (its status word is a
    static device array of the library)."""
    _check_corners(coords, src, n_tiles)
    st = lib().tmap_roundtrip_noalloc(ctypes.byref(src), ctypes.byref(dst), _ptr(coords), int(n_tiles),
                                      _opts(**opts), _stream(stream))
    _check(st, "tmap_roundtrip_noalloc")


def tmap_roundtrip_add_f32(src: tmap_t, dst: tmap_t, coords, n_tiles: int, addend: float, stream=None,
                           **opts) -> None:
    _check_corners(coords, src, n_tiles)
    st = lib().tmap_roundtrip_add_f32(ctypes.byref(src), ctypes.byref(dst), _ptr(coords), int(n_tiles),
                                      float(addend), _opts(**opts), _stream(stream))
    _check(st, "tmap_roundtrip_add_f32")


def tmap_bulk_copy(dst, src, nbytes: int, stream=None, **opts) -> None:
    _check_buffer(dst, int(nbytes), "dst")
    _check_buffer(src, int(nbytes), "src")
    st = lib().tmap_bulk_copy(_ptr(dst), _ptr(src), int(nbytes), _opts(**opts), _stream(stream))
    _check(st, "tmap_bulk_copy")


def tmap_box_bytes(m: tmap_t) -> int:
    return int(lib().tmap_box_bytes(ctypes.byref(m)))


def tmap_sweep_tiles(m: tmap_t) -> int:
    return int(lib().tmap_sweep_tiles(ctypes.byref(m)))


_ANY_CORNERS = ctypes.c_int32(0)  # a non-NULL corner pointer for the schedule query (never read)


def tmap_band_boxes(src: tmap_t, dst: Optional[tmap_t] = None, explicit_coords: bool = False,
                    flags: int = 0, band_rows: int = 0) -> int:
    """Boxes per stage on the band schedule a copy with these launch options
    would take, 0 for whole boxes (host only)."""
    corners = ctypes.addressof(_ANY_CORNERS) if explicit_coords else None
    return int(lib().tmap_band_boxes(ctypes.byref(src), None if dst is None else ctypes.byref(dst),
                                     corners, _opts(flags=int(flags), band_rows=int(band_rows))))


def tmap_plan_launch(direction, swept: tmap_t, dst: Optional[tmap_t] = None, explicit_coords: bool = False,
                     n_tiles: Optional[int] = None, **opts) -> dict:
    """The schedule a copy would run with (needs a gfx950 device; launches
    nothing).  direction: "load", "store" or "roundtrip"; n_tiles defaults
    to the full sweep."""
    d = DIRECTIONS[direction] if isinstance(direction, str) else int(direction)
    corners = ctypes.addressof(_ANY_CORNERS) if explicit_coords else None
    n = tmap_sweep_tiles(swept) if n_tiles is None else int(n_tiles)
    out = tmap_plan()
    st = lib().tmap_plan_launch(d, ctypes.byref(swept), None if dst is None else ctypes.byref(dst), corners, n,
                                _opts(**opts), ctypes.byref(out))
    _check(st, "tmap_plan_launch")
    r = {f: getattr(out, f) for f, _ in tmap_plan._fields_}
    r["variant"] = VARIANTS.get(out.variant, str(out.variant))
    return r


def tmap_inbounds_elems(m: tmap_t, host_coords, n_tiles: int) -> int:
    """host_coords: None (sweep) or a C-contiguous int32 numpy array [n][rank]."""
    out = ctypes.c_uint64()
    ptr = None if host_coords is None else host_coords.ctypes.data
    st = lib().tmap_inbounds_elems(ctypes.byref(m), ptr, int(n_tiles), ctypes.byref(out))
    _check(st, "tmap_inbounds_elems")
    return int(out.value)


def tmap_query(m: tmap_t) -> dict:
    info = tmap_info()
    _check(lib().tmap_query(ctypes.byref(m), ctypes.byref(info)), "tmap_query")
    r = info.rank
    return dict(global_address=info.global_address, rank=r, elem_size=info.elem_size, dtype=info.dtype,
                dims=list(info.dims[:r]), strides=list(info.strides[:r]), box=list(info.box[:r]),
                swizzle=(info.swizzle.b, info.swizzle.m, info.swizzle.s))


def tmap_status_string(st: int) -> str:
    return lib().tmap_status_string(int(st)).decode()


def tmap_last_error_detail() -> str:
    return lib().tmap_last_error_detail().decode()


def tmap_sync_status(stream=None) -> int:
    """Wait for the stream and return the status code (TIMEOUT if a readiness wait expired)."""
    return int(lib().tmap_sync_status(_stream(stream)))


# ------------------------------------------------------------------- convenience
_TORCH_DT = {"uint8": "u8", "int8": "i8", "uint16": "u16", "float16": "f16", "bfloat16": "bf16",
             "uint32": "u32", "int32": "i32", "float32": "f32", "uint64": "u64", "int64": "u64",
             "float64": "f64", "int16": "u16"}


def encode(t, box: Sequence[int], swizzle=(0, 0, 0), dims: Optional[Sequence[int]] = None) -> tmap_t:
    """Encode a map over torch tensor t: dims from reversed t.shape (innermost
    first), strides from reversed t.stride() times the element size.  The
    innermost stride must be 1.  `box` is innermost first."""
    shape = list(reversed(t.shape)) if dims is None else list(dims)
    es = t.element_size()
    st = list(reversed(t.stride()))
    if st and st[0] != 1:
        raise ValueError("innermost stride must be 1")
    name = str(t.dtype).replace("torch.", "")
    return tmap_encode(_TORCH_DT[name], len(shape), t.data_ptr(), shape, [s * es for s in st[1:]], box,
                       None, swizzle)
