"""GPU parity: the HIP path through the C ABI against the CPU oracle, byte for
byte, on seeded inputs.

* The five workloads at their full sizes, in the launch configuration the
  benchmark uses; the oracle recomputes every tile where it finishes in
  seconds (tile64, strips, pad5d) and a sample of tiles otherwise (ragged
  bf16, 2 GiB bytes), where closed forms cover the rest (a store of the loaded
  images restores every byte; an exact-tiling round trip is the identity).
* Seeded random maps of every rank, element size and swizzle (including
  swizzles that move data inside 16-byte chunks), random corners inside,
  across and outside the tensor, every ring depth and grid shape.
* Edge cases: zero tiles, one tile, fully out-of-bounds boxes, the largest box
  (64 KiB), box extents of 256, rank 1, and the budget-mismatch timeout.
"""
import os
import sys

import numpy as np
import pytest

import oracle
from oracle import Map
from tests import npref
from tiled_tensor_bulk_amd import inputs
from tiled_tensor_bulk_amd import tmap as T

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(nbytes, fill_seed=None):
    t = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    if fill_seed is not None:
        g = torch.Generator(device=DEV)
        g.manual_seed(fill_seed)
        n8 = (nbytes + 7) // 8
        x = torch.randint(-(2**63), 2**63 - 1, (n8,), dtype=torch.int64, generator=g, device=DEV)
        t.copy_(x.view(torch.uint8)[:nbytes])
    return t


def enc(dtype, t, dims, strides, box, swz=(0, 0, 0)):
    return T.tmap_encode(dtype, len(dims), t.data_ptr(), dims, strides, box, None, swz)


def dt_of(es):
    return {1: "u8", 2: "f16", 4: "f32", 8: "f64"}[es]


def check_ok(stream=None):
    st = T.tmap_sync_status(stream)
    assert st == T.SUCCESS, T.tmap_status_string(st)


def first_mismatch(a: np.ndarray, b: np.ndarray, bb: int, where=None):
    """None if equal, else the first differing byte (its tile and offset in
    packed images of bb bytes; `where(i)` may add what the byte holds)."""
    idx = np.flatnonzero(a != b)
    if idx.size == 0:
        return None
    i = int(idx[0])
    extra = f", {where(i)}" if where else ""
    return (f"byte {i} (tile {i // bb}, offset {i % bb}{extra}): got {a[i]:#x} want {b[i]:#x}; "
            f"{idx.size} bytes differ")


def packed_byte_source(es, box, swz, corners):
    """For the byte at offset i of packed load images: the box element whose
    bytes sit there (the swizzle is its own inverse), as a multi-index inside
    the box and as global coordinates (innermost first)."""
    n = int(np.prod(box))
    p = npref.perm(n, swz)

    def where(i):
        t, e = i // (n * es), int(p[(i % (n * es)) // es])
        idx = []
        for d in box:
            idx.append(e % d)
            e //= d
        g = [int(c) + k for c, k in zip(corners[t], idx)] if corners is not None else None
        return f"box element {tuple(idx)}" + (f", global {tuple(g)}" if g is not None else "")
    return where


def gpu_load(m, coords_np, n, **opts):
    bb = T.tmap_box_bytes(m)
    out = torch.empty(max(1, n * bb), dtype=torch.uint8, device=DEV)
    c = None if coords_np is None else torch.from_numpy(np.ascontiguousarray(coords_np, np.int32)).to(DEV)
    T.tmap_load_tiles(m, c, n, out, **opts)
    check_ok()
    return out[: n * bb]


# ----------------------------------------------------------------- workloads
def test_tile64_f32_roundtrip_load_store():
    w = inputs.WORKLOADS["tile64_f32"]
    say("tile64_f32: roundtrip, 1 stage, one box at (0,0)")
    src = inputs.device_bytes(w, DEV)
    dst = dev_tensor(w.alloc_bytes, fill_seed=101)
    dst0 = dst.cpu().numpy().copy()
    ms, md = enc("f32", src, w.dims, w.strides, w.box), enc("f32", dst, w.dims, w.strides, w.box)
    coords = torch.zeros((1, 2), dtype=torch.int32, device=DEV)
    T.tmap_roundtrip(ms, md, coords, 1, stages=1)
    check_ok()
    om = Map(es=4, dims=w.dims, strides=w.strides, box=w.box)
    want = dst0.copy()
    oracle.roundtrip(om, src.cpu().numpy(), om, want, np.zeros((1, 2), np.int32), 1)
    got = dst.cpu().numpy()
    assert (m := first_mismatch(got, want, 16384)) is None, m
    assert got.tobytes() == src.cpu().numpy().tobytes()       # exact tiling: identity
    packed = gpu_load(ms, np.zeros((1, 2), np.int32), 1, stages=1)
    assert packed.cpu().numpy().tobytes() == oracle.load_tiles(om, src.cpu().numpy(), np.zeros((1, 2), np.int32), 1).tobytes()
    dst2 = dev_tensor(w.alloc_bytes, fill_seed=102)
    T.tmap_store_tiles(enc("f32", dst2, w.dims, w.strides, w.box), coords, 1, packed, stages=1)
    check_ok()
    assert dst2.cpu().numpy().tobytes() == src.cpu().numpy().tobytes()


def test_strips_f16_load_page_schedule():
    """924 tiles; 132 workgroups, each walking the 7 column tiles of its strip."""
    w = inputs.WORKLOADS["strips_f16"]
    say("strips_f16: load sweep, 2 stages, 132 WGs x 7 tiles contiguous")
    src = inputs.device_bytes(w, DEV)
    m = enc("f16", src, w.dims, w.strides, w.box, w.swizzle)
    n = T.tmap_sweep_tiles(m)
    assert n == 924
    om = Map(es=2, dims=w.dims, strides=w.strides, box=w.box, swizzle=w.swizzle)
    want = oracle.load_tiles(om, src.cpu().numpy(), None, n)
    for opts in (dict(stages=2, grid_wgs=132, flags=T.FLAG_CONTIGUOUS | T.FLAG_WHOLE_BOX), dict(stages=2), dict()):
        got = gpu_load(m, None, n, **opts).cpu().numpy()
        assert (mm := first_mismatch(got, want, 32768)) is None, (opts, mm)


# Oracle results of the full-size workloads, computed once per session and
# shared by the tests that compare against them: host copies of the device
# inputs, the load images of the workload's corners, a store of those images
# into a sentinel-filled tensor and a round trip into another.  Each entry is
# written only by the oracle, from the very bytes the GPU used.
_EXPECT = {}
_SENTINEL_STORE, _SENTINEL_RT = 7, 8


def _corners(name, which):
    """The workload's corners: None for a sweep, the origin, or `which` =
    (count, seed) random ones."""
    w = inputs.WORKLOADS[name]
    if w.coords == "sweep":
        return None
    if w.coords == "origin":
        return np.zeros((1, w.rank), np.int32)
    return inputs.random_corners(w.dims, w.box, *which)


def expected(name, kind, which=(100_000, 40)):
    """Oracle result `kind` ("src", "load", "store", "roundtrip") of workload
    `name` over its corners (random ones: `which` = (count, seed))."""
    if kind == "src" or inputs.WORKLOADS[name].coords != "random":
        which = None                         # the same corners whatever `which` says
    key = (name, kind, which)
    if key in _EXPECT:
        return _EXPECT[key]
    w = inputs.WORKLOADS[name]
    om = Map(es=w.es, dims=w.dims, strides=w.strides, box=w.box, swizzle=w.swizzle)
    if kind == "src":
        # a host copy of the seeded device input (torch's Philox generator
        # gives the same bytes every time it is seeded alike)
        val = inputs.device_bytes(w, DEV).cpu().numpy()
        _EXPECT[key] = val
        return val
    host = expected(name, "src")
    corners = _corners(name, which)
    n = len(corners) if corners is not None else T.tmap_sweep_tiles(
        T.tmap_encode(w.dtype, w.rank, 0x7F0000000000, w.dims, w.strides, w.box, None, w.swizzle))
    say(f"oracle: {name} {kind} ({n} tiles)")
    if kind == "load":
        val = oracle.load_tiles(om, host, corners, n)
    elif kind == "store":
        val = inputs.sentinel_bytes(w.alloc_bytes, _SENTINEL_STORE)
        oracle.store_tiles(om, val, corners, n, expected(name, "load", which))
    else:
        val = inputs.sentinel_bytes(w.alloc_bytes, _SENTINEL_RT)
        oracle.roundtrip(om, host, om, val, corners, n)
    _EXPECT[key] = val
    return val


def forget(name):
    for k in [k for k in _EXPECT if k[0] == name]:
        del _EXPECT[k]


def host_sentinel(nbytes, seed):
    return torch.from_numpy(inputs.sentinel_bytes(nbytes, seed)).to(DEV)


def check_all_directions(name, opts, which=(100_000, 40), tag=""):
    """Load, store and round trip of workload `name` with launch options
    `opts`, every output byte compared with the oracle's."""
    w = inputs.WORKLOADS[name]
    src = inputs.device_bytes(w, DEV)
    # the oracle's inputs are a host copy of these very bytes (spot check)
    host = expected(name, "src")
    step = max(1, w.alloc_bytes // 1000003)
    assert np.array_equal(src[::step].cpu().numpy(), host[::step])
    m = enc(w.dtype, src, w.dims, w.strides, w.box, w.swizzle)
    cn = _corners(name, which)
    n = T.tmap_sweep_tiles(m) if cn is None else len(cn)
    bb = T.tmap_box_bytes(m)
    where = packed_byte_source(w.es, w.box, w.swizzle, cn if cn is not None else None)
    packed = gpu_load(m, cn, n, **opts)
    got = packed.cpu().numpy()
    assert (mm := first_mismatch(got, expected(name, "load", which), bb, where)) is None, (tag, "load", mm)
    del got
    c = None if cn is None else torch.from_numpy(cn).to(DEV)
    dst = host_sentinel(w.alloc_bytes, _SENTINEL_STORE)
    T.tmap_store_tiles(enc(w.dtype, dst, w.dims, w.strides, w.box, w.swizzle), c, n, packed, **opts)
    check_ok()
    del packed
    assert (mm := first_mismatch(dst.cpu().numpy(), expected(name, "store", which), 1 << 40)) is None, \
        (tag, "store", mm)
    del dst
    dst = host_sentinel(w.alloc_bytes, _SENTINEL_RT)
    T.tmap_roundtrip(m, enc(w.dtype, dst, w.dims, w.strides, w.box, w.swizzle), c, n, **opts)
    check_ok()
    assert (mm := first_mismatch(dst.cpu().numpy(), expected(name, "roundtrip", which), 1 << 40)) is None, \
        (tag, "roundtrip", mm)


@pytest.mark.parametrize("opts", [dict(flags=T.FLAG_NONTEMPORAL), dict(stages=4, flags=T.FLAG_NONTEMPORAL),
                                  dict(flags=T.FLAG_NONTEMPORAL | T.FLAG_WHOLE_BOX)],
                         ids=["benchmark_launch", "band_4_stages", "whole_box"])
def test_ragged_bf16_full_size(opts):
    """Every one of the 65,280 load images (the last tile row: 63 rows and a
    zero-filled one), the store of all of them and the round trip, against
    the oracle."""
    w = inputs.WORKLOADS["ragged_bf16"]
    say(f"ragged_bf16: load, store, round trip of 65280 tiles {opts}; full oracle")
    m = T.tmap_encode(w.dtype, w.rank, 0x7F0000000000, w.dims, w.strides, w.box, None, w.swizzle)
    assert T.tmap_sweep_tiles(m) == 65280
    check_all_directions("ragged_bf16", opts, tag=str(opts))


@pytest.mark.parametrize("opts", [dict(flags=T.FLAG_NONTEMPORAL), dict(stages=4, flags=T.FLAG_NONTEMPORAL),
                                  dict(stages=4, flags=T.FLAG_NONTEMPORAL | T.FLAG_WHOLE_BOX)],
                         ids=["benchmark_launch", "band_4_stages", "whole_box_4_stages"])
def test_sweep2g_u8_full_size(opts):
    """Every one of the 131,072 load images of the 2 GiB tensor, the store of
    all of them and the round trip, against the oracle; the round trip of an
    exact tiling is also the identity."""
    w = inputs.WORKLOADS["sweep2g_u8"]
    say(f"sweep2g_u8: load, store, round trip of 131072 tiles (2 GiB) {opts}; full oracle")
    m = T.tmap_encode(w.dtype, w.rank, 0x7F0000000000, w.dims, w.strides, w.box, None, w.swizzle)
    assert T.tmap_sweep_tiles(m) == 131072
    check_all_directions("sweep2g_u8", opts, tag=str(opts))
    assert np.array_equal(expected("sweep2g_u8", "roundtrip"), expected("sweep2g_u8", "src"))


def test_plus1_f32_full_size_in_the_benchmark_launch():
    """The fused +1.0f round trip of the 1 GiB fp32 matrix (64 x 64 boxes,
    128-byte swizzle) in the launch configuration the benchmark times (the
    tensor exceeds the last-level cache, so the tensor side carries
    non-temporal hints), every byte against the oracle's fp32 addition."""
    w = inputs.WORKLOADS["plus1_f32"]
    say("plus1_f32: fused +1.0f round trip of 65536 tiles (1 GiB); full oracle")
    src = inputs.device_bytes(w, DEV)
    ms = enc("f32", src, w.dims, w.strides, w.box, w.swizzle)
    n = T.tmap_sweep_tiles(ms)
    assert n == 65536
    dst = host_sentinel(w.alloc_bytes, _SENTINEL_RT)
    md = enc("f32", dst, w.dims, w.strides, w.box, w.swizzle)
    assert T.tmap_plan_launch("roundtrip", ms, md, False, n, flags=T.FLAG_NONTEMPORAL)["variant"] == "band"
    T.tmap_roundtrip_add_f32(ms, md, None, n, 1.0, flags=T.FLAG_NONTEMPORAL)
    check_ok()
    host = src.cpu().numpy()
    want = inputs.sentinel_bytes(w.alloc_bytes, _SENTINEL_RT)
    om = Map(es=4, dims=w.dims, strides=w.strides, box=w.box, swizzle=w.swizzle)
    oracle.roundtrip_add_f32(om, host, om, want, None, n, 1.0)
    got = dst.cpu().numpy()
    nan = np.isnan(want.view(np.float32))
    assert not nan.any()                               # normal(0,1) inputs: no NaN to compare loosely
    assert (mm := first_mismatch(got, want, 1 << 40)) is None, mm


@pytest.mark.parametrize("opts", [dict(), dict(stages=4), dict(stages=2, flags=T.FLAG_WHOLE_BOX)],
                         ids=["benchmark_launch", "shared_ring_4_stages", "shared_ring_2_stages"])
def test_pad5d_f32_random_corners_full(opts):
    say(f"pad5d_f32: load, store, round trip of 1e5 random corners {opts}; full oracle")
    check_all_directions("pad5d_f32", opts, tag=str(opts))


@pytest.mark.parametrize("opts", [dict(), dict(group=4), dict(regions=1), dict(stages=2)],
                         ids=["benchmark_launch", "corner4_group_4", "corner4_one_stream", "shared_ring_2_stages"])
def test_pad5d_sweep_f32_full(opts):
    """The padded 5-D tensor swept whole (19845 boxes, ragged in four
    dimensions): one stage on the 4-byte-lane corner kernel by default (one
    box to a wave, the waves dealt to the XCDs as 8 streams), 4 boxes to a
    wave, one stream, and the shared ring with two stages."""
    say(f"pad5d_sweep_f32: load, store, round trip of the whole sweep {opts}; full oracle")
    check_all_directions("pad5d_sweep_f32", opts, tag=str(opts))
    forget("pad5d_sweep_f32")


# ----------------------------------------------------------------- seeded fuzz
def _fuzz_case(rng, idx):
    mp = inputs.random_map(rng)
    es, dims, strides, box, swz = mp["es"], mp["dims"], mp["strides"], mp["box"], mp["swizzle"]
    if idx % 7 == 3 and es <= 4:
        # a swizzle that permutes elements inside 16-byte chunks
        n_el = int(np.prod(box))
        for mm in range(0, 4):
            if (1 << mm) * es < 16 and n_el % (1 << (mm + 1)) == 0:
                swz = (1, mm, 1 + int(rng.integers(0, 3)))
                break
    alloc = mp["alloc_bytes"]
    ncoords = int(rng.integers(1, 40))
    coords = inputs.random_corners(dims, box, ncoords, int(rng.integers(1 << 30)))
    opts = dict(stages=int(rng.integers(1, 5)), grid_wgs=int(rng.choice([0, 1, 2, 3, 7])),
                flags=int(rng.choice([0, T.FLAG_CONTIGUOUS, T.FLAG_NONTEMPORAL, T.FLAG_THREAD_COPY,
                                      T.FLAG_THREAD_COPY | T.FLAG_CONTIGUOUS, T.FLAG_PRODUCER_WAVE,
                                      T.FLAG_PRODUCER_WAVE | T.FLAG_CONTIGUOUS, T.FLAG_THREAD_COPY | T.FLAG_CACHED_PACKED,
                                      T.FLAG_PRODUCER_WAVE | T.FLAG_CACHED_PACKED | T.FLAG_NONTEMPORAL])),
                group=int(rng.choice([0, 1, 2, 4, 8, 64])),
                regions=int(rng.choice([0, 1, 2, 3, 8, 64])))
    return es, dims, strides, box, swz, alloc, coords, opts


def _wave_case(rng, idx):
    """A fuzz case for wave-per-box mode: boxes of at most 16 KiB, 1 or 2
    stages, the grid counting waves."""
    while True:
        case = _fuzz_case(rng, idx)
        if int(np.prod(case[3])) * case[0] <= 16384:
            break
    opts = case[7]
    opts["stages"] = int(rng.integers(1, 3))
    opts["flags"] = T.FLAG_WAVE_PER_BOX | int(rng.choice([0, T.FLAG_CONTIGUOUS, T.FLAG_NONTEMPORAL,
                                                        T.FLAG_CACHED_PACKED]))
    opts["grid_wgs"] = int(rng.choice([0, 0, 1, 2, 3, 5, 9]))
    return case


@pytest.mark.parametrize("chunk", range(6))
def test_fuzz_random_maps(chunk):
    """Seeded random maps of every rank, element size and swizzle, random
    corners in, across and outside the tensor, random launch options: load,
    round trip and store at those corners, and a store through the sweep;
    chunks 4 and 5 run wave-per-box mode."""
    rng = np.random.default_rng(9000 + chunk)
    for i in range(40):
        es, dims, strides, box, swz, alloc, coords, opts = (_fuzz_case if chunk < 4 else _wave_case)(rng, i)
        say(f"fuzz chunk {chunk} case {i}: es={es} dims={dims} strides={strides} box={box} swz={swz} "
            f"n={len(coords)} opts={opts}")
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        src = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        host = src.cpu().numpy()
        m = enc(dt_of(es), src, dims, strides, box, swz)
        bb = T.tmap_box_bytes(m)
        # load
        packed = gpu_load(m, coords, len(coords), **opts)
        want = oracle.load_tiles(om, host, coords, len(coords))
        got = packed.cpu().numpy()
        assert (mm := first_mismatch(got, want, bb, packed_byte_source(es, box, swz, coords))) is None, mm
        # round trip into a sentinel-filled tensor of another layout (same box, swizzle)
        dst = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        want_dst = dst.cpu().numpy().copy()
        c = torch.from_numpy(coords).to(DEV)
        T.tmap_roundtrip(m, enc(dt_of(es), dst, dims, strides, box, swz), c, len(coords), **opts)
        check_ok()
        oracle.roundtrip(om, host, om, want_dst, coords, len(coords))
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("roundtrip", mm)
        # store of the loaded images back through the same corners (boxes
        # that overlap write equal bytes: every image holds the source's)
        dst1 = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        want1 = dst1.cpu().numpy().copy()
        T.tmap_store_tiles(enc(dt_of(es), dst1, dims, strides, box, swz), c, len(coords), packed, **opts)
        check_ok()
        oracle.store_tiles(om, want1, coords, len(coords), want)
        assert (mm := first_mismatch(dst1.cpu().numpy(), want1, 1 << 40)) is None, ("store at corners", mm)
        # store of random images through a sweep (no two boxes overlap)
        ns = T.tmap_sweep_tiles(m)
        imgs = inputs.sentinel_bytes(ns * bb, int(rng.integers(1 << 30)))
        dst2 = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        want2 = dst2.cpu().numpy().copy()
        T.tmap_store_tiles(enc(dt_of(es), dst2, dims, strides, box, swz), None, ns,
                           torch.from_numpy(imgs).to(DEV), **opts)
        check_ok()
        oracle.store_tiles(om, want2, None, ns, imgs)
        assert (mm := first_mismatch(dst2.cpu().numpy(), want2, 1 << 40)) is None, ("store", mm)


@pytest.mark.parametrize("box_kib", [2, 8, 16])
def test_wave_per_box_workgroup_shapes(box_kib):
    """Wave-per-box mode runs four waves to a workgroup for boxes under 8 KiB
    and one wave to a workgroup from 8 KiB: loads, round trips and stores of
    scattered corners (in, across and outside the tensor) match the oracle
    for both shapes, 1 and 2 stages, and grids of waves that do and do not
    fill the last workgroup."""
    rng = np.random.default_rng(9300 + box_kib)
    es = 4
    box = {2: [16, 8, 4], 8: [32, 8, 8], 16: [64, 8, 8]}[box_kib]
    dims = [77, 29, 21]
    strides = [80 * es, 80 * es * 31]
    alloc = strides[1] * dims[2]
    swz = (2, 2, 3)
    om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
    src = dev_tensor(alloc, fill_seed=box_kib)
    host = src.cpu().numpy()
    m = enc("f32", src, dims, strides, box, swz)
    assert T.tmap_box_bytes(m) == box_kib * 1024
    coords = inputs.random_corners(dims, box, 301, seed=box_kib)
    want_load = oracle.load_tiles(om, host, coords, len(coords))
    c = torch.from_numpy(coords).to(DEV)
    for stages in (1, 2):
        p = T.tmap_plan_launch("load", m, None, True, len(coords), stages=stages, flags=T.FLAG_WAVE_PER_BOX)
        # one stage and boxes up to 8 KiB: the corner kernel in 4-byte lanes
        # (its rows of 64 and 128 bytes hold the swizzle's XOR)
        assert p["variant"] == ("corner4" if stages == 1 and box_kib <= 8 else "wave_per_box")
        assert p["workgroups"] == -(-p["walkers"] // (4 if box_kib < 8 else 1))
        for grid in (0, 1, 3, 6):
            say(f"wave workgroups: box {box_kib} KiB stages={stages} grid={grid}")
            opts = dict(stages=stages, grid_wgs=grid, flags=T.FLAG_WAVE_PER_BOX)
            got = gpu_load(m, coords, len(coords), **opts).cpu().numpy()
            assert (mm := first_mismatch(got, want_load, box_kib * 1024)) is None, ("load", stages, grid, mm)
            dst = dev_tensor(alloc, fill_seed=100 + grid)
            want_dst = dst.cpu().numpy().copy()
            T.tmap_roundtrip(m, enc("f32", dst, dims, strides, box, swz), c, len(coords), **opts)
            check_ok()
            oracle.roundtrip(om, host, om, want_dst, coords, len(coords))
            assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("roundtrip", mm)
            # the loaded images stored back: overlapping boxes carry equal bytes
            dst2 = dev_tensor(alloc, fill_seed=200 + grid)
            want2 = dst2.cpu().numpy().copy()
            T.tmap_store_tiles(enc("f32", dst2, dims, strides, box, swz), c, len(coords),
                               torch.from_numpy(want_load).to(DEV), **opts)
            check_ok()
            oracle.store_tiles(om, want2, coords, len(coords), want_load)
            assert (mm := first_mismatch(dst2.cpu().numpy(), want2, 1 << 40)) is None, ("store", mm)


@pytest.mark.parametrize("chunk", range(2))
def test_poisoned_stages_still_match(chunk):
    """With every stage filled with 0xDEADBEEF before its loads are issued, a
    read that the byte count let through too early would copy the pattern
    out; loads and round trips must still match the oracle byte for byte
    (shared ring, wave per box, producer wave, band schedule)."""
    rng = np.random.default_rng(9100 + chunk)
    for i in range(16):
        es, dims, strides, box, swz, alloc, coords, opts = (_fuzz_case if i % 2 else _wave_case)(rng, i)
        if opts["flags"] & T.FLAG_THREAD_COPY:
            opts["flags"] &= ~T.FLAG_THREAD_COPY
        opts["flags"] |= T.FLAG_DEBUG_POISON
        say(f"poison {chunk}/{i}: es={es} dims={dims} box={box} swz={swz} n={len(coords)} opts={opts}")
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        src = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        host = src.cpu().numpy()
        m = enc(dt_of(es), src, dims, strides, box, swz)
        got = gpu_load(m, coords, len(coords), **opts).cpu().numpy()
        want = oracle.load_tiles(om, host, coords, len(coords))
        assert (mm := first_mismatch(got, want, T.tmap_box_bytes(m))) is None, mm
        dst = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        want_dst = dst.cpu().numpy().copy()
        T.tmap_roundtrip(m, enc(dt_of(es), dst, dims, strides, box, swz), torch.from_numpy(coords).to(DEV),
                         len(coords), **opts)
        check_ok()
        oracle.roundtrip(om, host, om, want_dst, coords, len(coords))
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("roundtrip", mm)
    # a band-schedule sweep at full size: 2 GiB round trip, 3-stage ring of 16 KiB units
    w = inputs.WORKLOADS["sweep2g_u8"]
    if chunk == 0:
        say("poison: sweep2g_u8 round trip")
        src = inputs.device_bytes(w, DEV)
        dst = dev_tensor(w.alloc_bytes)
        dst.fill_(0)
        ms = enc("u8", src, w.dims, w.strides, w.box, w.swizzle)
        T.tmap_roundtrip(ms, enc("u8", dst, w.dims, w.strides, w.box, w.swizzle), None, T.tmap_sweep_tiles(ms),
                         flags=T.FLAG_NONTEMPORAL | T.FLAG_DEBUG_POISON)
        check_ok()
        assert torch.equal(dst, src)


@pytest.mark.parametrize("mode", [dict(), dict(flags=T.FLAG_WHOLE_BOX), dict(flags=T.FLAG_THREAD_COPY)],
                         ids=["default", "shared_ring", "thread_copy"])
def test_position_coded_elements_name_their_source(mode):
    """Every in-bounds element of a padded rank-5 fp32 tensor holds its own
    linear index + 1 and every padding word 0xFFFFFFFF, so a misplaced byte
    names where it came from.  Loads at 3000 random corners must put exactly
    index + 1 (or 0 outside the tensor) at each element's swizzled position,
    computed here in closed form without the oracle; storing those images
    into a fresh tensor must restore exactly the union of the boxes'
    footprints and leave every other word, padding included, untouched."""
    say(f"position-coded corners {mode}")
    dims, box, swz = [37, 11, 5, 3, 2], [8, 4, 2, 2, 1], (1, 2, 3)
    strides = [160, 160 * 11 + 32]
    strides += [strides[-1] * 5 + 16]
    strides += [strides[-1] * 3]
    words = strides[-1] * dims[-1] // 4
    grid = np.meshgrid(*[np.arange(n) for n in reversed(dims)], indexing="ij")   # outermost first
    g = [grid[len(dims) - 1 - d].reshape(-1) for d in range(len(dims))]           # innermost first
    word = sum(g[d] * (strides[d - 1] // 4 if d else 1) for d in range(len(dims)))
    lin = sum(g[d] * int(np.prod(dims[:d])) for d in range(len(dims)))
    host = np.full(words, 0xFFFFFFFF, np.uint32)
    host[word] = (lin + 1).astype(np.uint32)
    src = torch.from_numpy(host.view(np.uint8)).to(DEV)
    m = enc("f32", src, dims, strides, box, swz)
    corners = inputs.random_corners(dims, box, 3000, seed=61)
    n = len(corners)
    got = gpu_load(m, corners, n, **mode).cpu().numpy().view(np.uint32).reshape(n, -1)
    # closed form: box element e at image position perm(e)
    N = int(np.prod(box))
    e = np.arange(N)
    idx = []
    for d in range(len(box)):
        idx.append(e % box[d])
        e = e // box[d]
    gi = corners[:, None, :].astype(np.int64) + np.stack(idx, axis=1)[None, :, :]
    inb = np.all((gi >= 0) & (gi < np.array(dims)), axis=2)
    lin_box = sum(gi[:, :, d] * int(np.prod(dims[:d])) for d in range(len(dims)))
    want = np.zeros((n, N), np.uint32)
    want[:, npref.perm(N, swz)] = np.where(inb, lin_box + 1, 0).astype(np.uint32)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    # store them back into a fresh tensor
    dst = torch.full((words,), -1, dtype=torch.int32, device=DEV).view(torch.uint8)
    md = enc("f32", dst, dims, strides, box, swz)
    T.tmap_store_tiles(md, torch.from_numpy(corners).to(DEV), n, torch.from_numpy(want.view(np.uint8).reshape(-1)).to(DEV),
                       **mode)
    check_ok()
    out = dst.cpu().numpy().view(np.uint32)
    covered = np.zeros(words, bool)
    wbox = sum(np.where(inb, gi[:, :, d], 0) * (strides[d - 1] // 4 if d else 1) for d in range(len(dims)))
    covered[wbox[inb]] = True
    expect = np.where(covered, host, np.uint32(0xFFFFFFFF))
    assert np.array_equal(out, expect), np.argwhere(out != expect)[:5]
    assert covered.sum() < len(word)              # some in-bounds elements stay unwritten


# ----------------------------------------------------------------- edge cases
def test_sweep_equals_explicit_coords():
    say("sweep vs explicit corners")
    dims, strides, box, swz = [200, 37, 3], [416, 416 * 37], [32, 8, 2], (2, 3, 2)
    src = dev_tensor(416 * 37 * 3, fill_seed=5)
    m = enc("u16", src, dims, strides, box, swz)
    om = Map(es=2, dims=dims, strides=strides, box=box, swizzle=swz)
    n = T.tmap_sweep_tiles(m)
    corners = np.array([oracle.sweep_coords(om, t) for t in range(n)], np.int32)
    a = gpu_load(m, None, n).cpu().numpy()
    b = gpu_load(m, corners, n).cpu().numpy()
    assert a.tobytes() == b.tobytes() == oracle.load_tiles(om, src.cpu().numpy(), None, n).tobytes()


def test_largest_box_and_wide_rows():
    say("64 KiB box (16 slots per lane, 2 stages) and 256-wide boxes")
    cases = [(1, [256, 256], [256], [256, 256], (3, 4, 3)),        # 64 KiB u8 box
             (4, [300, 70], [1216], [256, 16], (0, 0, 0)),          # 16 KiB, 256 wide, ragged
             (8, [100, 9], [800], [64, 16], (2, 1, 3))]             # fp64, 8 KiB
    for es, dims, strides, box, swz in cases:
        alloc = dims[-1] * strides[-1]
        src = dev_tensor(alloc, fill_seed=17)
        m = enc(dt_of(es), src, dims, strides, box, swz)
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        coords = inputs.random_corners(dims, box, 50, 8)
        for st in ([1, 2] if T.tmap_box_bytes(m) > 32768 else [1, 2, 3, 4]):
            got = gpu_load(m, coords, len(coords), stages=st).cpu().numpy()
            want = oracle.load_tiles(om, src.cpu().numpy(), coords, len(coords))
            assert (mm := first_mismatch(got, want, T.tmap_box_bytes(m))) is None, (es, box, st, mm)


def test_rank1_and_fully_out_of_bounds():
    say("rank 1, boxes wholly outside the tensor")
    src = dev_tensor(4096, fill_seed=3)
    m = enc("u8", src, [4000], [], [256])
    om = Map(es=1, dims=[4000], strides=[], box=[256])
    coords = np.array([[-256], [4000], [3900], [-100], [0], [1 << 30], [-(1 << 31)]], np.int32)
    got = gpu_load(m, coords, len(coords)).cpu().numpy()
    want = oracle.load_tiles(om, src.cpu().numpy(), coords, len(coords))
    assert got.tobytes() == want.tobytes()
    assert not got[:256].any() and not got[256:512].any()


def test_largest_coordinates():
    """A dimension of 2^31 elements (the largest a map accepts): boxes ending
    exactly at the last element, reaching past it, wholly past it and at the
    most negative corner, in both directions of the copy."""
    say("2^31-element dimension: corners at the int32 limits")
    big = 1 << 31
    src = dev_tensor(big, fill_seed=77)
    m = enc("u8", src, [big, 1], [big], [128, 1])
    corners = np.array([[big - 128, 0], [big - 64, 0], [big - 1, 0], [2**31 - 1, 0], [-(2**31), 0],
                        [-100, 0], [0, 0], [big // 2 + 17, 0], [big - 128, -1], [big - 128, 1]], np.int32)
    n = len(corners)
    got = gpu_load(m, corners, n).cpu().numpy()
    om = Map(es=1, dims=[big, 1], strides=[big], box=[128, 1])
    host = src.cpu().numpy()
    want = oracle.load_tiles(om, host, corners, n)
    assert (mm := first_mismatch(got, want, 128)) is None, mm
    # store the images back over a zeroed copy: exactly the in-bounds bytes return
    dst = torch.zeros_like(src)
    T.tmap_store_tiles(enc("u8", dst, [big, 1], [big], [128, 1]), torch.from_numpy(corners).to(DEV), n,
                       torch.from_numpy(got).to(DEV))
    check_ok()
    want_dst = np.zeros(big, np.uint8)
    oracle.store_tiles(om, want_dst, corners, n, want)
    del host
    d = dst.cpu().numpy()
    assert (mm := first_mismatch(d, want_dst, 1 << 40)) is None, mm


def test_corner_offsets_far_and_wrapped():
    """The corner kernel sums corner offsets in 32 bits when both maps lie
    within 2 GiB of their bases, else in 64.  In the 32-bit case, corners
    far outside the tensor wrap to meaningless offsets whose boxes must
    still read as zeros and write nothing; in the 64-bit case, boxes more
    than 2 GiB from the base must land where they belong.  Load, store and
    round trip of 8 KiB boxes (rank 5) against the oracle, unswizzled (the
    4-byte lanes), with a swizzle inside the rows (the 4-byte lanes) and
    with one whose XOR reaches past them (the 16-byte lanes)."""
    big = 1 << 31
    i32 = np.iinfo(np.int32)
    for case, swz in (("wrapped", (0, 0, 0)), ("wrapped", (3, 2, 3)), ("wrapped", (3, 3, 3)),
                      ("far", (0, 0, 0)), ("far", (3, 4, 3)), ("far", (3, 5, 3))):
        if case == "wrapped":
            # the padded 5-D fp32 tensor (103 MB): corners whose offsets overflow 32 bits
            w = inputs.WORKLOADS["pad5d_f32"]
            es, dims, strides, box, dtype, alloc = 4, list(w.dims), list(w.strides), list(w.box), "f32", w.alloc_bytes
            extreme = [[0, i32.max, 0, 0, 0], [5, 0, i32.min, 0, 0], [i32.min, i32.min, 3, 1, 0],
                       [100, 60, 30, i32.max, 6], [7, 9, 11, 5, i32.min], [i32.max] * 5, [i32.min] * 5,
                       [-31, -7, -3, -1, 0], [128, 64, 32, 12, 6], [1 << 28, 0, 0, 0, 0], [0, 0, 0, 0, 1 << 29]]
            rand = inputs.random_corners(dims, box, 500, seed=4242)
        else:
            # a 2 GiB u8 tensor seen as 65536 x 256 x 128: boxes up to the last byte
            es, dims, strides, box, dtype, alloc = 1, [65536, 256, 128], [65536, 65536 * 256], [128, 64, 1], "u8", big
            extreme = [[65536 - 128, 256 - 64, 127], [65536 - 100, 200, 127], [0, 0, 127], [-64, -32, 127],
                       [65500, 250, 126], [i32.max, 0, 127], [0, 0, i32.max], [i32.min, 5, 64], [77, 3, 128]]
            rng = np.random.default_rng(4343)
            rand = np.stack([rng.integers(-128, 65536, 300), rng.integers(-64, 256, 300),
                             rng.integers(100, 129, 300)], axis=1)
        corners = np.ascontiguousarray(np.concatenate([np.array(extreme, np.int64), rand.astype(np.int64)]), np.int32)
        n = len(corners)
        c = torch.from_numpy(corners).to(DEV)
        src = dev_tensor(alloc, fill_seed=91)
        host = src.cpu().numpy()
        m = enc(dtype, src, dims, strides, box, swz)
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        past_row = swz in ((3, 3, 3), (3, 5, 3))
        assert T.tmap_plan_launch("load", m, None, True, n)["variant"] == ("corner" if past_row else "corner4")
        case = f"{case}, swizzle {swz}"
        say(f"corner kernel, {case} offsets: load")
        got = gpu_load(m, corners, n).cpu().numpy()
        want = oracle.load_tiles(om, host, corners, n)
        bb = T.tmap_box_bytes(m)
        assert (mm := first_mismatch(got, want, bb)) is None, (case, "load", mm)
        say(f"corner kernel, {case} offsets: store")
        dst = dev_tensor(alloc, fill_seed=92)
        want_dst = dst.cpu().numpy().copy()
        T.tmap_store_tiles(enc(dtype, dst, dims, strides, box, swz), c, n, torch.from_numpy(want).to(DEV))
        check_ok()
        oracle.store_tiles(om, want_dst, corners, n, want)
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, (case, "store", mm)
        say(f"corner kernel, {case} offsets: round trip")
        dst = dev_tensor(alloc, fill_seed=93)
        want_dst = dst.cpu().numpy().copy()
        T.tmap_roundtrip(m, enc(dtype, dst, dims, strides, box, swz), c, n)
        check_ok()
        oracle.roundtrip(om, host, om, want_dst, corners, n)
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, (case, "roundtrip", mm)
        del src, dst, host, want_dst
        torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,swz", [("bf16", (3, 3, 3)), ("u8", (3, 4, 3))], ids=["bf16_128B_swizzle", "u8_128B_swizzle"])
def test_scattered_narrow_swizzled_boxes_full(dtype, swz):
    """10^5 scattered 8 KiB boxes of 2- and 1-byte elements with the 128-byte
    swizzle, on a padded 5-D tensor of the scattered workload's shape (box
    rows of 128 bytes, row pitch the dims rounded up to 16 bytes): the 4-byte
    lanes' swizzled instances and their element-by-element pass for words the
    x edge cuts, at full size.  Every packed image, the store of all of them
    through the same corners and the round trip, against the oracle."""
    es = 1 if dtype == "u8" else 2
    dims = [129, 65, 33, 13, 7]
    box = [128 // es, 8, 4, 2, 1]
    pitch = -(-129 * es // 16) * 16
    strides = [pitch, pitch * 65, pitch * 65 * 33, pitch * 65 * 33 * 13]
    alloc = strides[-1] * 7
    say(f"scattered {dtype} boxes, swizzle {swz}: load, store, round trip of 1e5 corners; full oracle")
    src = dev_tensor(alloc, fill_seed=77 + es)
    host = src.cpu().numpy()
    m = enc(dtype, src, dims, strides, box, swz)
    om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
    corners = inputs.random_corners(dims, box, 100_000, seed=50 + es)
    n = len(corners)
    assert T.tmap_plan_launch("load", m, None, True, n)["variant"] == "corner4"
    packed = gpu_load(m, corners, n)
    want = oracle.load_tiles(om, host, corners, n)
    assert (mm := first_mismatch(packed.cpu().numpy(), want, 8192)) is None, ("load", mm)
    c = torch.from_numpy(corners).to(DEV)
    dst = dev_tensor(alloc, fill_seed=90 + es)
    want_dst = dst.cpu().numpy().copy()
    T.tmap_store_tiles(enc(dtype, dst, dims, strides, box, swz), c, n, packed)
    check_ok()
    oracle.store_tiles(om, want_dst, corners, n, want)
    assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("store", mm)
    del packed, want
    dst = dev_tensor(alloc, fill_seed=95 + es)
    want_dst = dst.cpu().numpy().copy()
    T.tmap_roundtrip(m, enc(dtype, dst, dims, strides, box, swz), c, n)
    check_ok()
    oracle.roundtrip(om, host, om, want_dst, corners, n)
    assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("roundtrip", mm)


def _corner4_case(rng):
    """A map the corner kernels run in 4-byte lanes: unswizzled elements of
    any size, box rows of a power of two from 16 to 256 bytes, at most 64
    rows and 8 KiB to a box, padded rows and planes; and a second layout of
    other dims and pitch with the same box."""
    es = int(rng.choice([1, 2, 4, 8]))
    rank = int(rng.integers(1, 6))
    row = int(rng.choice([16, 32, 64, 128, 256]))
    max_rows = min(64, 8192 // row)
    box, rows = [row // es], 1
    for _ in range(1, rank):
        b = int(rng.integers(1, max_rows // rows + 1))
        box.append(b)
        rows *= b

    def layout():
        dims = [int(rng.integers(1, 2 * box[0] + 40))] + [int(rng.integers(1, 2 * b + 4)) for b in box[1:]]
        s = (-(-dims[0] * es // 16) + int(rng.integers(0, 3))) * 16
        strides = []
        for d in range(1, rank):
            strides.append(s)
            s *= dims[d] + int(rng.integers(0, 2))
        return dims, strides, s
    # half the maps take a swizzle the 4-byte lanes handle: whole words
    # (target bit tb >= 2) moved within a row (tb + B <= log2(row))
    lg, lrow = es.bit_length() - 1, row.bit_length() - 1
    swz = (0, 0, 0)
    tb_min = 4 if rng.integers(0, 2) and lrow - max(lg, 4) >= 1 else 2   # whole chunks, or word granules
    b_max = min(4, lrow - max(lg, tb_min))     # m >= max(0, tb_min - lg) and m + lg + b <= lrow
    if rng.integers(0, 2) and b_max >= 1:
        b = int(rng.integers(1, b_max + 1))
        m = int(rng.integers(max(0, tb_min - lg), lrow - lg - b + 1))
        swz = (b, m, int(rng.integers(b, b + 4)))
    return es, box, swz, layout(), layout()


@pytest.mark.parametrize("chunk", range(4))
def test_corner4_random_maps(chunk):
    """The corner kernels in 4-byte lanes, on seeded random maps they take
    (every rank and element size, every row width from 16 to 256 bytes, with
    and without a swizzle inside the rows; with 1- and 2-byte elements the
    tensor's x edge cuts words), random corners in, across and outside the
    tensor and random deals: load, store of the loaded images at the same corners, round trip
    into a tensor of the same layout and into one of another layout, and the
    fp32 +1.0f round trip, against the oracle; some with every stage
    poisoned before its loads."""
    rng = np.random.default_rng(9700 + chunk)
    for i in range(30):
        es, box, swz, (dims, strides, alloc), (ddims, dstrides, dalloc) = _corner4_case(rng)
        coords = inputs.random_corners(dims, box, int(rng.integers(1, 400)), int(rng.integers(1 << 30)))
        n = len(coords)
        opts = dict(grid_wgs=int(rng.choice([0, 0, 1, 3])), group=int(rng.choice([0, 1, 2, 4])),
                    regions=int(rng.choice([0, 1, 2, 3])),
                    flags=int(rng.choice([0, T.FLAG_NONTEMPORAL, T.FLAG_CACHED_PACKED, T.FLAG_DEBUG_POISON])))
        say(f"corner4 chunk {chunk} case {i}: es={es} dims={dims} strides={strides} box={box} swz={swz} "
            f"ddims={ddims} dstrides={dstrides} n={n} opts={opts}")
        dt = dt_of(es)
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        omd = Map(es=es, dims=ddims, strides=dstrides, box=box, swizzle=swz)
        src = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        host = src.cpu().numpy()
        m = enc(dt, src, dims, strides, box, swz)
        bb = T.tmap_box_bytes(m)
        assert T.tmap_plan_launch("load", m, None, True, n, **opts)["variant"] == "corner4"
        packed = gpu_load(m, coords, n, **opts)
        want = oracle.load_tiles(om, host, coords, n)
        assert (mm := first_mismatch(packed.cpu().numpy(), want, bb)) is None, ("load", mm)
        c = torch.from_numpy(coords).to(DEV)
        dst = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        want_dst = dst.cpu().numpy().copy()
        T.tmap_store_tiles(enc(dt, dst, dims, strides, box, swz), c, n, packed, **opts)
        check_ok()
        oracle.store_tiles(om, want_dst, coords, n, want)
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("store", mm)
        for other in (False, True):
            d_dims, d_strides, d_alloc, od = (ddims, dstrides, dalloc, omd) if other else (dims, strides, alloc, om)
            dst = dev_tensor(d_alloc, fill_seed=int(rng.integers(1 << 30)))
            want_dst = dst.cpu().numpy().copy()
            md = enc(dt, dst, d_dims, d_strides, box, swz)
            assert T.tmap_plan_launch("roundtrip", m, md, True, n, **opts)["variant"] == "corner4"
            add = es == 4 and bool(rng.integers(0, 2))
            if add:
                T.tmap_roundtrip_add_f32(m, md, c, n, 1.0, **opts)
                oracle.roundtrip_add_f32(om, host, od, want_dst, coords, n, 1.0)
            else:
                T.tmap_roundtrip(m, md, c, n, **opts)
                oracle.roundtrip(om, host, od, want_dst, coords, n)
            check_ok()
            got = dst.cpu().numpy()
            if add:
                nan = np.isnan(want_dst.view(np.float32))
                assert np.array_equal(got.view(np.uint32)[~nan], want_dst.view(np.uint32)[~nan]), \
                    ("round trip +1.0f", other)
                assert np.all(np.isnan(got.view(np.float32)[nan]))
            else:
                assert (mm := first_mismatch(got, want_dst, 1 << 40)) is None, ("roundtrip", other, mm)


@pytest.mark.parametrize("chunk", range(2))
def test_corner4_sweeps(chunk):
    """Sweeps the band kernel does not take run on the corner kernel in
    4-byte lanes, their corners walked by the kernel's carry-add cursor:
    seeded random maps of every rank, element size, row width and in-row
    swizzle, random deals (groups, streams, grids, contiguous runs) and
    hints.  Load of every tile, store of random images through the sweep,
    round trip into the same layout and into another one, against the
    oracle."""
    rng = np.random.default_rng(9800 + chunk)
    for i in range(30):
        es, box, swz, (dims, strides, alloc), (ddims, dstrides, dalloc) = _corner4_case(rng)
        if len(box) < 3:
            # at least rank 3, so that a small tensor never takes the band schedule
            while len(box) < 3:
                box, dims, strides = box + [1], dims + [int(rng.integers(1, 4))], strides + [alloc]
                alloc *= dims[-1]
            ddims, dstrides, dalloc = dims, strides, alloc
        # a map whose extents above dimension 1 are all 1 may fold into a
        # rank-2 sweep (dense planes a whole number of boxes tall), which the
        # band kernel can take
        variant = ("corner4", "band") if all(b == 1 for b in box[2:]) else "corner4"
        _check_sweep(rng, f"corner4 sweep {chunk}/{i}", variant, es, box, swz,
                     (dims, strides, alloc), (ddims, dstrides, dalloc))


def _corner16_case(rng):
    """A map of rank 3 to 5 with boxes of at most 8 KiB that the corner
    kernel takes in 16-byte lanes only: box rows that are not a power of two
    from 16 to 256 bytes, more than 64 rows, or a swizzle of whole chunks
    whose XOR reaches past the row; and a second layout with the same box."""
    while True:
        es = int(rng.choice([1, 2, 4, 8]))
        lg = es.bit_length() - 1
        rank = int(rng.integers(3, 6))
        kind = int(rng.integers(0, 3))
        swz = (0, 0, 0)
        if kind == 0:
            row = 16 * int(rng.choice([3, 5, 6, 7, 9, 12, 32]))
            max_rows = 8192 // row
        elif kind == 1:
            row = int(rng.choice([16, 32]))
            max_rows = 8192 // row
        else:
            row = int(rng.choice([16, 32, 64]))
            max_rows = min(64, 8192 // row)
        if row // es > 256:
            continue
        box, rows = [row // es], 1
        for d in range(1, rank):
            b = int(rng.integers(1, min(256, max_rows // rows) + 1))
            if kind == 1 and d == 1:
                b = int(rng.integers(65, min(256, max_rows) + 1))
            box.append(b)
            rows *= b
        if kind == 1 and rows <= 64:
            continue
        if all(b == 1 for b in box[2:]):
            continue  # the band schedule could take it
        if kind == 2:
            lrow = row.bit_length() - 1
            n_el = int(np.prod(box))
            picks = [(b, m) for b in (1, 2, 3) for m in range(max(0, 4 - lg), 6)
                     if m + lg + b > lrow and n_el % (1 << (m + b)) == 0]
            if not picks:
                continue
            b, m = picks[int(rng.integers(0, len(picks)))]
            swz = (b, m, int(rng.integers(b, b + 4)))

        def layout():
            dims = [int(rng.integers(1, 2 * box[0] + 40))] + [int(rng.integers(1, 2 * b + 4)) for b in box[1:]]
            st = (-(-dims[0] * es // 16) + int(rng.integers(0, 3))) * 16
            strides = []
            for d in range(1, rank):
                strides.append(st)
                st *= dims[d] + int(rng.integers(0, 2))
            return dims, strides, st
        return es, box, swz, layout(), layout()


@pytest.mark.parametrize("chunk", range(2))
def test_corner_sweeps_in_16_byte_lanes(chunk):
    """Sweeps of rank 3 to 5 whose boxes the 4-byte lanes do not take run on
    the corner kernel in 16-byte lanes, their corners walked by the same
    cursor: random row widths, row counts and chunk swizzles, random deals
    and hints; load, store and round trips against the oracle."""
    rng = np.random.default_rng(9900 + chunk)
    for i in range(20):
        es, box, swz, lay, dlay = _corner16_case(rng)
        _check_sweep(rng, f"corner sweep {chunk}/{i}", "corner", es, box, swz, lay, dlay)


def _check_sweep(rng, tag, variant, es, box, swz, lay, dlay):
    """Load, store and round trips (into the same layout and into dlay) of
    the whole sweep of one map under random deals and hints, every byte
    against the oracle; the plan must name `variant`."""
    dims, strides, alloc = lay
    opts = dict(grid_wgs=int(rng.choice([0, 0, 1, 3])), group=int(rng.choice([0, 1, 2, 4])),
                regions=int(rng.choice([0, 1, 2, 3, 8])),
                flags=int(rng.choice([0, T.FLAG_NONTEMPORAL, T.FLAG_CONTIGUOUS, T.FLAG_DEBUG_POISON])))
    dt = dt_of(es)
    src = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
    host = src.cpu().numpy()
    m = enc(dt, src, dims, strides, box, swz)
    om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
    n = T.tmap_sweep_tiles(m)
    bb = T.tmap_box_bytes(m)
    say(f"{tag}: es={es} dims={dims} strides={strides} box={box} swz={swz} n={n} opts={opts}")
    got = T.tmap_plan_launch("load", m, None, False, n, **opts)["variant"]
    assert got in variant if isinstance(variant, tuple) else got == variant, (got, variant)
    packed = gpu_load(m, None, n, **opts)
    want = oracle.load_tiles(om, host, None, n)
    assert (mm := first_mismatch(packed.cpu().numpy(), want, bb)) is None, ("load", mm)
    imgs = inputs.sentinel_bytes(n * bb, int(rng.integers(1 << 30)))
    dst = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
    want_dst = dst.cpu().numpy().copy()
    T.tmap_store_tiles(enc(dt, dst, dims, strides, box, swz), None, n, torch.from_numpy(imgs).to(DEV), **opts)
    check_ok()
    oracle.store_tiles(om, want_dst, None, n, imgs)
    assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("store", mm)
    for other in (False, True):
        d_dims, d_strides, d_alloc = dlay if other else lay
        od = Map(es=es, dims=d_dims, strides=d_strides, box=box, swizzle=swz)
        dst = dev_tensor(d_alloc, fill_seed=int(rng.integers(1 << 30)))
        want_dst = dst.cpu().numpy().copy()
        T.tmap_roundtrip(m, enc(dt, dst, d_dims, d_strides, box, swz), None, n, **opts)
        check_ok()
        oracle.roundtrip(om, host, od, want_dst, None, n)
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("roundtrip", other, mm)


def test_batched_sweeps_run_on_the_band_kernel():
    """Sweeps of 2-D boxes over a batch of matrices (boxes of extent 1 above
    dimension 1): dense planes a whole number of boxes tall fold into one
    taller matrix; other batches of rank 3 walk their planes with the band
    kernel's third cursor digit (ragged plane heights, padded planes, a
    round trip into planes of another height or into fewer planes); a
    padded batch of rank 4 runs elsewhere.  Every direction against the
    oracle."""
    say("batched sweeps")
    cases = [  # dims, strides (bytes), variant
        ([512, 256, 6], [1024, 1024 * 256], "band"),
        ([512, 256, 3, 2], [1024, 1024 * 256, 1024 * 256 * 3], "band"),
        ([512, 250, 6], [1024, 1024 * 250], "band"),           # 250 rows: the last tile row of a plane is ragged
        ([512, 256, 6], [1024, 1024 * 256 + 512], "band"),     # padded planes
        ([512, 250, 3, 2], [1024, 1024 * 256, 1024 * 256 * 4], "corner4"),  # rank 4: 8 KiB boxes, 4-byte lanes
    ]
    box, swz = [64, 64, 1], (3, 3, 3)
    for dims, strides, variant in cases:
        bx = box + [1] * (len(dims) - 3)
        alloc = dims[-1] * strides[-1]
        src = dev_tensor(alloc, fill_seed=len(dims) + dims[1])
        host = src.cpu().numpy()
        m = enc("bf16", src, dims, strides, bx, swz)
        om = Map(es=2, dims=dims, strides=strides, box=bx, swizzle=swz)
        n = T.tmap_sweep_tiles(m)
        for direction in ("load", "store", "roundtrip"):
            p = T.tmap_plan_launch(direction, m, m if direction == "roundtrip" else None, False, n)
            assert p["variant"] == variant, (dims, strides, direction, p)
        packed = gpu_load(m, None, n)
        want = oracle.load_tiles(om, host, None, n)
        assert (mm := first_mismatch(packed.cpu().numpy(), want, T.tmap_box_bytes(m))) is None, ("load", dims, mm)
        dst = dev_tensor(alloc, fill_seed=7)
        want_dst = dst.cpu().numpy().copy()
        T.tmap_store_tiles(enc("bf16", dst, dims, strides, bx, swz), None, n, packed)
        check_ok()
        oracle.store_tiles(om, want_dst, None, n, want)
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("store", dims, mm)
        dst = dev_tensor(alloc, fill_seed=8)
        want_dst = dst.cpu().numpy().copy()
        T.tmap_roundtrip(m, enc("bf16", dst, dims, strides, bx, swz), None, n)
        check_ok()
        oracle.roundtrip(om, host, om, want_dst, None, n)
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("roundtrip", dims, mm)
    # round trips into planes of another height, and into fewer planes
    # (those past the destination's last are not written)
    dims, strides = [512, 256, 6], [1024, 1024 * 256]
    src = dev_tensor(dims[-1] * strides[-1], fill_seed=11)
    for ddims, dstrides in (([512, 320, 6], [1024, 1024 * 320]), ([512, 200, 4], [1024, 1024 * 208])):
        dst = dev_tensor(ddims[-1] * dstrides[-1], fill_seed=12)
        m, md = enc("bf16", src, dims, strides, box, swz), enc("bf16", dst, ddims, dstrides, box, swz)
        n = T.tmap_sweep_tiles(m)
        assert T.tmap_plan_launch("roundtrip", m, md, False, n)["variant"] == "band"
        want_dst = dst.cpu().numpy().copy()
        T.tmap_roundtrip(m, md, None, n)
        check_ok()
        oracle.roundtrip(Map(es=2, dims=dims, strides=strides, box=box, swizzle=swz), src.cpu().numpy(),
                         Map(es=2, dims=ddims, strides=dstrides, box=box, swizzle=swz), want_dst, None, n)
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst, 1 << 40)) is None, ("roundtrip into", ddims, mm)


def test_binding_rejects_buffers_the_copy_would_overrun():
    """Given tensors, the binding checks sizes before launching: a packed
    buffer or corner array too small for n_tiles, a host tensor or int64
    corners never reach the GPU."""
    say("binding argument guards")
    src = dev_tensor(64 * 256, fill_seed=1)
    m = enc("f32", src, [64, 64], [256], [16, 16])
    n = T.tmap_sweep_tiles(m)
    bb = T.tmap_box_bytes(m)
    ok = torch.empty(n * bb, dtype=torch.uint8, device=DEV)
    cases = [
        lambda: T.tmap_load_tiles(m, None, n, torch.empty(n * bb - 16, dtype=torch.uint8, device=DEV)),
        lambda: T.tmap_load_tiles(m, None, n, torch.empty(n * bb, dtype=torch.uint8)),
        lambda: T.tmap_store_tiles(m, torch.zeros((n, 2), dtype=torch.int64, device=DEV), n, ok),
        lambda: T.tmap_store_tiles(m, torch.zeros((n - 1, 2), dtype=torch.int32, device=DEV), n, ok),
        lambda: T.tmap_roundtrip(m, m, torch.zeros((1, 2), dtype=torch.int32, device=DEV), 2),
        lambda: T.tmap_load_tiles(m, None, n, ok.view(2, -1)[:, ::2]),
        lambda: T.tmap_bulk_copy(torch.empty(64, dtype=torch.uint8, device=DEV), src, 128),
    ]
    for i, bad in enumerate(cases):
        with pytest.raises(ValueError):
            bad()
    T.tmap_load_tiles(m, None, n, ok)
    check_ok()


def test_plan_query_reports_the_schedules():
    """The schedule each workload's copies take by default, and what the
    mode flags turn it into, as tmap_plan_launch reports it."""
    W = inputs.WORKLOADS
    def plan(name, direction, **opts):
        w = W[name]
        m = T.tmap_encode(w.dtype, w.rank, 0x7F0000000000, w.dims, w.strides, w.box, None, w.swizzle)
        corners = w.coords != "sweep"
        n = None if not corners else (1 if w.coords == "origin" else w.n_random)
        return T.tmap_plan_launch(direction, m, m if direction == "roundtrip" else None, corners, n, **opts)
    say("plan query")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = plan("sweep2g_u8", "roundtrip", flags=T.FLAG_NONTEMPORAL)
    assert (p["variant"], p["band_boxes"], p["band_rows"], p["stages"], p["group"], p["regions"]) == \
        ("band", 16, 8, 3, 2, 1)
    # 512 boxes a row in units of 16, 256 box rows of 16 bands each
    assert p["units"] == (512 // 16) * 256 * 16 and p["walkers"] == p["workgroups"] == p["units"] // 2
    # the ragged sweep's 32640-byte pitch is not a power of two: its round
    # trip takes 2-row bands of 64 boxes, dealt as two streams
    p = plan("ragged_bf16", "roundtrip", flags=T.FLAG_NONTEMPORAL)
    assert (p["variant"], p["band_boxes"], p["band_rows"], p["stages"], p["group"], p["regions"]) == \
        ("band", 64, 2, 3, 2, 2)
    p = plan("sweep2g_u8", "load", flags=T.FLAG_NONTEMPORAL)
    assert (p["variant"], p["band_boxes"], p["band_rows"], p["stages"], p["group"], p["regions"]) == \
        ("band", 8, 16, 3, 2, 2)
    # the padded 5-D fp32 boxes: the corner kernels in 4-byte lanes, one box
    # to a wave in every direction; 8 KiB boxes: one wave to a workgroup,
    # each with its own one-box stage
    # the waves, one to a workgroup, are dealt as 8 interleaved streams, one
    # to each XCD's workgroups; four-wave workgroups keep one stream
    for direction in ("load", "store", "roundtrip"):
        p = plan("pad5d_f32", direction)
        assert (p["variant"], p["stages"], p["slots"], p["group"], p["regions"]) == ("corner4", 1, 8, 1, 8), direction
        assert p["walkers"] == 100000 and p["workgroups"] == p["walkers"], direction
        assert p["lds_bytes"] == 8192 + 8, direction
    # 2 KiB boxes: four waves to a workgroup, two boxes to a wave, one
    # stream; 4 KiB boxes one box to a wave, dealt as 32 streams (one per XCD
    # and wave slot); 1 KiB boxes four to a wave
    m = T.tmap_encode("f32", 2, 0x7F0000000000, [1000, 1000], [4000], [32, 16])
    p = T.tmap_plan_launch("load", m, None, True, 1000)
    assert (p["variant"], p["slots"], p["group"], p["walkers"], p["regions"]) == ("corner4", 2, 2, 500, 1)
    assert T.tmap_plan_launch("load", m, None, True, 1000, regions=3)["regions"] == 3
    assert p["workgroups"] == 125 and p["lds_bytes"] == 4 * 2048 + 4 * 8
    m = T.tmap_encode("f32", 2, 0x7F0000000000, [1000, 1000], [4000], [32, 32])
    for direction in ("load", "store", "roundtrip"):
        p = T.tmap_plan_launch(direction, m, m if direction == "roundtrip" else None, True, 1000)
        assert (p["variant"], p["slots"], p["group"], p["walkers"], p["workgroups"], p["regions"]) == \
            ("corner4", 4, 1, 1000, 250, 32), direction
    m = T.tmap_encode("f32", 2, 0x7F0000000000, [1000, 1000], [4000], [32, 8])
    p = T.tmap_plan_launch("store", m, None, True, 1000)
    assert (p["variant"], p["slots"], p["group"], p["walkers"], p["regions"]) == ("corner4", 1, 4, 250, 1)
    # 16-bit elements in 8 KiB boxes with a swizzle whose XOR reaches past a
    # 128-byte row: the corner kernel in 16-byte lanes; its loads reserve
    # 11 KiB of LDS to a workgroup; one box to a wave in every direction
    m = T.tmap_encode("bf16", 2, 0x7F0000000000, [1000, 1000], [2048], [64, 64], None, (3, 4, 3))
    p = T.tmap_plan_launch("load", m, None, True, 1000)
    assert (p["variant"], p["group"], p["lds_bytes"], p["walkers"], p["regions"]) == ("corner", 1, 11264, 1000, 8)
    p = T.tmap_plan_launch("store", m, None, True, 1000)
    assert (p["variant"], p["group"], p["lds_bytes"], p["walkers"]) == ("corner", 1, 8192 + 8, 1000)
    assert T.tmap_plan_launch("roundtrip", m, m, True, 1000)["group"] == 1
    # sweeps of rank 5 (never the band schedule) whose boxes suit the 4-byte
    # lanes run there, one stage, one box to a wave, the waves dealt to the
    # XCDs; two stages keep the shared ring
    w = W["pad5d_sweep_f32"]
    m5 = T.tmap_encode(w.dtype, w.rank, 0x7F0000000000, w.dims, w.strides, w.box)
    n5 = T.tmap_sweep_tiles(m5)
    assert n5 == 5 * 9 * 9 * 7 * 7
    for direction in ("load", "roundtrip", "store"):
        p = T.tmap_plan_launch(direction, m5, m5 if direction == "roundtrip" else None, False, n5)
        assert (p["variant"], p["stages"], p["group"], p["regions"]) == ("corner4", 1, 1, 8), (direction, p)
    p = T.tmap_plan_launch("load", m5, None, False, n5, stages=2)
    assert (p["variant"], p["regions"]) == ("ring", 1)
    # what the 4-byte lanes take: box rows of a power of two from 16 to 256
    # bytes, at most 64 rows to a box, no swizzle or one that moves whole
    # 16-byte chunks within rows with a key of at most 4 bits
    def variant(dtype, pitch, box, swz=(0, 0, 0)):
        strides = [pitch * 1000 ** k for k in range(len(box) - 1)]
        mm = T.tmap_encode(dtype, len(box), 0x7F0000000000, [1000] * len(box), strides, box, None, swz)
        return T.tmap_plan_launch("roundtrip", mm, mm, True, 100)["variant"]
    assert variant("f32", 4000, [32, 64]) == "corner4"            # 128-byte rows, 64 rows
    assert variant("f64", 8000, [2, 8, 4]) == "corner4"           # 16-byte rows, 32 rows
    assert variant("f32", 4000, [64, 32]) == "corner4"            # 256-byte rows
    assert variant("f32", 4000, [128, 16]) == "corner"            # 512-byte rows
    assert variant("f32", 4000, [4, 128]) == "corner"             # 128 rows
    assert variant("f32", 4000, [12, 16]) == "corner"             # 48-byte rows
    assert variant("f32", 4000, [32, 64], (3, 2, 3)) == "corner4"  # 128-byte swizzle, 128-byte rows
    assert variant("bf16", 2000, [64, 64], (3, 3, 3)) == "corner4"
    assert variant("f32", 4000, [16, 64], (3, 2, 3)) == "corner"   # 128-byte swizzle, 64-byte rows
    assert variant("f32", 4000, [32, 64], (3, 3, 3)) == "corner"   # its XOR reaches past the row
    assert variant("f32", 4000, [32, 64], (1, 0, 1)) == "corner4"  # 4-byte granules: whole words
    assert variant("f64", 8000, [16, 64], (2, 0, 3)) == "corner4"  # 8-byte granules
    assert variant("bf16", 2000, [64, 64], (1, 1, 2)) == "corner4"  # 4-byte granules of 2 elements
    assert variant("bf16", 2000, [64, 64], (1, 0, 1)) == "wave_per_box"  # 2-byte granules: inside words
    assert variant("u8", 1008, [128, 64], (2, 1, 3)) == "wave_per_box"
    assert variant("bf16", 2000, [64, 64]) == "corner4"           # 2-byte elements
    assert variant("u8", 1008, [16, 8, 4]) == "corner4"           # bytes, 16-byte rows
    assert plan("pad5d_f32", "roundtrip", stages=2)["variant"] == "wave_per_box"
    assert plan("pad5d_f32", "load", flags=T.FLAG_WHOLE_BOX)["variant"] == "ring"
    assert plan("pad5d_f32", "load", stages=3)["variant"] == "ring"
    assert plan("tile64_f32", "roundtrip")["variant"] == "ring"              # a 16 KiB box: the shared ring
    # a cache-resident sweep on the band kernel: the tallest band that fits
    # (half of a 32 KiB box), 2 stages x 2 units
    p = plan("strips_f16", "load")
    assert (p["variant"], p["band_boxes"], p["band_rows"], p["stages"], p["group"], p["regions"]) == \
        ("band", 1, 32, 2, 2, 1)
    assert plan("strips_f16", "load", flags=T.FLAG_THREAD_COPY)["variant"] == "thread_copy"
    p = plan("sweep2g_u8", "load", flags=T.FLAG_PRODUCER_WAVE)
    assert (p["variant"], p["band_boxes"], p["workgroups"]) == ("producer_wave", 0, 8 * cus)
    assert plan("sweep2g_u8", "load", flags=T.FLAG_CONTIGUOUS | T.FLAG_WHOLE_BOX)["group"] == 0
    # whole boxes on the band kernel: round trips of 16 KiB boxes take 4
    # stages x 4 units in one stream, everything else 3 x 2 in two streams
    whole = T.FLAG_NONTEMPORAL | T.FLAG_WHOLE_BOX
    for name, direction, want in (("sweep2g_u8", "roundtrip", (1, 128, 4, 4, 1)), ("sweep2g_u8", "load", (1, 128, 3, 2, 2)),
                                  ("plus1_f32", "roundtrip", (1, 64, 4, 4, 1)), ("ragged_bf16", "roundtrip", (2, 64, 3, 2, 2))):
        p = plan(name, direction, flags=whole)
        assert p["variant"] == "band", (name, direction)
        assert (p["band_boxes"], p["band_rows"], p["stages"], p["group"], p["regions"]) == want, (name, direction, p)


def test_zero_tiles_launch_nothing():
    src = dev_tensor(16384, fill_seed=1)
    m = enc("f32", src, [64, 64], [256], [64, 64])
    out = dev_tensor(16)
    T.tmap_load_tiles(m, torch.zeros((1, 2), dtype=torch.int32, device=DEV), 0, out)
    check_ok()


def test_launch_options_out_of_range_are_rejected():
    """Launch options outside their documented ranges (flag bits the header
    does not define among them) give INVALID_VALUE before anything is
    launched, and the destination stays untouched."""
    src = dev_tensor(16384, fill_seed=1)
    m = enc("f32", src, [64, 64], [256], [16, 16])
    n = T.tmap_sweep_tiles(m)
    out = dev_tensor(n * 1024, fill_seed=2)
    before = out.clone()
    for bad in (dict(stages=5), dict(group=3), dict(group=128), dict(regions=65),
                dict(flags=T.FLAG_BAND | T.FLAG_WHOLE_BOX),
                dict(flags=T.FLAG_THREAD_COPY | T.FLAG_PRODUCER_WAVE),
                dict(flags=T.FLAG_WAVE_PER_BOX | T.FLAG_THREAD_COPY),
                dict(flags=T.FLAG_WAVE_PER_BOX | T.FLAG_PRODUCER_WAVE), dict(flags=T.FLAG_WAVE_PER_BOX, stages=3),
                dict(flags=0x400), dict(flags=0x800), dict(flags=T.FLAG_NONTEMPORAL | 0x80000000)):
        with pytest.raises(T.TmapError) as e:
            T.tmap_load_tiles(m, None, n, out, **bad)
        assert e.value.status == T.INVALID_VALUE, bad
    check_ok()
    assert torch.equal(out, before)
    for ok in (dict(regions=64), dict(regions=1), dict(group=64, regions=7)):
        T.tmap_load_tiles(m, None, n, out, **ok)
        check_ok()


def test_budget_mismatch_times_out_on_the_band_schedule():
    """The same on a band-schedule sweep: each 16 KiB unit's record never
    reaches zero outstanding bytes."""
    say("budget mismatch -> TIMEOUT (band schedule)")
    src = dev_tensor(1024 * 64, fill_seed=2)
    m = enc("u8", src, [1024, 64], [1024], [128, 16])
    assert T.tmap_band_boxes(m, None, False, T.FLAG_BAND) == 8
    n = T.tmap_sweep_tiles(m)
    out = dev_tensor(n * 2048)
    T.tmap_load_tiles(m, None, n, out, flags=T.FLAG_INJECT_BUDGET_MISMATCH | T.FLAG_BAND, spin_limit=2000)
    assert T.tmap_sync_status() == T.TIMEOUT
    T.tmap_load_tiles(m, None, n, out, flags=T.FLAG_BAND)
    check_ok()
    om = Map(es=1, dims=[1024, 64], strides=[1024], box=[128, 16])
    assert out.cpu().numpy().tobytes() == oracle.load_tiles(om, src.cpu().numpy(), None, n).tobytes()


@pytest.mark.parametrize("mode", [0, T.FLAG_PRODUCER_WAVE, T.FLAG_WAVE_PER_BOX])
def test_budget_mismatch_times_out_instead_of_hanging(mode):
    """Announce 16 more bytes than delivered: the stage never becomes ready; the
    bounded wait ends the kernel and the status reports a timeout."""
    say(f"budget mismatch -> TIMEOUT (flags {mode})")
    src = dev_tensor(16384, fill_seed=1)
    m = enc("f32", src, [64, 64], [256], [64, 64])
    out = dev_tensor(16384 * 4)
    coords = torch.zeros((4, 2), dtype=torch.int32, device=DEV)
    T.tmap_load_tiles(m, coords, 4, out, stages=2, flags=T.FLAG_INJECT_BUDGET_MISMATCH | mode, spin_limit=2000)
    assert T.tmap_sync_status() == T.TIMEOUT
    # the library keeps working afterwards
    T.tmap_load_tiles(m, coords, 4, out, stages=2, flags=mode)
    check_ok()
    assert torch.equal(out.view(4, -1)[3], src)


def test_timeouts_are_reported_to_their_own_stream():
    """Each stream that launches copies has its own status word: a copy
    whose readiness wait expires on one stream is reported to that stream
    alone, and checking another stream neither sees it nor clears it."""
    say("timeouts per stream")
    src = dev_tensor(256 * 100, fill_seed=3)
    dims, box = [64, 100], [64, 32]
    m = enc("f32", src, dims, [256], box)
    coords = torch.tensor([[0, 0], [0, 50], [-9, 90]], dtype=torch.int32, device=DEV)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    out_a, out_b = dev_tensor(8192 * 3), dev_tensor(8192 * 3)
    torch.cuda.synchronize()
    for _ in range(2):
        T.tmap_load_tiles(m, coords, 3, out_a, flags=T.FLAG_INJECT_BUDGET_MISMATCH, spin_limit=2000, stream=sa)
        T.tmap_load_tiles(m, coords, 3, out_b, stream=sb)
        assert T.tmap_sync_status(sb) == T.SUCCESS
        assert T.tmap_sync_status() == T.SUCCESS       # the current stream launched nothing
        assert T.tmap_sync_status(sa) == T.TIMEOUT
        assert T.tmap_sync_status(sa) == T.SUCCESS     # read and cleared
    om = Map(es=4, dims=dims, strides=[256], box=box)
    want = oracle.load_tiles(om, src.cpu().numpy(), coords.cpu().numpy(), 3)
    assert out_b.cpu().numpy().tobytes() == want.tobytes()


@pytest.mark.parametrize("dtype", ["u8", "f32"])
def test_budget_mismatch_times_out_in_the_corner_kernels(dtype):
    """The same for boxes at explicit corners, one wave per box: the corner
    kernel in 16-byte lanes (swizzled u8) and in 4-byte lanes (fp32), each
    direction."""
    es = 1 if dtype == "u8" else 4
    box = [128 // es, 64]
    dims = [256 // es, 100]
    swz = (3, 5, 3) if es == 1 else (0, 0, 0)     # its XOR reaches past the 128-byte row
    src = dev_tensor(256 * 100, fill_seed=3)
    dst = dev_tensor(256 * 100, fill_seed=4)
    m, md = enc(dtype, src, dims, [256], box, swz), enc(dtype, dst, dims, [256], box, swz)
    assert T.tmap_plan_launch("load", m, None, True, 4)["variant"] == ("corner" if es == 1 else "corner4")
    coords = torch.tensor([[0, 0], [3, 5], [-7, 60], [200 // es, -10]], dtype=torch.int32, device=DEV)
    out = dev_tensor(8192 * 4)
    for direction in ("load", "store", "roundtrip"):
        say(f"budget mismatch -> TIMEOUT ({dtype} corner kernel, {direction})")
        for flags in (T.FLAG_INJECT_BUDGET_MISMATCH, 0):
            if direction == "load":
                T.tmap_load_tiles(m, coords, 4, out, flags=flags, spin_limit=2000)
            elif direction == "store":
                T.tmap_store_tiles(md, coords, 4, out, flags=flags, spin_limit=2000)
            else:
                T.tmap_roundtrip(m, md, coords, 4, flags=flags, spin_limit=2000)
            assert T.tmap_sync_status() == (T.TIMEOUT if flags else T.SUCCESS), (direction, flags)
    # the library keeps working afterwards
    T.tmap_load_tiles(m, coords, 4, out)
    check_ok()
    om = Map(es=es, dims=dims, strides=[256], box=box, swizzle=swz)
    assert out.cpu().numpy().tobytes() == oracle.load_tiles(om, src.cpu().numpy(), coords.cpu().numpy(), 4).tobytes()


def test_repeat_is_deterministic():
    w = inputs.WORKLOADS["pad5d_f32"]
    src = inputs.device_bytes(w, DEV)
    coords = inputs.random_corners(w.dims, w.box, 5000, seed=4)
    m = enc("f32", src, w.dims, w.strides, w.box)
    a = gpu_load(m, coords, len(coords))
    for st in (1, 2, 3, 4):
        b = gpu_load(m, coords, len(coords), stages=st, grid_wgs=97)
        assert torch.equal(a, b), st


@pytest.mark.parametrize("name", ["tile64_f32", "strips_f16", "ragged_bf16", "pad5d_f32", "pad5d_sweep_f32", "sweep2g_u8"])
def test_other_modes_match_the_oracle(name):
    """The register-path, producer-wave and wave-per-box variants, the ring
    on whole boxes, and other deals of the groups to the grid (regions), at
    full size: load, store and round trip of every workload, each output
    byte against the oracle."""
    w = inputs.WORKLOADS[name]
    modes = {"thread_copy": dict(flags=T.FLAG_THREAD_COPY), "producer_wave": dict(flags=T.FLAG_PRODUCER_WAVE),
             "wave_per_box": dict(flags=T.FLAG_WAVE_PER_BOX), "whole_box": dict(flags=T.FLAG_WHOLE_BOX),
             "regions_3": dict(regions=3), "regions_1": dict(regions=1)}
    which = (20000, 44)
    for mode, alt in modes.items():
        say(f"{mode} vs oracle: {name}")
        m = T.tmap_encode(w.dtype, w.rank, 0x7F0000000000, w.dims, w.strides, w.box, None, w.swizzle)
        if mode == "wave_per_box" and T.tmap_box_bytes(m) > 16384:
            # a wave's stage holds at most 16 KiB: rejected before any launch
            src = inputs.device_bytes(w, DEV)
            m = enc(w.dtype, src, w.dims, w.strides, w.box, w.swizzle)
            out = torch.empty(T.tmap_box_bytes(m), dtype=torch.uint8, device=DEV)
            with pytest.raises(T.TmapError) as e:
                T.tmap_load_tiles(m, torch.zeros((1, w.rank), dtype=torch.int32, device=DEV), 1, out, **alt)
            assert e.value.status == T.INVALID_VALUE
            continue
        check_all_directions(name, alt, which, tag=mode)
    forget(name)


@pytest.mark.parametrize("rank", [2, 3, 5])
def test_corner_round_trip_between_layouts(rank):
    """Round trips of scattered corners (in, across and outside both tensors)
    from one tensor into another of a different size and pitch: the corner
    kernel's instances for destinations that differ from the source, against
    the oracle, for 8 KiB boxes (a wave to a workgroup) and 2 KiB boxes (four
    waves to a workgroup), with the fp32 +1.0f update too."""
    rng = np.random.default_rng(9500 + rank)
    for box_kib in (2, 8):
        es = 4
        if rank == 2:
            box, dims, ddims = ([32, 16] if box_kib == 2 else [64, 32]), [301, 77], [333, 60]
        elif rank == 3:
            box, dims, ddims = ([16, 8, 4] if box_kib == 2 else [32, 8, 8]), [77, 29, 21], [90, 25, 23]
        else:
            box, dims, ddims = ([8, 4, 4, 2, 2] if box_kib == 2 else [16, 8, 4, 2, 2]), [37, 11, 9, 5, 3], \
                [41, 9, 10, 5, 4]

        def layout(d):
            strides, s = [], (-(-d[0] * es // 16) + 1) * 16
            for k in range(1, len(d)):
                strides.append(s)
                s *= d[k]
            return strides, s
        strides, alloc = layout(dims)
        dstrides, dalloc = layout(ddims)
        src = dev_tensor(alloc, fill_seed=int(rng.integers(1 << 30)))
        host = src.cpu().numpy()
        # a 64-byte-granule swizzle whose XOR reaches past every row here:
        # the corner kernel in 16-byte lanes
        swz = (3, 4, 3)
        ms = enc("f32", src, dims, strides, box, swz)
        corners = inputs.random_corners(dims, box, 700, seed=int(rng.integers(1 << 30)))
        c = torch.from_numpy(corners).to(DEV)
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        omd = Map(es=es, dims=ddims, strides=dstrides, box=box, swizzle=swz)
        for add in (False, True):
            say(f"corner round trip between layouts: rank {rank}, box {box_kib} KiB, add={add}")
            dst = dev_tensor(dalloc, fill_seed=int(rng.integers(1 << 30)))
            want = dst.cpu().numpy().copy()
            md = enc("f32", dst, ddims, dstrides, box, swz)
            assert T.tmap_plan_launch("roundtrip", ms, md, True, len(corners))["variant"] == "corner"
            if add:
                T.tmap_roundtrip_add_f32(ms, md, c, len(corners), 1.0)
                oracle.roundtrip_add_f32(om, host, omd, want, corners, len(corners), 1.0)
            else:
                T.tmap_roundtrip(ms, md, c, len(corners))
                oracle.roundtrip(om, host, omd, want, corners, len(corners))
            check_ok()
            got = dst.cpu().numpy()
            if add:
                nan = np.isnan(want.view(np.float32))
                assert np.array_equal(got.view(np.uint32)[~nan], want.view(np.uint32)[~nan]), "round trip +1.0f"
                assert np.all(np.isnan(got.view(np.float32)[nan]))
            else:
                assert (mm := first_mismatch(got, want, 1 << 40)) is None, (rank, box_kib, mm)
