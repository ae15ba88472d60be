"""GPU parity of the band schedule (sweeps of narrow boxes staged as bands
of rows of neighbouring boxes, 16 KiB to a stage) against the CPU oracle,
byte for byte.

Seeded random maps that take the band schedule (the host query says so for
every case): element sizes 1..8, box rows of 64..512 bytes, dimension-1
extents 16..128, band heights 1..64 rows, ranks 2..5 with higher box extents
1, swizzles that map a band onto itself (often with a period longer than a
band, so that the bands of a box differ by an XOR), ragged last rows and
columns, and rows of the sweep whose last unit holds fewer boxes than a full
one.  Each case loads, stores and round
trips (into a destination map of another size and pitch, so that the boxes
missing from a short last unit would land inside it if they were stored),
and fp32 cases also run the fused +addend round trip.
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import Map
from tiled_tensor_bulk_amd import inputs
from tiled_tensor_bulk_amd import tmap as T

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda:0"
DT = {1: "u8", 2: "f16", 4: "f32", 8: "f64"}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_ok():
    st = T.tmap_sync_status()
    assert st == T.SUCCESS, T.tmap_status_string(st)


def dev_bytes(nbytes, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    n8 = (nbytes + 7) // 8
    x = torch.randint(-(2**63), 2**63 - 1, (n8,), dtype=torch.int64, generator=g, device=DEV)
    return x.view(torch.uint8)[:nbytes].contiguous()


def first_mismatch(a, b):
    idx = np.flatnonzero(a != b)
    return None if idx.size == 0 else f"byte {int(idx[0])}: got {a[idx[0]]:#x} want {b[idx[0]]:#x}; {idx.size} differ"


def _strides(rng, dims, es):
    row = -(-dims[0] * es // 16) * 16 + 16 * int(rng.integers(0, 3))
    out, s = [], row
    for d in range(1, len(dims)):
        out.append(s)
        s *= dims[d]
    return out, s


def _swizzle(rng, es, box0, box1, rows):
    """A random swizzle the encoder accepts that maps a band of `rows` box
    rows onto itself (rows * box0 a multiple of 2^(m+b)); often one whose
    period is longer than a band, so that bands differ by an XOR."""
    n_el = box0 * box1
    k_el = 16 // es
    for _ in range(20):
        b = int(rng.integers(0, 4))
        if b == 0:
            return (0, 0, 0)
        m = int(rng.integers(k_el.bit_length() - 1, 5))
        s = int(rng.integers(b, 7))
        if n_el % (1 << (m + b)) == 0 and (rows * box0) % (1 << (m + b)) == 0 and b + m + s <= 20:
            return (b, m, s)
    return (0, 0, 0)


def _band_case(rng):
    """(es, dims, box, swizzle, band_rows asked for (0: the default 16),
    boxes per unit)."""
    while True:
        es = int(rng.choice([1, 2, 4, 8]))
        rc = int(rng.choice([4, 8, 16, 32]))     # 16-byte chunks per box row
        box0 = rc * 16 // es
        if box0 <= 256:
            break
    box1 = int(rng.choice([16, 32, 64, 128]))
    while box0 * es * box1 > 65536:
        box1 //= 2
    want_rows = int(rng.choice([0, 0, 1, 2, 4, 8, 16, 32, 64]))
    while want_rows > box1 or want_rows * rc > 1024:
        want_rows //= 2
    rows = want_rows or 16
    g = 1024 // (rows * rc)
    rank = int(rng.choice([2, 2, 2, 3, 4, 5]))
    tiles0 = int(rng.integers(g, 3 * g + 3))
    dims0 = tiles0 * box0 - int(rng.integers(0, box0))
    dims1 = int(rng.integers(1, (3 if rank == 2 else 2) * box1 + 2))
    dims = [dims0, dims1] + [int(rng.integers(1, 3)) for _ in range(rank - 2)]
    box = [box0, box1] + [1] * (rank - 2)
    return es, dims, box, _swizzle(rng, es, box0, box1, rows), want_rows, g


def _opts(rng, band_rows):
    # these tensors are small: TMAP_FLAG_BAND takes the band schedule anyway
    return dict(stages=int(rng.integers(1, 5)), grid_wgs=int(rng.choice([0, 0, 1, 3, 7])),
                group=int(rng.choice([0, 1, 2, 4, 8])), regions=int(rng.choice([0, 0, 1, 2, 3])),
                flags=T.FLAG_BAND | int(rng.choice([0, T.FLAG_NONTEMPORAL, T.FLAG_CONTIGUOUS])),
                band_rows=band_rows)


@pytest.mark.parametrize("chunk", range(4))
def test_band_schedule_random_sweeps(chunk):
    rng = np.random.default_rng(7100 + chunk)
    for i in range(24):
        es, dims, box, swz, rows, g_want = _band_case(rng)
        strides, alloc = _strides(rng, dims, es)
        opts = _opts(rng, rows)
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        src = dev_bytes(alloc, int(rng.integers(1 << 30)))
        m = T.tmap_encode(DT[es], len(dims), src.data_ptr(), dims, strides, box, None, swz)
        g = T.tmap_band_boxes(m, None, False, opts["flags"], rows)
        say(f"band {chunk}/{i}: es={es} dims={dims} strides={strides} box={box} swz={swz} boxes/unit={g} {opts}")
        # an explicit height gives exactly its unit; the default takes the
        # direction's height or a taller one, at most the 16 rows built for
        assert g == g_want if rows else g >= g_want
        n = T.tmap_sweep_tiles(m)
        bb = T.tmap_box_bytes(m)
        host = src.cpu().numpy()
        # load
        packed = torch.empty(n * bb, dtype=torch.uint8, device=DEV)
        T.tmap_load_tiles(m, None, n, packed, **opts)
        check_ok()
        want = oracle.load_tiles(om, host, None, n)
        assert (mm := first_mismatch(packed.cpu().numpy(), want, )) is None, ("load", mm)
        # store of random images into a sentinel-filled tensor
        imgs = dev_bytes(n * bb, int(rng.integers(1 << 30)))
        dst = dev_bytes(alloc, int(rng.integers(1 << 30)))
        want_dst = dst.cpu().numpy().copy()
        T.tmap_store_tiles(T.tmap_encode(DT[es], len(dims), dst.data_ptr(), dims, strides, box, None, swz),
                           None, n, imgs, **opts)
        check_ok()
        oracle.store_tiles(om, want_dst, None, n, imgs.cpu().numpy())
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst)) is None, ("store", mm)
        # round trip into a destination of another size and pitch
        ddims = [max(1, d + int(rng.integers(-b // 2, 2 * b + 1))) for d, b in zip(dims, box)]
        dstrides, dalloc = _strides(rng, ddims, es)
        dst2 = dev_bytes(dalloc, int(rng.integers(1 << 30)))
        want2 = dst2.cpu().numpy().copy()
        md = T.tmap_encode(DT[es], len(dims), dst2.data_ptr(), ddims, dstrides, box, None, swz)
        g_rt = T.tmap_band_boxes(m, md, False, opts["flags"], rows)
        assert g_rt == g if rows else g_rt >= g_want
        T.tmap_roundtrip(m, md, None, n, **opts)
        check_ok()
        omd = Map(es=es, dims=ddims, strides=dstrides, box=box, swizzle=swz)
        oracle.roundtrip(om, host, omd, want2, None, n)
        assert (mm := first_mismatch(dst2.cpu().numpy(), want2)) is None, ("roundtrip", ddims, mm)
        if es == 4:
            dst3 = dev_bytes(dalloc, int(rng.integers(1 << 30)))
            want3 = dst3.cpu().numpy().copy()
            md3 = T.tmap_encode("f32", len(dims), dst3.data_ptr(), ddims, dstrides, box, None, swz)
            T.tmap_roundtrip_add_f32(m, md3, None, n, 1.0, **opts)
            check_ok()
            oracle.roundtrip_add_f32(om, host, omd, want3, None, n, 1.0)
            got3 = dst3.cpu().numpy()
            nan = np.isnan(want3.view(np.float32))
            w32, g32 = want3.view(np.uint32), got3.view(np.uint32)
            assert np.array_equal(g32[~nan], w32[~nan]), "roundtrip +1.0f"
            assert np.all(np.isnan(got3.view(np.float32)[nan]))


def test_band_and_whole_box_agree_on_a_short_last_unit():
    """1200 x 50 bytes in 128 x 16 boxes: 10 boxes to a row of the sweep, so
    the second unit of each row holds 2 boxes of 8 (the last one 48 bytes
    wide), and the last band of the sweep is partial; the destination is
    2048 bytes wide, so the unit's 6 missing boxes would be visible."""
    say("band vs whole box: short last unit")
    assert -(-1200 // 128) % 8 == 2
    src = dev_bytes(1200 * 50, 5)
    dst_a = dev_bytes(2048 * 64, 6)
    dst_b = dst_a.clone()
    ms = T.tmap_encode("u8", 2, src.data_ptr(), [1200, 50], [1200], [128, 16], None, (3, 4, 3))
    n = T.tmap_sweep_tiles(ms)
    for dst in (dst_a, dst_b):
        md = T.tmap_encode("u8", 2, dst.data_ptr(), [2048, 64], [2048], [128, 16], None, (3, 4, 3))
        T.tmap_roundtrip(ms, md, None, n, flags=T.FLAG_BAND if dst is dst_a else T.FLAG_WHOLE_BOX)
        check_ok()
    assert T.tmap_band_boxes(ms, md, False, T.FLAG_BAND) == 8
    assert torch.equal(dst_a, dst_b)
    want = dev_bytes(2048 * 64, 6).cpu().numpy()
    om = Map(es=1, dims=[1200, 50], strides=[1200], box=[128, 16], swizzle=(3, 4, 3))
    omd = Map(es=1, dims=[2048, 64], strides=[2048], box=[128, 16], swizzle=(3, 4, 3))
    oracle.roundtrip(om, src.cpu().numpy(), omd, want, None, n)
    assert (mm := first_mismatch(dst_a.cpu().numpy(), want)) is None, mm


@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("flags", [T.FLAG_BAND, T.FLAG_WHOLE_BOX], ids=["band", "whole_box"])
def test_long_rings_keep_every_stage(stages, flags):
    """Few workgroups, hundreds of tiles each: every stage of the ring is
    refilled many times while the later stages' loads are still in flight,
    which is exactly what each stage's wait for its own loads must get right.
    64 MiB of u8 in 128x128 boxes with the 128-byte swizzle: load, store and
    round trip, checked against closed forms and a sample of the oracle."""
    dims, strides, box, swz = [8192, 8192], [8192], [128, 128], (3, 4, 3)
    say(f"long rings: stages={stages} flags={flags}")
    src = dev_bytes(8192 * 8192, 41)
    ms = T.tmap_encode("u8", 2, src.data_ptr(), dims, strides, box, None, swz)
    n = T.tmap_sweep_tiles(ms)
    opts = dict(stages=stages, grid_wgs=7, flags=flags | T.FLAG_NONTEMPORAL)
    dst = torch.zeros_like(src)
    md = T.tmap_encode("u8", 2, dst.data_ptr(), dims, strides, box, None, swz)
    T.tmap_roundtrip(ms, md, None, n, **opts)
    check_ok()
    assert torch.equal(dst, src)                       # exact tiling: identity
    packed = torch.empty(n * 16384, dtype=torch.uint8, device=DEV)
    T.tmap_load_tiles(ms, None, n, packed, **opts)
    check_ok()
    om = Map(es=1, dims=dims, strides=strides, box=box, swizzle=swz)
    rng = np.random.default_rng(stages)
    tiles = np.unique(np.concatenate([[0, 1, n - 1], rng.integers(0, n, 60)]))
    corners = np.array([oracle.sweep_coords(om, int(t)) for t in tiles], np.int32)
    want = oracle.load_tiles(om, src.cpu().numpy(), corners, len(corners)).reshape(len(tiles), -1)
    got = packed.view(n, -1)[torch.from_numpy(tiles).to(DEV)].cpu().numpy()
    assert np.array_equal(got, want)
    dst.zero_()
    T.tmap_store_tiles(md, None, n, packed, **opts)
    check_ok()
    assert torch.equal(dst, src)                       # storing every image back restores the tensor


@pytest.mark.parametrize("rows", [1, 2, 4, 8, 16, 32, 64, 128])
def test_every_band_height_of_the_128_byte_swizzle(rows):
    """16384 x 520 bytes in 128 x 128 boxes with the 128-byte swizzle (3,4,3),
    whose period is 8 rows: every band height from 1 row (128 boxes to a
    unit) to a whole box (one box).  Heights under 8 rows stage bands that
    differ from a box's first band by an XOR.  Load, store and round trip
    against the oracle; the last tile row is ragged."""
    dims, strides, box, swz = [16384, 520], [16384], [128, 128], (3, 4, 3)
    say(f"band height {rows}")
    src = dev_bytes(16384 * 520, 70 + rows)
    ms = T.tmap_encode("u8", 2, src.data_ptr(), dims, strides, box, None, swz)
    assert T.tmap_band_boxes(ms, None, False, T.FLAG_BAND, rows) == 128 // rows
    n = T.tmap_sweep_tiles(ms)
    opts = dict(flags=T.FLAG_BAND | T.FLAG_NONTEMPORAL, band_rows=rows)
    om = Map(es=1, dims=dims, strides=strides, box=box, swizzle=swz)
    host = src.cpu().numpy()
    packed = torch.empty(n * 16384, dtype=torch.uint8, device=DEV)
    T.tmap_load_tiles(ms, None, n, packed, **opts)
    check_ok()
    want = oracle.load_tiles(om, host, None, n)
    assert (mm := first_mismatch(packed.cpu().numpy(), want)) is None, ("load", mm)
    dst = dev_bytes(16384 * 520, 170 + rows)
    want_dst = dst.cpu().numpy().copy()
    md = T.tmap_encode("u8", 2, dst.data_ptr(), dims, strides, box, None, swz)
    T.tmap_store_tiles(md, None, n, packed, **opts)
    check_ok()
    oracle.store_tiles(om, want_dst, None, n, want)
    assert (mm := first_mismatch(dst.cpu().numpy(), want_dst)) is None, ("store", mm)
    dst2 = dev_bytes(16384 * 520, 270 + rows)
    md2 = T.tmap_encode("u8", 2, dst2.data_ptr(), dims, strides, box, None, swz)
    T.tmap_roundtrip(ms, md2, None, n, **opts)
    check_ok()
    assert torch.equal(dst2, src)                      # every byte is inside some box


def test_band_rows_that_do_not_fit_are_rejected():
    """An explicit band height that the box, the swizzle or the sweep cannot
    take is an argument error on the band schedule (no launch happens), and
    is ignored where the band schedule does not apply."""
    say("band rows rejected")
    t = torch.zeros(4096 * 256, dtype=torch.uint8, device=DEV)
    m = T.tmap_encode("u8", 2, t.data_ptr(), [4096, 256], [4096], [128, 128], None, (3, 4, 3))
    n = T.tmap_sweep_tiles(m)
    packed = torch.empty(n * 16384, dtype=torch.uint8, device=DEV)
    for rows in (3, 256, 1):     # not a power of two; taller than the box; a unit wider than the row of the sweep
        with pytest.raises(T.TmapError) as e:
            T.tmap_load_tiles(m, None, n, packed, flags=T.FLAG_BAND, band_rows=rows)
        assert e.value.status == T.INVALID_VALUE
    # whole boxes ignore it
    T.tmap_load_tiles(m, None, n, packed, flags=T.FLAG_WHOLE_BOX, band_rows=3)
    check_ok()
    # a 64-byte box row with the (3,4,3) swizzle: its 128-element blocks span
    # two rows, so a one-row band is not mapped onto itself
    m64 = T.tmap_encode("u8", 2, t.data_ptr(), [4096, 256], [4096], [64, 128], None, (3, 4, 3))
    n64 = T.tmap_sweep_tiles(m64)
    assert T.tmap_band_boxes(m64, None, False, T.FLAG_BAND, 1) == 0
    assert T.tmap_band_boxes(m64, None, False, T.FLAG_BAND, 4) == 64
    with pytest.raises(T.TmapError):
        T.tmap_load_tiles(m64, None, n64, packed, flags=T.FLAG_BAND, band_rows=1)


def _lean_case(rng):
    """A rank-2 band sweep whose dimension-0 rows are whole 16-byte chunks
    (the case the lean band kernels take): ragged in boxes both ways."""
    while True:
        es = int(rng.choice([1, 2, 4, 8]))
        rc = int(rng.choice([4, 8, 16, 32]))
        box0 = rc * 16 // es
        if box0 <= 256:
            break
    k = 16 // es
    box1 = int(rng.choice([16, 32, 64, 128]))
    while box0 * es * box1 > 65536:
        box1 //= 2
    want_rows = int(rng.choice([0, 0, 1, 2, 4, 8, 16, 32]))
    while want_rows > box1 or want_rows * rc > 1024:
        want_rows //= 2
    rows = want_rows or 2
    g = 1024 // (rows * rc)
    tiles0 = int(rng.integers(g, 3 * g + 3))
    dims0 = tiles0 * box0 - k * int(rng.integers(0, box0 // k))
    dims1 = int(rng.integers(1, 3 * box1 + 2))
    return es, [dims0, dims1], [box0, box1], _swizzle(rng, es, box0, box1, rows), want_rows


@pytest.mark.parametrize("chunk", range(4))
def test_band_kernel_random_sweeps(chunk):
    """Rank-2 band sweeps with whole-chunk rows run the band kernel (the plan
    says so); load, store, round trip into a destination of another size and
    pitch (also whole-chunk rows), and for fp32 the +1.0f round trip, each
    against the oracle, over ring depths 1..4, groups, grids, regions, cache
    hints and the poison debug flag."""
    rng = np.random.default_rng(7300 + chunk)
    for i in range(24):
        es, dims, box, swz, rows = _lean_case(rng)
        strides, alloc = _strides(rng, dims, es)
        opts = _opts(rng, rows)
        opts["flags"] |= int(rng.choice([0, 0, T.FLAG_DEBUG_POISON, T.FLAG_CACHED_PACKED]))
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        src = dev_bytes(alloc, int(rng.integers(1 << 30)))
        m = T.tmap_encode(DT[es], 2, src.data_ptr(), dims, strides, box, None, swz)
        n = T.tmap_sweep_tiles(m)
        bb = T.tmap_box_bytes(m)
        say(f"band kernel {chunk}/{i}: es={es} dims={dims} strides={strides} box={box} swz={swz} n={n} {opts}")
        for direction in ("load", "store"):
            p = T.tmap_plan_launch(direction, m, None, False, n, **opts)
            assert p["variant"] == "band", (direction, p)
        host = src.cpu().numpy()
        packed = torch.empty(n * bb, dtype=torch.uint8, device=DEV)
        T.tmap_load_tiles(m, None, n, packed, **opts)
        check_ok()
        want = oracle.load_tiles(om, host, None, n)
        assert (mm := first_mismatch(packed.cpu().numpy(), want)) is None, ("load", mm)
        imgs = dev_bytes(n * bb, int(rng.integers(1 << 30)))
        dst = dev_bytes(alloc, int(rng.integers(1 << 30)))
        want_dst = dst.cpu().numpy().copy()
        T.tmap_store_tiles(T.tmap_encode(DT[es], 2, dst.data_ptr(), dims, strides, box, None, swz),
                           None, n, imgs, **opts)
        check_ok()
        oracle.store_tiles(om, want_dst, None, n, imgs.cpu().numpy())
        assert (mm := first_mismatch(dst.cpu().numpy(), want_dst)) is None, ("store", mm)
        k = 16 // es
        ddims = [max(k, (dims[0] + k * int(rng.integers(-box[0] // (2 * k), 2 * box[0] // k + 1))) // k * k),
                 max(1, dims[1] + int(rng.integers(-box[1] // 2, 2 * box[1] + 1)))]
        dstrides, dalloc = _strides(rng, ddims, es)
        dst2 = dev_bytes(dalloc, int(rng.integers(1 << 30)))
        want2 = dst2.cpu().numpy().copy()
        md = T.tmap_encode(DT[es], 2, dst2.data_ptr(), ddims, dstrides, box, None, swz)
        assert T.tmap_plan_launch("roundtrip", m, md, False, n, **opts)["variant"] == "band"
        T.tmap_roundtrip(m, md, None, n, **opts)
        check_ok()
        omd = Map(es=es, dims=ddims, strides=dstrides, box=box, swizzle=swz)
        oracle.roundtrip(om, host, omd, want2, None, n)
        assert (mm := first_mismatch(dst2.cpu().numpy(), want2)) is None, ("roundtrip", ddims, mm)
        if es == 4:
            dst3 = dev_bytes(dalloc, int(rng.integers(1 << 30)))
            want3 = dst3.cpu().numpy().copy()
            md3 = T.tmap_encode("f32", 2, dst3.data_ptr(), ddims, dstrides, box, None, swz)
            T.tmap_roundtrip_add_f32(m, md3, None, n, 1.0, **opts)
            check_ok()
            oracle.roundtrip_add_f32(om, host, omd, want3, None, n, 1.0)
            got3 = dst3.cpu().numpy()
            nan = np.isnan(want3.view(np.float32))
            w32, g32 = want3.view(np.uint32), got3.view(np.uint32)
            assert np.array_equal(g32[~nan], w32[~nan]), "roundtrip +1.0f"
            assert np.all(np.isnan(got3.view(np.float32)[nan]))


def test_band_kernel_budget_mismatch_times_out():
    """The band kernel's bounded wait: a byte budget 16 bytes above what is
    delivered never completes a stage; every wave gives up after spin_limit
    polls and the status reports a timeout; the next launch is correct."""
    say("budget mismatch -> TIMEOUT (band kernel)")
    src = dev_bytes(2048 * 64, 3)
    m = T.tmap_encode("u8", 2, src.data_ptr(), [2048, 64], [2048], [128, 16])
    n = T.tmap_sweep_tiles(m)
    out = torch.empty(n * 2048, dtype=torch.uint8, device=DEV)
    for stages in (1, 3):
        assert T.tmap_plan_launch("load", m, None, False, n, flags=T.FLAG_BAND, stages=stages)["variant"] == "band"
        T.tmap_load_tiles(m, None, n, out, stages=stages, group=4,
                          flags=T.FLAG_INJECT_BUDGET_MISMATCH | T.FLAG_BAND, spin_limit=2000)
        assert T.tmap_sync_status() == T.TIMEOUT
    T.tmap_load_tiles(m, None, n, out, flags=T.FLAG_BAND)
    check_ok()
    om = Map(es=1, dims=[2048, 64], strides=[2048], box=[128, 16])
    assert out.cpu().numpy().tobytes() == oracle.load_tiles(om, src.cpu().numpy(), None, n).tobytes()
