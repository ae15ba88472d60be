"""Pins for the CPU oracle (no GPU).

The oracle is only trusted because these tests tie it to things other than
itself: values the pages print (tests/golden/pages_pins.json, each cited),
closed forms (a 64x64 box at the origin of a 64x64 tensor is the tensor; a
swizzle-free exact tiling is the tensor re-blocked with reshape/transpose;
the 128-byte swizzle moves 16-byte chunk k of row r to chunk k ^ (r mod 8)),
invariants (every swizzle is a bijection and an involution of the tile;
out-of-bounds elements are exactly the zeros; load then store restores every
in-bounds byte) and an independent numpy slicing formulation (tests/npref.py)
on seeded random maps of every rank.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import Map
from tests import npref
from tiled_tensor_bulk_amd import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_pins.json")))


# ------------------------------------------------------------- page values
def test_tile_bytes_64x64_f32():
    g = GOLD["tile_bytes_f32_64x64"]
    m = Map(es=g["es"], dims=[64, 64], strides=[256], box=g["box"])
    assert oracle.box_bytes(m) == g["bytes"] == 16384


def test_smem_request_f16_strip():
    g = GOLD["smem_request_f16"]
    m = Map(es=g["es"], dims=[1792, 8448], strides=[3584], box=g["box"], swizzle=(0, 4, 3))
    assert oracle.box_bytes(m) == g["payload"]
    # the request is the payload plus one 8-byte barrier record; the budget is the payload only
    assert oracle.box_bytes(m) + g["barrier_bytes"] == g["request"]


def test_strip_decomposition_924():
    g = GOLD["strip_decomposition_f16"]
    m = Map(es=g["es"], dims=g["dims"], strides=[g["row_stride"]], box=g["box"], swizzle=(0, 4, 3))
    assert oracle.sweep_count(m) == g["tiles"] == g["strips"] * g["tiles_per_strip"]
    # every tile of the page's decomposition: block b, iteration j -> t = 7b + j,
    # rows [64b, 64b+64), columns [256j, 256j+256)
    for b in range(g["strips"]):
        for j in range(g["tiles_per_strip"]):
            assert oracle.sweep_coords(m, g["tiles_per_strip"] * b + j) == [256 * j, 64 * b]


def test_strip_example_tile():
    g = GOLD["strip_example_tile"]
    s = GOLD["strip_decomposition_f16"]
    m = Map(es=2, dims=s["dims"], strides=[s["row_stride"]], box=s["box"])
    c = oracle.sweep_coords(m, g["sweep_index"])
    assert c == g["corner"]
    assert [c[1], c[1] + m.box[1] - 1] == g["rows"]
    assert [c[0], c[0] + m.box[0] - 1] == g["cols"]


def test_roundtrip_matrix_16_tiles():
    g = GOLD["roundtrip_matrix_f32"]
    m = Map(es=g["es"], dims=g["dims"], strides=[g["row_stride"]], box=g["box"])
    assert oracle.sweep_count(m) == g["tiles"]


def test_identity_swizzle_pages():
    b, mm, s = GOLD["identity_swizzle"]["swizzle"]
    for e in range(0, 1 << 15, 7):
        assert oracle.swizzle(e, b, mm, s) == e


# ------------------------------------------------------------- swizzle
def test_swizzle_b0_identity_all_params():
    for mm in range(0, 8):
        for s in range(0, 8):
            for e in [0, 1, 5, 127, 128, 1000, 65535]:
                assert oracle.swizzle(e, 0, mm, s) == e


@pytest.mark.parametrize("b", [1, 2, 3])
def test_swizzle_bijection_involution_bruteforce(b):
    for mm in range(0, 5):
        for s in range(b, 5):
            period = 1 << (mm + b)
            for n in sorted({period, 2 * period, 4 * period, 1 << (mm + s + b)}):
                if n > 4096:
                    continue
                img = [oracle.swizzle(e, b, mm, s) for e in range(n)]
                assert sorted(img) == list(range(n)), (b, mm, s, n)
                assert all(oracle.swizzle(x, b, mm, s) == e for e, x in enumerate(img))
                # only bits [M, M+B) ever change
                mask = ((1 << b) - 1) << mm
                assert all(((x ^ e) & ~mask) == 0 for e, x in enumerate(img))
                # with S >= B some element moves once the tile spans the source bits
                if n >= 1 << (mm + s + b):
                    assert img != list(range(n))


@pytest.mark.parametrize("es,swz,width", [(1, (3, 4, 3), 128), (2, (3, 3, 3), 64), (4, (3, 2, 3), 32)])
def test_swizzle_128_byte_rows_closed_form(es, swz, width):
    """128-byte swizzle: in a box with 128-byte rows, 16-byte chunk k of row r
    lands at chunk k ^ (r mod 8) of the same row; bytes inside a chunk stay."""
    k = 16 // es
    for r in range(0, 24):
        for c in range(width):
            e = r * width + c
            want = r * width + (((c // k) ^ (r % 8)) * k) + (c % k)
            assert oracle.swizzle(e, *swz) == want


# ------------------------------------------------------------- load closed forms
def test_load_whole_tensor_box_is_identity():
    w = inputs.WORKLOADS["tile64_f32"]
    src = inputs.tensor_bytes(w)
    m = Map(es=4, dims=w.dims, strides=w.strides, box=w.box)
    packed = oracle.load_tiles(m, src, np.zeros((1, 2), np.int32), 1)
    assert packed.tobytes() == src.tobytes()


def test_load_exact_tiling_is_reblocked_tensor():
    """The page's fp16 strip decomposition, swizzle-free: the packed tiles in
    sweep order equal the matrix re-blocked as [strip][column tile][64][256]."""
    w = inputs.WORKLOADS["strips_f16"]
    src = inputs.tensor_bytes(w)
    m = Map(es=2, dims=w.dims, strides=w.strides, box=w.box, swizzle=w.swizzle)
    n = oracle.sweep_count(m)
    packed = oracle.load_tiles(m, src, None, n)
    mat = src.view(np.uint16).reshape(8448, 1792)
    want = mat.reshape(132, 64, 7, 256).transpose(0, 2, 1, 3).reshape(-1)
    assert np.array_equal(packed.view(np.uint16), want)


def test_coordinate_order_innermost_first():
    """Corner (x, y) reads rows y.. and columns x..; the swapped corner reads
    the transposed block position."""
    h = w_ = 256
    mat = (np.arange(h * w_, dtype=np.uint32) + 1).reshape(h, w_)
    m = Map(es=4, dims=[w_, h], strides=[w_ * 4], box=[64, 64])
    for (x, y) in [(64, 128), (128, 64), (192, 0)]:
        got = oracle.load_tiles(m, mat.view(np.uint8).reshape(-1), np.array([[x, y]], np.int32), 1)
        assert np.array_equal(got.view(np.uint32).reshape(64, 64), mat[y:y + 64, x:x + 64])
        swapped = oracle.load_tiles(m, mat.view(np.uint8).reshape(-1), np.array([[y, x]], np.int32), 1)
        assert np.array_equal(swapped.view(np.uint32).reshape(64, 64), mat[x:x + 64, y:y + 64])
        assert not np.array_equal(got, swapped)


def test_position_values_name_their_source():
    """Each element holds its own linear index + 1; a loaded element must hold
    the index of the element its box position names, or 0 out of bounds."""
    dims, box, swz = [40, 24, 3], [16, 8, 2], (2, 2, 2)
    n = int(np.prod(dims))
    buf = (np.arange(n, dtype=np.uint32) + 1).view(np.uint8)
    m = Map(es=4, dims=dims, strides=[160, 160 * 24], box=box, swizzle=swz)
    corners = np.array([[-5, 20, 1], [30, -3, 2], [0, 0, 0], [8, 16, -1]], np.int32)
    packed = oracle.load_tiles(m, buf, corners, len(corners)).view(np.uint32).reshape(len(corners), -1)
    for t, c in enumerate(corners):
        for e in range(int(np.prod(box))):
            i0, i1, i2 = e % 16, (e // 16) % 8, e // 128
            g = (c[0] + i0, c[1] + i1, c[2] + i2)
            inb = all(0 <= g[d] < dims[d] for d in range(3))
            want = (g[0] + 40 * g[1] + 40 * 24 * g[2] + 1) if inb else 0
            assert packed[t, oracle.swizzle(e, *swz)] == want


def test_oob_zero_set_is_exactly_out_of_bounds():
    rng = np.random.default_rng(11)
    dims, box = [48, 20], [32, 8]
    buf = rng.integers(1, 2**16, size=48 * 20, dtype=np.uint16).view(np.uint8)  # no zero elements
    m = Map(es=2, dims=dims, strides=[96], box=box)
    corners = np.array([[-32, -8], [48, 20], [-31, -7], [40, 15], [-5, 3], [16, 12]], np.int32)
    packed = oracle.load_tiles(m, buf, corners, len(corners)).view(np.uint16).reshape(len(corners), 8, 32)
    for t, c in enumerate(corners):
        mask = npref.inbounds_mask(2, dims, box, c)
        assert np.array_equal(packed[t] != 0, mask)
    assert not packed[0].any() and not packed[1].any()       # wholly outside: all zero


def test_oob_before_the_base_and_past_the_row_is_zero():
    """The tensor sits inside a larger buffer whose bytes before its base and
    in its row padding are nonzero: elements at coordinate -1 (one element
    before the base in the innermost dimension) and past dims_0 (the padding)
    must still load as zero, and match the independent numpy formulation."""
    rng = np.random.default_rng(12)
    es, dims, pitch, box = 2, [40, 12], 96, [16, 4]
    prefix = 64
    big = rng.integers(1, 256, size=prefix + pitch * dims[1] + 64, dtype=np.uint8)  # nothing is zero
    src = big[prefix:]
    m = Map(es=es, dims=dims, strides=[pitch], box=box, swizzle=(1, 3, 1))
    corners = np.array([[-1, 0], [-3, -1], [-1, -3], [30, 9], [-15, 5], [25, -2], [38, 11]], np.int32)
    got = oracle.load_tiles(m, src, corners, len(corners))
    want = npref.load_tiles(src, es, dims, [pitch], box, (1, 3, 1), corners)
    assert np.array_equal(got, want)
    inv = npref.perm(int(np.prod(box)), (1, 3, 1))
    tiles = got.view(np.uint16).reshape(len(corners), -1)
    for t, c in enumerate(corners):
        mask = npref.inbounds_mask(es, dims, box, c).reshape(-1)
        assert np.array_equal(tiles[t, inv] != 0, mask)


def test_roundtrip_between_layouts_matches_numpy():
    """A round trip from one layout into another (different dims and pitch,
    same element size, box and swizzle), over corners in, across and outside
    both tensors, equals loading each box from the source and storing it
    through the destination in tile order, in the numpy formulation."""
    rng = np.random.default_rng(13)
    es, box, swz = 4, [8, 4, 2], (2, 2, 2)
    sdims, sstr = [37, 9, 3], [160, 160 * 9]
    ddims, dstr = [29, 12, 2], [128, 128 * 12]
    src = rng.integers(0, 256, size=sstr[1] * sdims[2], dtype=np.uint8)
    dst0 = rng.integers(0, 256, size=dstr[1] * ddims[2], dtype=np.uint8)
    corners = inputs.random_corners([max(a, b) for a, b in zip(sdims, ddims)], box, 60, seed=14)
    sm = Map(es=es, dims=sdims, strides=sstr, box=box, swizzle=swz)
    dm = Map(es=es, dims=ddims, strides=dstr, box=box, swizzle=swz)
    got = dst0.copy()
    oracle.roundtrip(sm, src, dm, got, corners, len(corners))
    want = dst0.copy()
    for c in corners:
        tile = npref.load_tiles(src, es, sdims, sstr, box, swz, c[None, :])
        npref.store_tiles(want, es, ddims, dstr, box, swz, c[None, :], tile)
    assert np.array_equal(got, want)
    assert not np.array_equal(got, dst0)


# ------------------------------------------------------------- store / round trip
def test_store_of_load_restores_sweep():
    w = inputs.WORKLOADS["ragged_bf16"]
    small = Map(es=2, dims=[200, 130], strides=[400], box=[64, 64], swizzle=(3, 3, 3))
    src = inputs.tensor_bytes(w, nbytes=130 * 400)
    n = oracle.sweep_count(small)
    assert n == 4 * 3
    packed = oracle.load_tiles(small, src, None, n)
    dst = inputs.sentinel_bytes(src.size, 7)
    oracle.store_tiles(small, dst, None, n, packed)
    assert dst.tobytes() == src.tobytes()


def test_roundtrip_random_corners_union_of_footprints():
    """Round trip through random corners: in-bounds bytes inside some box equal
    the source; every other byte (padding included) keeps the sentinel."""
    dims, box = [21, 9, 5], [8, 4, 2]
    strides = [96, 96 * 9]            # rows of 84 bytes padded to 96
    alloc = 96 * 9 * 5
    src = inputs.sentinel_bytes(alloc, 3)
    dst0 = inputs.sentinel_bytes(alloc, 4)
    corners = inputs.random_corners(dims, box, 60, seed=5)
    m = Map(es=4, dims=dims, strides=strides, box=box)
    dst = dst0.copy()
    oracle.roundtrip(m, src, m, dst, corners, len(corners))
    cover = np.zeros((5, 9, 21), dtype=bool)
    for c in corners:
        msk = npref.inbounds_mask(4, dims, box, c)
        sl = tuple(slice(max(int(c[d]), 0), min(int(c[d]) + box[d], dims[d])) for d in reversed(range(3)))
        ms = tuple(slice(max(int(c[d]), 0) - int(c[d]), min(int(c[d]) + box[d], dims[d]) - int(c[d])) for d in reversed(range(3)))
        if msk.any():
            cover[sl] |= msk[ms]
    sv = npref.tensor_view(src, 4, dims, strides)
    dv = npref.tensor_view(dst, 4, dims, strides)
    d0 = npref.tensor_view(dst0, 4, dims, strides)
    assert np.array_equal(dv[cover], sv[cover])
    assert np.array_equal(dv[~cover], d0[~cover])
    # padding bytes of every row are untouched
    rows = dst.reshape(45, 96)
    assert rows[:, 84:].tobytes() == dst0.reshape(45, 96)[:, 84:].tobytes()


def test_roundtrip_equals_store_after_load():
    rng = np.random.default_rng(21)
    for _ in range(20):
        mp = inputs.random_map(rng)
        m = Map(es=mp["es"], dims=mp["dims"], strides=mp["strides"], box=mp["box"], swizzle=mp["swizzle"])
        src = inputs.sentinel_bytes(mp["alloc_bytes"], int(rng.integers(1 << 30)))
        dst0 = inputs.sentinel_bytes(mp["alloc_bytes"], int(rng.integers(1 << 30)))
        corners = inputs.random_corners(mp["dims"], mp["box"], 12, int(rng.integers(1 << 30)))
        a = dst0.copy()
        oracle.roundtrip(m, src, m, a, corners, len(corners))
        b = dst0.copy()
        oracle.store_tiles(m, b, corners, len(corners), oracle.load_tiles(m, src, corners, len(corners)))
        assert a.tobytes() == b.tobytes()


# ------------------------------------------------------------- independent formulation
@pytest.mark.parametrize("seed", range(12))
def test_oracle_matches_numpy_slicing(seed):
    rng = np.random.default_rng(1000 + seed)
    for _ in range(6):
        mp = inputs.random_map(rng)
        es, dims, strides, box, swz = mp["es"], mp["dims"], mp["strides"], mp["box"], mp["swizzle"]
        m = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        src = inputs.sentinel_bytes(mp["alloc_bytes"], int(rng.integers(1 << 30)))
        corners = inputs.random_corners(dims, box, 16, int(rng.integers(1 << 30)))
        got = oracle.load_tiles(m, src, corners, len(corners))
        want = npref.load_tiles(src, es, dims, strides, box, swz, corners)
        assert got.tobytes() == want.tobytes(), mp
        # store: non-overlapping corners (one per box-aligned position) so order does not matter
        n_sweep = oracle.sweep_count(m)
        sc = np.array([oracle.sweep_coords(m, t) for t in range(n_sweep)], np.int32).reshape(n_sweep, len(dims))
        packed = inputs.sentinel_bytes(n_sweep * oracle.box_bytes(m), int(rng.integers(1 << 30)))
        d1 = inputs.sentinel_bytes(mp["alloc_bytes"], 99)
        d2 = d1.copy()
        oracle.store_tiles(m, d1, None, n_sweep, packed)
        npref.store_tiles(d2, es, dims, strides, box, swz, sc, packed)
        assert d1.tobytes() == d2.tobytes(), mp
        assert oracle.inb_elems(m, corners, len(corners)) == sum(
            int(npref.inbounds_mask(es, dims, box, c).sum()) for c in corners)


def test_sweep_count_matches_enumeration():
    rng = np.random.default_rng(5)
    for _ in range(30):
        mp = inputs.random_map(rng)
        m = Map(es=mp["es"], dims=mp["dims"], strides=mp["strides"], box=mp["box"])
        n = oracle.sweep_count(m)
        # brute force: every box-aligned corner whose box touches the tensor, in
        # innermost-fastest order
        import itertools
        axes = [list(range(0, mp["dims"][d], mp["box"][d])) for d in range(len(mp["dims"]))]
        want = [list(reversed(p)) for p in itertools.product(*reversed(axes))]
        assert n == len(want)
        assert [oracle.sweep_coords(m, t) for t in range(n)] == want


# ------------------------------------------------------------- validator
BASE = 0x7F0000000000


def _ok(**kw):
    p = dict(es=4, rank=2, base=BASE, dims=[64, 64], strides=[256], box=[64, 64], estrides=[1, 1],
             swizzle=(0, 0, 0))
    p.update(kw)
    return oracle.validate(p["es"], p["rank"], p["base"], p["dims"], p["strides"], p["box"],
                           p["estrides"], p["swizzle"])


def test_validator_accepts_page_examples_and_boundaries():
    r = GOLD["encode_rules"]
    assert _ok() == 0
    assert _ok(box=[r["max_box_dim"], 16], dims=[512, 64], strides=[2048]) == 0      # box 256 allowed
    assert _ok(strides=[r["stride_multiple"] * 16]) == 0
    assert _ok(es=2, dims=[1792, 8448], strides=[3584], box=[256, 64], swizzle=(0, 4, 3)) == 0
    assert _ok(rank=5, dims=[129, 65, 33, 13, 7], strides=[528, 34320, 1132560, 14723280],
               box=[32, 8, 4, 2, 1], estrides=[1] * 5) == 0
    assert _ok(es=1, dims=[65536, 32768], strides=[65536], box=[128, 128], swizzle=(3, 4, 3)) == 0
    assert _ok(es=2, dims=[16320, 16383], strides=[32640], box=[64, 64], swizzle=(3, 3, 3)) == 0


def test_validator_rejects_each_page_rule():
    r = GOLD["encode_rules"]
    assert _ok(box=[r["max_box_dim"] + 1, 1], dims=[512, 64], strides=[2048]) == 2
    assert _ok(strides=[r["stride_multiple"] * 16 + 8]) == 3
    assert _ok(base=BASE + 8) == 4
    assert _ok(rank=r["max_rank"] + 1, dims=[4] * 6, strides=[16] * 5, box=[4] * 6, estrides=[1] * 6) == 1
    assert _ok(rank=0) == 1


def test_validator_rejects_library_rules():
    assert _ok(base=0) == 5
    assert _ok(es=3) == 6
    assert _ok(dims=[0, 64]) == 7
    assert _ok(dims=[64, (1 << 31) + 1]) == 7
    assert _ok(dims=[64, 1 << 31]) == 0
    assert _ok(box=[64, 0]) == 8
    assert _ok(strides=[0]) == 9
    assert _ok(strides=[1 << 40]) == 9
    assert _ok(estrides=[1, 2]) == 10
    assert _ok(box=[6, 64]) == 11                    # 24-byte box rows
    assert _ok(box=[256, 128], dims=[512, 256], strides=[2048]) == 12   # 128 KiB box
    assert _ok(swizzle=(9, 0, 9)) == 13
    assert _ok(swizzle=(3, 2, 2)) == 14
    assert _ok(es=4, box=[4, 1], dims=[64, 64], swizzle=(3, 2, 3)) == 15
    assert _ok(rank=2, box=[4, 256], strides=[(1 << 40) - 16], dims=[64, 300]) == 16


# ------------------------------------------------------------- fused +1.0f round trip
def _as_f32(b):
    return np.ascontiguousarray(b).view(np.float32)


def test_plus_one_on_the_day76_matrix():
    """The round-trip program's matrix: 256x256 fp32, 16 boxes of 64x64, each
    element +1.0f in on-chip memory; integer-valued inputs make the result exact."""
    g = GOLD["roundtrip_matrix_f32"]
    vals = (np.arange(256 * 256, dtype=np.float32) - 30000.0)
    src = vals.view(np.uint8).copy()
    dst = np.zeros_like(src)
    m = Map(es=4, dims=g["dims"], strides=[g["row_stride"]], box=g["box"])
    n = oracle.sweep_count(m)
    assert n == g["tiles"]
    oracle.roundtrip_add_f32(m, src, m, dst, None, n, 1.0)
    assert np.array_equal(_as_f32(dst), vals + np.float32(1.0))
    assert np.all(_as_f32(dst) - vals == 1.0)          # off by exactly 1.0f, never stale


def test_plus_addend_matches_numpy_float32_including_specials():
    rng = np.random.default_rng(17)
    v = rng.standard_normal(64 * 40).astype(np.float32)
    v[:8] = np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-42, 3.4e38, np.nan], np.float32)
    src = v.view(np.uint8).copy()
    m = Map(es=4, dims=[64, 40], strides=[256], box=[32, 8], swizzle=(3, 2, 3))
    for addend in (1.0, -0.5, 1e-38, 65504.0):
        dst = np.zeros_like(src)
        oracle.roundtrip_add_f32(m, src, m, dst, None, oracle.sweep_count(m), addend)
        got, want = _as_f32(dst), v + np.float32(addend)
        fin = ~np.isnan(want)
        assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
        assert np.all(np.isnan(got[~fin]))


def test_plus_one_is_clipped_like_the_store():
    dims, box = [20, 9], [16, 4]
    v = np.arange(20 * 9, dtype=np.float32)
    src = np.zeros(9 * 96, np.uint8)
    npref.tensor_view(src, 4, dims, [96])[:] = v.reshape(9, 20).view(np.uint32)
    dst0 = inputs.sentinel_bytes(src.size, 9)
    dst = dst0.copy()
    corners = np.array([[-5, -2], [10, 7], [4, 2]], np.int32)
    m = Map(es=4, dims=dims, strides=[96], box=box)
    oracle.roundtrip_add_f32(m, src, m, dst, corners, 3, 1.0)
    plain = dst0.copy()
    oracle.roundtrip(m, src, m, plain, corners, 3)
    touched = dst != dst0
    # exactly the bytes a plain round trip rewrites are rewritten, each element + 1.0f
    assert np.array_equal(touched, plain != dst0)
    got = npref.tensor_view(dst, 4, dims, [96]).view(np.float32)
    cov = npref.tensor_view(plain, 4, dims, [96]).view(np.float32)
    w = npref.tensor_view(dst0, 4, dims, [96]).view(np.float32)
    mask = npref.tensor_view(plain, 4, dims, [96]) != npref.tensor_view(dst0, 4, dims, [96])
    assert np.array_equal(got[mask], cov[mask] + np.float32(1.0))


def test_bulk_copy_is_a_byte_range_copy():
    src = inputs.sentinel_bytes(4096, 1)
    dst = np.zeros(4096, np.uint8)
    oracle.bulk_copy(dst, src, 3008)
    assert dst[:3008].tobytes() == src[:3008].tobytes() and not dst[3008:].any()
