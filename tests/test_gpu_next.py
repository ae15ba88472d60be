"""GPU parity for the rows after the core path: the fused +addend round trip
and the raw 1-D bulk copy, through the C ABI, against the CPU oracle.

fp32 results are compared bit for bit; where the oracle's result is a NaN
the GPU result only has to be a NaN (payload bits of a NaN produced by an add
are the hardware's).
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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bytes(nbytes, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    n8 = (nbytes + 7) // 8
    x = torch.randint(-(2**63), 2**63 - 1, (n8,), dtype=torch.int64, generator=g, device=DEV)
    return x.view(torch.uint8)[:nbytes].contiguous()


def check_ok():
    st = T.tmap_sync_status()
    assert st == T.SUCCESS, T.tmap_status_string(st)


def same_f32(got: np.ndarray, want: np.ndarray):
    g = got.view(np.uint32)
    w = want.view(np.uint32)
    wf = want.view(np.float32)
    nan = np.isnan(wf)
    assert np.array_equal(g[~nan], w[~nan]), f"{int(np.sum(g[~nan] != w[~nan]))} fp32 words differ"
    assert np.all(np.isnan(got.view(np.float32)[nan]))


def test_plus_one_day76_matrix():
    """256x256 fp32, sixteen 64x64 boxes, +1.0f in on-chip memory, exact."""
    say("plus one: the 256x256 fp32 round-trip program")
    vals = torch.arange(256 * 256, dtype=torch.float32, device=DEV) - 30000.0
    src = vals.view(torch.uint8)
    dst = torch.zeros_like(src)
    ms = T.tmap_encode("f32", 2, src.data_ptr(), [256, 256], [1024], [64, 64])
    md = T.tmap_encode("f32", 2, dst.data_ptr(), [256, 256], [1024], [64, 64])
    n = T.tmap_sweep_tiles(ms)
    assert n == 16
    for st in (1, 2):
        dst.zero_()
        T.tmap_roundtrip_add_f32(ms, md, None, n, 1.0, stages=st)
        check_ok()
        out = dst.view(torch.float32)
        assert torch.equal(out, vals + 1.0)
        assert torch.all(out - vals == 1.0)          # off by exactly 1.0f: the store ran, after the load


@pytest.mark.parametrize("chunk", range(2))
def test_plus_addend_fuzz(chunk):
    rng = np.random.default_rng(5500 + chunk)
    for i in range(30):
        mp = inputs.random_map(rng, es_choices=(4,))
        dims, strides, box, swz = mp["dims"], mp["strides"], mp["box"], mp["swizzle"]
        if i % 5 == 2:
            n_el = int(np.prod(box))
            for mm in range(0, 2):
                if n_el % (1 << (mm + 1)) == 0:
                    swz = (1, mm, 2)          # permutes elements inside 16-byte chunks
                    break
        addend = float(rng.choice([1.0, -2.5, 1e-39, 3.0e38]))
        coords = inputs.random_corners(dims, box, int(rng.integers(1, 30)), int(rng.integers(1 << 30)))
        opts = dict(stages=int(rng.integers(1, 5)), grid_wgs=int(rng.choice([0, 1, 3])),
                    group=int(rng.choice([0, 1, 4])))
        say(f"plus addend {chunk}/{i}: dims={dims} box={box} swz={swz} addend={addend} n={len(coords)} {opts}")
        src = dev_bytes(mp["alloc_bytes"], int(rng.integers(1 << 30)))
        dst = dev_bytes(mp["alloc_bytes"], int(rng.integers(1 << 30)))
        want = dst.cpu().numpy().copy()
        ms = T.tmap_encode("f32", len(dims), src.data_ptr(), dims, strides, box, None, swz)
        md = T.tmap_encode("f32", len(dims), dst.data_ptr(), dims, strides, box, None, swz)
        T.tmap_roundtrip_add_f32(ms, md, torch.from_numpy(coords).to(DEV), len(coords), addend, **opts)
        check_ok()
        om = Map(es=4, dims=dims, strides=strides, box=box, swizzle=swz)
        oracle.roundtrip_add_f32(om, src.cpu().numpy(), om, want, coords, len(coords), addend)
        same_f32(dst.cpu().numpy(), want)


def test_plus_one_rejects_non_f32():
    t = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    m = T.tmap_encode("u32", 2, t.data_ptr(), [16, 64], [64], [16, 16])
    with pytest.raises(T.TmapError) as e:
        T.tmap_roundtrip_add_f32(m, m, None, T.tmap_sweep_tiles(m), 1.0)
    assert e.value.status == T.INVALID_VALUE


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 16384, 16384 * 3 + 48, 1 << 20, (5 << 20) + 1024 * 16 + 16])
def test_bulk_copy_sizes(nbytes):
    say(f"bulk copy {nbytes} bytes")
    src = dev_bytes(nbytes + 64, 11)
    dst = dev_bytes(nbytes + 64, 12)
    want = dst.cpu().numpy().copy()
    T.tmap_bulk_copy(dst, src, nbytes)
    check_ok()
    oracle.bulk_copy(want, src.cpu().numpy(), nbytes)
    got = dst.cpu().numpy()
    assert got.tobytes() == want.tobytes()          # the 64 bytes past the range are untouched


@pytest.mark.parametrize("nbytes", [(16 << 20) - 16, 16 << 20, (16 << 20) + 37 * 65536 + 4096 + 16,
                                    (256 << 20) + 37 * 65536 + 4096 + 16])
def test_bulk_copy_row_view_and_remainder(nbytes):
    """From 16 MiB the bulk copy moves the whole 64 KiB rows as a 2-D sweep
    on the band schedule (here with a short last row of boxes) and the rest
    in 16 KiB tiles; every byte matches the oracle and the bytes past the
    range stay untouched."""
    say(f"bulk copy {nbytes} bytes (row view)")
    src = dev_bytes(nbytes + 64, 13)
    dst = dev_bytes(nbytes + 64, 14)
    want = dst.cpu().numpy().copy()
    T.tmap_bulk_copy(dst, src, nbytes)
    check_ok()
    oracle.bulk_copy(want, src.cpu().numpy(), nbytes)
    got = dst.cpu().numpy()
    assert np.array_equal(got, want), int(np.flatnonzero(got != want)[0])


def test_bulk_copy_2gib_and_argument_rules():
    say("bulk copy 2 GiB")
    src = inputs.device_bytes(inputs.WORKLOADS["sweep2g_u8"], DEV)
    dst = torch.empty_like(src)
    T.tmap_bulk_copy(dst, src, src.numel())
    check_ok()
    assert torch.equal(dst, src)
    for bad in (lambda: T.tmap_bulk_copy(dst.data_ptr() + 8, src, 64),
                lambda: T.tmap_bulk_copy(dst, src, 24),
                lambda: T.tmap_bulk_copy(src.data_ptr() + 64, src, 4096)):
        with pytest.raises(T.TmapError) as e:
            bad()
        assert e.value.status == T.INVALID_VALUE
    T.tmap_bulk_copy(dst, src, 0)
