"""Copies captured in a HIP graph and replayed, and copies running at the same
time on several streams: every result matches the oracle.

A caller with a launch-bound loop of copies can capture it once and replay
it.  The library's launches are plain kernel launches on the caller's
stream; nothing in them allocates, copies or clears memory once the device's
status word exists (the first launch on a device allocates it, so one eager
launch comes before the capture).  Between replays the test rewrites the
source tensor with ordinary eager work and synchronizes, then checks the
packed images, a scattered-corner round trip and a store of the images
against the oracle, three replays in a row.
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


def fill_random(t, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    n8 = (t.numel() + 7) // 8
    x = torch.randint(-(2**63), 2**63 - 1, (n8,), dtype=torch.int64, generator=g, device=DEV)
    t.copy_(x.view(torch.uint8)[: t.numel()])


def test_graph_replays_match_the_oracle():
    # a swizzled byte sweep on the band schedule (16-row bands of 128-byte boxes)
    a_dims, a_strides, a_box, a_swz = [1200, 50], [1216], [128, 32], (3, 4, 3)
    a = torch.empty(1216 * 50, dtype=torch.uint8, device=DEV)
    b = torch.empty_like(a)
    ma = T.tmap_encode("u8", 2, a.data_ptr(), a_dims, a_strides, a_box, None, a_swz)
    mb = T.tmap_encode("u8", 2, b.data_ptr(), a_dims, a_strides, a_box, None, a_swz)
    n = T.tmap_sweep_tiles(ma)
    bb = T.tmap_box_bytes(ma)
    packed = torch.empty(n * bb, dtype=torch.uint8, device=DEV)
    oa = Map(es=1, dims=a_dims, strides=a_strides, box=a_box, swizzle=a_swz)
    # scattered 8 KiB fp32 boxes (one wave per box and workgroup, 4-byte lanes) for a round trip
    c_dims, c_strides, c_box = [300, 150], [1280], [32, 64]
    c = torch.empty(1280 * 150, dtype=torch.uint8, device=DEV)
    d = torch.empty_like(c)
    mc = T.tmap_encode("f32", 2, c.data_ptr(), c_dims, c_strides, c_box)
    md = T.tmap_encode("f32", 2, d.data_ptr(), c_dims, c_strides, c_box)
    corners = inputs.random_corners(c_dims, c_box, 200, seed=71)
    corners_dev = torch.from_numpy(corners).to(DEV)
    oc = Map(es=4, dims=c_dims, strides=c_strides, box=c_box)
    assert T.tmap_plan_launch("roundtrip", mc, md, True, len(corners))["variant"] == "corner4"
    fill_random(b, 1)
    fill_random(d, 2)

    def copies():
        T.tmap_load_tiles(ma, None, n, packed, flags=T.FLAG_BAND)
        T.tmap_roundtrip(mc, md, corners_dev, len(corners))
        T.tmap_store_tiles(mb, None, n, packed, flags=T.FLAG_BAND)

    # one eager pass first: it also allocates the device's status word
    fill_random(a, 10)
    fill_random(c, 20)
    copies()
    assert T.tmap_sync_status() == T.SUCCESS

    say("graph: capture")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            copies()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(3):
        say(f"graph: replay {rep}")
        fill_random(a, 100 + rep)
        fill_random(c, 200 + rep)
        torch.cuda.synchronize()
        host_a, host_c = a.cpu().numpy(), c.cpu().numpy()
        want_d = d.cpu().numpy().copy()
        want_b = b.cpu().numpy().copy()
        g.replay()
        torch.cuda.synchronize()
        assert T.tmap_sync_status() == T.SUCCESS
        want_packed = oracle.load_tiles(oa, host_a, None, n)
        assert np.array_equal(packed.cpu().numpy(), want_packed), ("packed", rep)
        oracle.roundtrip(oc, host_c, oc, want_d, corners, len(corners))
        assert np.array_equal(d.cpu().numpy(), want_d), ("roundtrip", rep)
        oracle.store_tiles(oa, want_b, None, n, want_packed)
        assert np.array_equal(b.cpu().numpy(), want_b), ("store", rep)
        # the replay changed what it had to: b now holds a's bytes
        assert np.array_equal(want_b.reshape(50, 1216)[:, :1200], host_a.reshape(50, 1216)[:, :1200])


def test_concurrent_streams_match_the_oracle():
    """Three streams (default priority) each repeat a different copy -- a
    band-schedule load, a wave-per-box round trip and a shared-ring store --
    with no ordering between them; every output matches the oracle and no
    readiness wait expires.  Each launch has its own LDS records, so copies on
    different streams share nothing but the device's status word."""
    a_dims, a_strides, a_box, a_swz = [1200, 50], [1216], [128, 32], (3, 4, 3)
    a = torch.empty(1216 * 50, dtype=torch.uint8, device=DEV)
    fill_random(a, 31)
    ma = T.tmap_encode("u8", 2, a.data_ptr(), a_dims, a_strides, a_box, None, a_swz)
    n = T.tmap_sweep_tiles(ma)
    packed = torch.empty(n * T.tmap_box_bytes(ma), dtype=torch.uint8, device=DEV)
    c_dims, c_strides, c_box = [300, 150], [1280], [32, 64]
    c = torch.empty(1280 * 150, dtype=torch.uint8, device=DEV)
    fill_random(c, 32)
    d = torch.empty_like(c)
    fill_random(d, 33)
    mc = T.tmap_encode("f32", 2, c.data_ptr(), c_dims, c_strides, c_box)
    md = T.tmap_encode("f32", 2, d.data_ptr(), c_dims, c_strides, c_box)
    corners = inputs.random_corners(c_dims, c_box, 300, seed=72)
    corners_dev = torch.from_numpy(corners).to(DEV)
    # images to store with the shared ring: a's own images, loaded once up front
    e = torch.empty_like(a)
    fill_random(e, 34)
    me = T.tmap_encode("u8", 2, e.data_ptr(), a_dims, a_strides, a_box, None, a_swz)
    imgs = torch.empty_like(packed)
    T.tmap_load_tiles(ma, None, n, imgs)
    assert T.tmap_sync_status() == T.SUCCESS
    want_e = e.cpu().numpy().copy()
    want_d = d.cpu().numpy().copy()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    say("concurrent streams: 3 x 20 launches")
    for _ in range(20):
        T.tmap_load_tiles(ma, None, n, packed, stream=streams[0], flags=T.FLAG_BAND)
        T.tmap_roundtrip(mc, md, corners_dev, len(corners), stream=streams[1])
        T.tmap_store_tiles(me, None, n, imgs, stream=streams[2], flags=T.FLAG_WHOLE_BOX)
    torch.cuda.synchronize()
    for st in streams:
        assert T.tmap_sync_status(st) == T.SUCCESS
    oa = Map(es=1, dims=a_dims, strides=a_strides, box=a_box, swizzle=a_swz)
    host_a = a.cpu().numpy()
    want_packed = oracle.load_tiles(oa, host_a, None, n)
    assert np.array_equal(packed.cpu().numpy(), want_packed)
    assert np.array_equal(imgs.cpu().numpy(), want_packed)
    oc = Map(es=4, dims=c_dims, strides=c_strides, box=c_box)
    oracle.roundtrip(oc, c.cpu().numpy(), oc, want_d, corners, len(corners))
    assert np.array_equal(d.cpu().numpy(), want_d)
    oracle.store_tiles(oa, want_e, None, n, want_packed)
    assert np.array_equal(e.cpu().numpy(), want_e)
