"""tmap_roundtrip_noalloc, the round trip that allocates nothing, called
through the C ABI: its output equals tmap_roundtrip's byte for byte (and the
oracle's) on two calls in a row, the second on a smaller input; its status
word reports a readiness timeout through tmap_sync_status and is cleared by
it; bad arguments are refused before anything is launched."""
import ctypes
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
    return torch.from_numpy(inputs.sentinel_bytes(nbytes, seed)).to(DEV)


def noalloc(src, dst, coords, n, **opts):
    """tmap_roundtrip_noalloc through the C ABI (ctypes), on torch's current stream."""
    c = None if coords is None else coords.data_ptr()
    return T.lib().tmap_roundtrip_noalloc(ctypes.byref(src), ctypes.byref(dst), c, int(n), T._opts(**opts),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def check_ok():
    st = T.tmap_sync_status()
    assert st == T.SUCCESS, T.tmap_status_string(st)


CASES = [
    # a ragged band sweep of 128 x 32-byte boxes with the 128-byte swizzle
    # (the band kernel), 24 MiB
    dict(dtype="u8", dims=[6144, 4001], strides=[6160], box=[128, 32], swz=(3, 4, 3), corners=None,
         opts=dict(flags=T.FLAG_BAND)),
    # then a smaller input: 3000 scattered 2 KiB fp32 boxes of a rank-3
    # tensor, in, across and outside it (wave per box)
    dict(dtype="f32", dims=[77, 29, 21], strides=[320, 320 * 31], box=[16, 8, 4], swz=(2, 2, 3), corners=3000,
         opts=dict()),
]


def test_noalloc_matches_the_round_trip_twice_in_a_row():
    for i, case in enumerate(CASES):
        dims, strides, box, swz = case["dims"], case["strides"], case["box"], case["swz"]
        es = inputs.ELEM_SIZE[case["dtype"]]
        alloc = dims[-1] * strides[-1]
        say(f"noalloc call {i}: {case['dtype']} dims={dims} box={box} swz={swz} corners={case['corners']}")
        src = dev_bytes(alloc, 10 + i)
        ms = T.tmap_encode(case["dtype"], len(dims), src.data_ptr(), dims, strides, box, None, swz)
        if case["corners"] is None:
            cn, coords, n = None, None, T.tmap_sweep_tiles(ms)
        else:
            cn = inputs.random_corners(dims, box, case["corners"], seed=20 + i)
            coords, n = torch.from_numpy(cn).to(DEV), len(cn)
        a = dev_bytes(alloc, 30 + i)
        b = a.clone()
        ma = T.tmap_encode(case["dtype"], len(dims), a.data_ptr(), dims, strides, box, None, swz)
        mb = T.tmap_encode(case["dtype"], len(dims), b.data_ptr(), dims, strides, box, None, swz)
        assert noalloc(ms, ma, coords, n, **case["opts"]) == T.SUCCESS, T.tmap_last_error_detail()
        check_ok()
        T.tmap_roundtrip(ms, mb, coords, n, **case["opts"])
        check_ok()
        got, ref = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]
        want = inputs.sentinel_bytes(alloc, 30 + i)
        om = Map(es=es, dims=dims, strides=strides, box=box, swizzle=swz)
        oracle.roundtrip(om, src.cpu().numpy(), om, want, cn, n)
        assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


def test_noalloc_reports_a_timeout_and_recovers():
    """A byte budget 16 bytes above what is delivered never completes a stage:
    the kernels give up after spin_limit polls and set the static status word,
    which tmap_sync_status reports and clears; the next call is correct."""
    say("noalloc: budget mismatch -> TIMEOUT, then a clean call")
    dims, strides, box = [1024, 64], [1024], [128, 16]
    src = dev_bytes(1024 * 64, 41)
    dst = dev_bytes(1024 * 64, 42)
    ms = T.tmap_encode("u8", 2, src.data_ptr(), dims, strides, box)
    md = T.tmap_encode("u8", 2, dst.data_ptr(), dims, strides, box)
    n = T.tmap_sweep_tiles(ms)
    assert noalloc(ms, md, None, n, flags=T.FLAG_INJECT_BUDGET_MISMATCH | T.FLAG_BAND, spin_limit=2000) == T.SUCCESS
    assert T.tmap_sync_status() == T.TIMEOUT
    check_ok()                                     # cleared by the read
    assert noalloc(ms, md, None, n, flags=T.FLAG_BAND) == T.SUCCESS
    check_ok()
    assert torch.equal(src, dst)


def test_noalloc_refuses_bad_arguments_before_launching():
    say("noalloc: argument checks")
    src = dev_bytes(64 * 256, 51)
    dst = dev_bytes(64 * 256, 52)
    before = dst.clone()
    ms = T.tmap_encode("f32", 2, src.data_ptr(), [64, 64], [256], [16, 16])
    md_other_box = T.tmap_encode("f32", 2, dst.data_ptr(), [64, 64], [256], [16, 8])
    md = T.tmap_encode("f32", 2, dst.data_ptr(), [64, 64], [256], [16, 16])
    n = T.tmap_sweep_tiles(ms)
    assert noalloc(ms, md_other_box, None, n) == T.INVALID_VALUE
    assert noalloc(ms, md, None, n + 1) == T.INVALID_VALUE          # a sweep needs its own tile count
    assert noalloc(ms, md, None, n, stages=5) == T.INVALID_VALUE
    assert noalloc(T.tmap_t(), md, None, n) == T.INVALID_VALUE      # never encoded
    assert noalloc(ms, md, None, 0) == T.INVALID_VALUE              # a sweep of zero tiles is not this sweep
    corners = torch.zeros((1, 2), dtype=torch.int32, device=DEV)
    assert noalloc(ms, md, corners, 0) == T.SUCCESS                 # zero explicit corners: a no-op
    check_ok()
    assert torch.equal(dst, before)
