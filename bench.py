"""Benchmark of the tiled bulk copy on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--op OP]

One step is one pass of the whole copy path over the workload: every tile
loaded from HBM into an LDS stage (swizzled, zero-filled, byte-counted) and
written back out.  The default workload is the 2 GiB byte tensor
(32768 x 65536 u8, 128x128-byte boxes, 128-byte swizzle (3,4,3), 131072 tiles)
moved by tmap_roundtrip into a second tensor: the large swizzled load/store
sweep.  Inputs are generated on the device before timing.

The default 50 untimed warm-up steps take the GPU past the first tens of
milliseconds of sustained HBM load, during which launch times swing by up to
30% as the device's clocks settle; the 100 timed steps then measure the
steady state a sustained caller sees.

Prints one JSON line: achieved GB/s (algorithmic bytes read + written per
step / step time), tiles/s, the dominant kernel's roofline (its average
launch duration: one pair of HIP events on the launch stream around the timed
launches, divided by their number; against 8 TB/s HBM), HBM traffic from the committed
rocprofv3 counter summary when it was taken on the current kernel sources,
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (read+write) and % of MI355X peak; tiles/sec"
PEAK_HBM_GBPS = 8000.0


def traffic_from_profile(workload: str, op: str):
    """Per-launch HBM bytes from profiles/traffic_<workload>_<op>.txt, if it was
    measured on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{op}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    from tiled_tensor_bulk_amd.profile_summary import kernel_source_sha
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="sweep2g_u8")
    ap.add_argument("--op", default="roundtrip", choices=["roundtrip", "load", "store", "roundtrip_add", "bulk"])
    ap.add_argument("--stages", type=int, default=0)
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--flags", type=int, default=-1,
                    help="TMAP_FLAG_* bits; default: non-temporal hints when the tensor exceeds the 256 MB MALL")
    ap.add_argument("--group", type=int, default=0)
    ap.add_argument("--regions", type=int, default=0)
    ap.add_argument("--band-rows", type=int, default=0, help="box rows per band on the band schedule")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the copy shards with no exchange step, so the "
              "whole-job rate at N GPUs is N times the one-GPU rate; run with --gpus 1.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from tiled_tensor_bulk_amd import inputs
    from tiled_tensor_bulk_amd import tmap as T

    T.lib()  # raises if the HIP library is not built
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = inputs.WORKLOADS[args.workload]
    es = w.es
    src = inputs.device_bytes(w, dev)
    ms = T.tmap_encode(w.dtype, w.rank, src.data_ptr(), w.dims, w.strides, w.box, None, w.swizzle)
    bb = T.tmap_box_bytes(ms)
    if w.coords == "sweep":
        n = T.tmap_sweep_tiles(ms)
        coords_np, coords = None, None
    elif w.coords == "origin":
        n = 1
        coords_np = np.zeros((1, w.rank), np.int32)
        coords = torch.from_numpy(coords_np).to(dev)
    else:
        coords_np = inputs.random_corners(w.dims, w.box, w.n_random, seed=w.seed * 10)
        n = len(coords_np)
        coords = torch.from_numpy(coords_np).to(dev)
    inb = T.tmap_inbounds_elems(ms, coords_np, n) * es
    if args.flags < 0:
        args.flags = T.FLAG_NONTEMPORAL if w.alloc_bytes > (256 << 20) else 0
    # 0 = the library's default for stages, grid and group
    opts = dict(stages=args.stages, grid_wgs=args.grid, flags=args.flags, group=args.group, regions=args.regions,
                band_rows=args.band_rows)

    # every launch names the stream, so that a short kernel's launch does not
    # also pay for looking up torch's current stream
    stream = torch.cuda.current_stream()
    dst = packed = None
    if args.op == "bulk":
        # raw 1-D bulk copy of the whole allocation: no map, no swizzle
        dst = torch.empty(w.alloc_bytes, dtype=torch.uint8, device=dev)
        algo_bytes = 2 * w.alloc_bytes
        n = -(-w.alloc_bytes // 16384)
        bb = 16384

        def launch():
            T.tmap_bulk_copy(dst, src, w.alloc_bytes, stream=stream, **opts)
    elif args.op == "roundtrip_add":
        dst = torch.empty(w.alloc_bytes, dtype=torch.uint8, device=dev)
        md = T.tmap_encode(w.dtype, w.rank, dst.data_ptr(), w.dims, w.strides, w.box, None, w.swizzle)
        algo_bytes = 2 * inb

        def launch():
            T.tmap_roundtrip_add_f32(ms, md, coords, n, 1.0, stream=stream, **opts)
    elif args.op == "roundtrip":
        dst = torch.empty(w.alloc_bytes, dtype=torch.uint8, device=dev)
        md = T.tmap_encode(w.dtype, w.rank, dst.data_ptr(), w.dims, w.strides, w.box, None, w.swizzle)
        algo_bytes = 2 * inb                                   # in-bounds read + in-bounds write

        def launch():
            T.tmap_roundtrip(ms, md, coords, n, stream=stream, **opts)
    elif args.op == "load":
        packed = torch.empty(n * bb, dtype=torch.uint8, device=dev)
        algo_bytes = inb + n * bb                              # in-bounds read + whole images written

        def launch():
            T.tmap_load_tiles(ms, coords, n, packed, stream=stream, **opts)
    else:
        packed = torch.empty(n * bb, dtype=torch.uint8, device=dev)
        T.tmap_load_tiles(ms, coords, n, packed, stream=stream, **opts)
        dst = torch.empty(w.alloc_bytes, dtype=torch.uint8, device=dev)
        md = T.tmap_encode(w.dtype, w.rank, dst.data_ptr(), w.dims, w.strides, w.box, None, w.swizzle)
        algo_bytes = n * bb + inb                              # whole images read + in-bounds written

        def launch():
            T.tmap_store_tiles(md, coords, n, packed, stream=stream, **opts)

    plan = None
    if args.op == "bulk":
        # the library moves ranges of 256 MiB and more as 64 KiB rows of
        # 16 x 128 8-byte boxes (the rest as rank-1 16 KiB tiles); the plan
        # of that 2-D sweep names its schedule
        schedule = "rank-1 16 KiB tiles"
        rows = w.alloc_bytes // 65536
        if w.alloc_bytes >= (256 << 20):
            mv = T.tmap_encode("u64", 2, src.data_ptr(), [8192, rows], [65536], [16, 128])
            plan = T.tmap_plan_launch("roundtrip", mv, mv, False, None, **opts)
            schedule = "64 KiB rows as 16x128 u64 boxes" + (
                f", band: {plan['band_boxes']} boxes x {plan['band_rows']} rows per stage" if plan["band_boxes"] else "")
    else:
        # the schedule the library chose for these options
        direction = {"load": "load", "store": "store"}.get(args.op, "roundtrip")
        swept = md if args.op == "store" else ms
        plan = T.tmap_plan_launch(direction, swept, md if direction == "roundtrip" else None, coords is not None,
                                  n, **opts)
        if plan["band_boxes"] and (args.flags & T.FLAG_WHOLE_BOX):
            schedule = f"whole boxes on the band kernel: {plan['band_boxes']} per stage"
        elif plan["band_boxes"]:
            schedule = f"band: {plan['band_boxes']} boxes x {plan['band_rows']} rows per stage"
        elif plan["variant"] in ("wave_per_box", "corner", "corner4"):
            schedule = "whole boxes, one wave per box" + {"corner": ", drained box held in registers",
                                                          "corner4": ", 4-byte lanes"}.get(plan["variant"], "")
        else:
            schedule = "whole boxes" + ("" if plan["variant"] == "ring" else f" ({plan['variant']})")

    kernel_name = {"ring": "copy_kernel", "wave_per_box": "wave_kernel", "thread_copy": "thread_kernel",
                   "producer_wave": "ws_kernel", "band": "band_kernel",
                   "corner": "corner_kernel", "corner4": "corner4_kernel"}[plan["variant"]] if plan else "copy_kernel"
    for _ in range(args.warmup):
        launch()
    st = T.tmap_sync_status(stream)
    if st != T.SUCCESS:
        raise RuntimeError(f"warmup failed: {T.tmap_status_string(st)}")

    # The timed region: K launches back to back on `stream`, one HIP event
    # before the first and one after the last, so that the average launch
    # duration is the events' interval over K.  No event sits between two
    # launches: each one the GPU processes costs a few microseconds of its
    # own, which would be charged to microsecond-scale kernels.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        launch()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = T.tmap_sync_status(stream)
    if st != T.SUCCESS:
        raise RuntimeError(f"timed run failed: {T.tmap_status_string(st)}")
    kern_avg_s = start.elapsed_time(end) / args.steps / 1e3
    ms_per_step = wall / args.steps * 1e3
    value = algo_bytes / (wall / args.steps) / 1e9

    # context: a plain device-to-device copy of the same byte count
    ref = torch.empty(w.alloc_bytes, dtype=torch.uint8, device=dev)
    ref.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        ref.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * w.alloc_bytes / (e0.elapsed_time(e1) / 5 / 1e3) / 1e9
    del ref

    achieved = algo_bytes / kern_avg_s / 1e9
    traffic = traffic_from_profile(args.workload, args.op)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded on device, torch Philox)",
        "config": {"workload": w.name, "op": args.op, "dims": list(w.dims), "strides": list(w.strides),
                   "box": list(w.box), "swizzle": list(w.swizzle), "tiles": n, "box_bytes": bb,
                   "schedule": schedule, "stages": args.stages or "auto", "grid_wgs": args.grid or "auto",
                   "flags": args.flags,
                   "group": args.group or "auto", "regions": args.regions or "auto",
                   "band_rows": args.band_rows or "auto", "plan": plan,
                   "algorithmic_bytes_per_step": algo_bytes},
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "tiles_per_s": round(n / (wall / args.steps), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic / kern_avg_s / 1e9, 2),
                     "kernel_ms": round(kern_avg_s * 1e3, 4),
                     "kernel": f"tmap {kernel_name} ({args.op})"},
        "reference_d2d_copy_GBps": round(copy_gbps, 1),
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.op, src, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def cpu_baseline(w, op, src, budget_s):
    """The CPU oracle (single thread, as it stands) on a bounded sample: whole
    tile rows of the sweep (slabs one box deep in the outermost dimension),
    one after another, until ~budget_s of oracle time.  Reported in the same
    algorithmic GB/s as the GPU line."""
    import numpy as np

    import oracle

    if w.coords != "sweep":
        return _cpu_baseline_corners(w, op, src, budget_s)
    if w.rank < 2:
        return None
    row_bytes = w.strides[-1] * w.box[-1]                     # one tile row of the tensor
    rows_per_chunk = 4
    total_t = 0.0
    total_bytes = 0
    tiles = 0
    chunk = 0
    n_rows = -(-w.dims[-1] // w.box[-1])
    while total_t < budget_s and chunk * rows_per_chunk < n_rows:
        r0 = chunk * rows_per_chunk
        r1 = min(n_rows, r0 + rows_per_chunk)
        lo = r0 * row_bytes
        hi = min(w.alloc_bytes, r1 * row_bytes)
        host = src[lo:hi].cpu().numpy()
        sub_rows = min(w.dims[-1], r1 * w.box[-1]) - r0 * w.box[-1]
        m = oracle.Map(es=w.es, dims=list(w.dims[:-1]) + [sub_rows], strides=w.strides, box=w.box,
                       swizzle=w.swizzle)
        nt = oracle.sweep_count(m)
        t0 = time.perf_counter()
        if op == "bulk":
            dst = np.empty_like(host)
            oracle.bulk_copy(dst, host, host.size)
            total_t += time.perf_counter() - t0
            total_bytes += 2 * host.size
            tiles += -(-host.size // 16384)
            chunk += 1
            continue
        if op == "roundtrip":
            dst = np.empty_like(host)
            oracle.roundtrip(m, host, m, dst, None, nt)
        elif op == "roundtrip_add":
            dst = np.empty_like(host)
            oracle.roundtrip_add_f32(m, host, m, dst, None, nt, 1.0)
        elif op == "load":
            oracle.load_tiles(m, host, None, nt)
        else:
            packed = oracle.load_tiles(m, host, None, nt)
            t0 = time.perf_counter()
            dst = np.empty_like(host)
            oracle.store_tiles(m, dst, None, nt, packed)
        total_t += time.perf_counter() - t0
        inb = oracle.inb_elems(m, None, nt) * w.es
        total_bytes += 2 * inb if op in ("roundtrip", "roundtrip_add") else inb + nt * oracle.box_bytes(m)
        tiles += nt
        chunk += 1
    return {"value": round(total_bytes / total_t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tiles_per_s": round(tiles / total_t, 1),
            "sample": f"{tiles} tiles ({min(n_rows, chunk * rows_per_chunk)} of {n_rows} tile rows, from the top) of {w.name}, "
                      f"{op}, {total_t:.1f} s of single-thread oracle time",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def _cpu_baseline_corners(w, op, src, budget_s):
    """The oracle on explicit corners: growing prefixes of the corner list
    (random corners) or repeats of the single box (origin), until ~budget_s
    of oracle time, in the same algorithmic GB/s as the GPU line."""
    import numpy as np

    import oracle
    from tiled_tensor_bulk_amd import inputs

    if op == "bulk":
        return None
    host = src.cpu().numpy()
    m = oracle.Map(es=w.es, dims=w.dims, strides=w.strides, box=w.box, swizzle=w.swizzle)
    if w.coords == "origin":
        all_corners = np.zeros((1, w.rank), np.int32)
    else:
        all_corners = inputs.random_corners(w.dims, w.box, w.n_random, seed=w.seed * 10)
    bb = oracle.box_bytes(m)
    dst = np.empty_like(host)
    total_t, total_bytes, tiles, start = 0.0, 0, 0, 0
    chunk = 256
    while total_t < budget_s:
        if w.coords == "origin":
            c = all_corners
        else:
            if start >= len(all_corners):
                break
            c = np.ascontiguousarray(all_corners[start:start + chunk])
            start += chunk
        n = len(c)
        inb = oracle.inb_elems(m, c, n) * w.es
        if op == "store":
            packed = oracle.load_tiles(m, host, c, n)
        t0 = time.perf_counter()
        if op == "load":
            oracle.load_tiles(m, host, c, n)
        elif op == "store":
            oracle.store_tiles(m, dst, c, n, packed)
        elif op == "roundtrip_add":
            oracle.roundtrip_add_f32(m, host, m, dst, c, n, 1.0)
        else:
            oracle.roundtrip(m, host, m, dst, c, n)
        total_t += time.perf_counter() - t0
        total_bytes += 2 * inb if op in ("roundtrip", "roundtrip_add") else inb + n * bb
        tiles += n
    what = "repeats of the one box" if w.coords == "origin" else f"the first {tiles} of its {len(all_corners)} corners"
    return {"value": round(total_bytes / total_t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tiles_per_s": round(tiles / total_t, 1),
            "sample": f"{tiles} tiles ({what}) of {w.name}, {op}, {total_t:.1f} s of single-thread oracle time",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
