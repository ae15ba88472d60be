"""The measurement plumbing on the CPU: the rocprofv3 summaries
(tiled_tensor_bulk_amd/profile_summary.py) computed from small synthetic
counter tables, the kernel-source stamp that ties a traffic summary to the
code it was taken on, and bench.py's lookup that reports traffic only while
that stamp matches."""
import csv
import os
import sys
import types

import pytest

from tiled_tensor_bulk_amd import inputs
from tiled_tensor_bulk_amd import profile_summary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


KERNEL = "void tmap::(anonymous namespace)::copy_kernel<2, 3, 4, 2, true>(tmap::KArgs)"
COPY = "__amd_rocclr_copyBuffer"


def test_code_only_ignores_comments_and_whitespace():
    a = "int x = 1; // one\n/* block\n comment */ int  y =\t2;"
    b = "int x = 1;\nint y = 2; // two"
    assert ps._code_only(a) == ps._code_only(b)
    assert ps._code_only('const char *s = "// not a comment";') != ps._code_only("const char *s = \"\";")
    assert ps._code_only("int x = 1;") != ps._code_only("int x = 2;")


def test_traffic_scales_each_counter_by_the_reference_copy(tmp_path):
    w = inputs.WORKLOADS["sweep2g_u8"]
    kib = w.alloc_bytes / 1024
    # the reference copy reads half of its true bytes on FETCH_SIZE and all of them on WRITE_SIZE;
    # two copy-kernel dispatches read 0.5 and 0.5 of the tensor and write all of it
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    _write_counters(fetch, [(1, COPY, "FETCH_SIZE", kib / 2), (2, KERNEL, "FETCH_SIZE", kib / 4),
                            (3, KERNEL, "FETCH_SIZE", kib / 4), (4, COPY, "FETCH_SIZE", 3.0)])
    _write_counters(write, [(1, COPY, "WRITE_SIZE", kib), (2, KERNEL, "WRITE_SIZE", kib),
                            (3, KERNEL, "WRITE_SIZE", kib)])
    out = tmp_path / "t.txt"
    ps.cmd_traffic(types.SimpleNamespace(workload="sweep2g_u8", op="roundtrip", fetch=str(fetch), write=str(write),
                                         out=str(out), cmd="x"))
    kv = dict(line.split(": ", 1) for line in open(out) if not line.startswith("#"))
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    # 0.25 of the tensor read per dispatch (raw) x 2 = a half; plus one whole tensor written
    assert int(kv["hbm_read_bytes_per_launch"]) == pytest.approx(w.alloc_bytes / 2, rel=1e-9)
    assert int(kv["hbm_bytes_per_launch"]) == pytest.approx(1.5 * w.alloc_bytes, rel=1e-9)
    assert kv["kernel_source_sha"].strip() == ps.kernel_source_sha()


def test_counters_average_the_copy_kernel_dispatches_only(tmp_path):
    path = tmp_path / "c.csv"
    _write_counters(path, [(1, KERNEL, "SQ_WAVES", 100), (1, KERNEL, "SQ_WAVES", 28),
                           (2, KERNEL, "SQ_WAVES", 128), (3, COPY, "SQ_WAVES", 9999),
                           (1, KERNEL, "SQ_LDS_BANK_CONFLICT", 0), (2, KERNEL, "SQ_LDS_BANK_CONFLICT", 4)])
    out = tmp_path / "c.txt"
    ps.cmd_counters(types.SimpleNamespace(csv=str(path), workload="w", op="load", out=str(out), cmd="x"))
    kv = dict(line.strip().split(": ", 1) for line in open(out) if not line.startswith("#"))
    assert kv["SQ_WAVES"] == "128" and kv["SQ_LDS_BANK_CONFLICT"] == "2"


def test_summaries_keep_the_timed_kernel_only(tmp_path):
    """A store's bench fills its packed images with one load before the
    timed stores: the summaries average the kernel dispatched most often."""
    load = KERNEL.replace("<2,", "<0,")
    path = tmp_path / "c.csv"
    _write_counters(path, [(1, load, "SQ_WAVES", 5000), (2, KERNEL, "SQ_WAVES", 100), (3, KERNEL, "SQ_WAVES", 300)])
    out = tmp_path / "c.txt"
    ps.cmd_counters(types.SimpleNamespace(csv=str(path), workload="w", op="store", out=str(out), cmd="x"))
    kv = dict(line.strip().split(": ", 1) for line in open(out) if not line.startswith("#"))
    assert kv["SQ_WAVES"] == "200"
    assert ps.timed_kernel([load, KERNEL, KERNEL, COPY]) == KERNEL


def test_copy_kernel_names_cover_every_variant():
    for k in ("copy_kernel<0, 1, 8, 5, false>", "wave_kernel<1, 1, 8, 5>", "thread_kernel<2, 4, 2>",
              "ws_kernel<0, 2, 4, 2>", "band_kernel<2, 3, true, true, false>",
              "corner_kernel<2, 8, 5, false, false, false, true>",
              "corner4_kernel<1, 8, 5, false, true, false, false>"):
        assert ps.is_copy_kernel(f"void tmap::(anonymous namespace)::{k}(tmap::KArgs)")
    assert not ps.is_copy_kernel("__amd_rocclr_copyBuffer")
    full = "void tmap::(anonymous namespace)::{}(tmap::KArgs)".format
    assert ps.short(full("band_kernel<2, 3, true, true, true>")) == \
        "tmap band_kernel<roundtrip, stages=3, nt loads=true, nt stores=true, +addend>"
    assert ps.short(full("corner_kernel<0, 8, 5, false, true, false, false>")) == \
        "tmap corner_kernel<load, nslot=8, dims=5, nt loads=false, nt stores=true>"
    assert ps.short(full("thread_kernel<0, 8, 2>")) == "tmap thread_kernel<load, nslot=8, dims=2>"
    assert ps.short(full("ws_kernel<1, 2, 4, 5>")) == "tmap ws_kernel<store, stages=2, nslot=4, dims=5>"
    assert ps.short(full("corner_kernel<2, 8, 5, false, false, false, true>")) == \
        "tmap corner_kernel<roundtrip, nslot=8, dims=5, nt loads=false, nt stores=false, same maps>"
    assert ps.short(full("corner4_kernel<2, 8, 5, false, false, true, true>")) == \
        "tmap corner4_kernel<roundtrip, nslot=8, dims=5, nt loads=false, nt stores=false, +addend, same maps>"


def test_bench_reports_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    # a copy of the repository layout bench.py reads: profiles/ beside bench.py
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.traffic_from_profile("sweep2g_u8", "roundtrip") is None          # no summary at all
    text = "# x\nkernel_source_sha: {}\nhbm_bytes_per_launch: 4295000000\n"
    path = root / "profiles" / "traffic_sweep2g_u8_roundtrip.txt"
    path.write_text(text.format(ps.kernel_source_sha()))
    assert bench.traffic_from_profile("sweep2g_u8", "roundtrip") == 4295000000.0
    path.write_text(text.format("0000000000000000"))                               # taken on other sources
    assert bench.traffic_from_profile("sweep2g_u8", "roundtrip") is None


def test_committed_traffic_summaries_are_well_formed():
    d = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(d) if n.startswith("traffic_") and n.endswith(".txt")]
    assert len(names) >= 12
    for n in names:
        kv = dict(line.strip().split(": ", 1) for line in open(os.path.join(d, n)) if ": " in line
                  and not line.startswith("#"))
        read, wrote = int(kv["hbm_read_bytes_per_launch"]), int(kv["hbm_write_bytes_per_launch"])
        assert int(kv["hbm_bytes_per_launch"]) == pytest.approx(read + wrote, abs=2), n
        assert float(kv["fetch_scale"]) > 0 and float(kv["write_scale"]) > 0, n
        assert len(kv["kernel_source_sha"]) == 16, n
