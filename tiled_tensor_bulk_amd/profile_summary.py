"""Summaries of rocprofv3 runs for profiles/ (kernel time and HBM traffic).

    python -m tiled_tensor_bulk_amd.profile_summary stats  <kernel_stats.csv> --out FILE --cmd "..."
    python -m tiled_tensor_bulk_amd.profile_summary traffic --fetch <counter_collection.csv>
        --write <counter_collection.csv> --workload W --op OP --out FILE --cmd "..."
    python -m tiled_tensor_bulk_amd.profile_summary counters <counter_collection.csv>
        --workload W --op OP --out FILE --cmd "..."

`stats` condenses a --kernel-trace --stats kernel_stats.csv into a short
markdown table.  `traffic` turns a FETCH_SIZE run and a WRITE_SIZE run (each
in KiB per dispatch) into HBM bytes per launch of the copy kernel.  Each
counter is scaled by what it reads for the plain device-to-device copy of a
known byte count that the same benchmark process runs (torch's copy of the
whole tensor: it reads and writes exactly alloc_bytes), and the result is
stamped with the hash of the kernel sources so that bench.py reports it only
while the kernels are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _code_only(text: str) -> str:
    """The source without comments and with whitespace collapsed, so that a
    comment edit does not mark the measured kernels as changed."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_tensor_bulk_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("tmap_") and name.endswith((".h", ".hip", ".cpp")):
            h.update(name.encode())
            h.update(_code_only(open(os.path.join(csrc, name), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


_KERNEL = re.compile(r"\b(copy|wave|thread|ws|band|corner|corner4)_kernel<")


def is_copy_kernel(name: str) -> bool:
    """A dispatch of one of libtmap's copy kernels (any variant)."""
    return bool(_KERNEL.search(name))


def short(name: str) -> str:
    m = re.search(r"copy_kernel<(\d+), (\d+), (\d+), (\d+)(?:, (true|false))?>", name)
    if m:
        mode = {"0": "load", "1": "store", "2": "roundtrip"}[m.group(1)]
        sched = ", band" if m.group(5) == "true" else ""
        return f"tmap copy_kernel<{mode}, stages={m.group(2)}, nslot={m.group(3)}, dims={m.group(4)}{sched}>"
    m = re.search(r"wave_kernel<(\d+), (\d+), (\d+), (\d+)>", name)
    if m:
        mode = {"0": "load", "1": "store", "2": "roundtrip"}[m.group(1)]
        return f"tmap wave_kernel<{mode}, stages={m.group(2)}, nslot={m.group(3)}, dims={m.group(4)}>"
    m = re.search(r"band_kernel<(\d+), (\d+), (true|false), (true|false), (true|false)>", name)
    if m:
        mode = {"0": "load", "1": "store", "2": "roundtrip"}[m.group(1)]
        extra = ", +addend" if m.group(5) == "true" else ""
        return (f"tmap band_kernel<{mode}, stages={m.group(2)}, nt loads={m.group(3)}, "
                f"nt stores={m.group(4)}{extra}>")
    m = re.search(r"corner_kernel<(\d+), (\d+), (\d+), (true|false), (true|false), (true|false)(?:, (true|false))?>",
                  name)
    if m:
        mode = {"0": "load", "1": "store", "2": "roundtrip"}[m.group(1)]
        extra = (", +addend" if m.group(6) == "true" else "") + (", same maps" if m.group(7) == "true" else "")
        return (f"tmap corner_kernel<{mode}, nslot={m.group(2)}, dims={m.group(3)}, nt loads={m.group(4)}, "
                f"nt stores={m.group(5)}{extra}>")
    m = re.search(r"corner4_kernel<(\d+), (\d+), (\d+), (true|false), (true|false), (true|false), (true|false)>",
                  name)
    if m:
        mode = {"0": "load", "1": "store", "2": "roundtrip"}[m.group(1)]
        extra = (", +addend" if m.group(6) == "true" else "") + (", same maps" if m.group(7) == "true" else "")
        return (f"tmap corner4_kernel<{mode}, nslot={m.group(2)}, dims={m.group(3)}, nt loads={m.group(4)}, "
                f"nt stores={m.group(5)}{extra}>")
    m = re.search(r"thread_kernel<(\d+), (\d+), (\d+)>", name)
    if m:
        mode = {"0": "load", "1": "store", "2": "roundtrip"}[m.group(1)]
        return f"tmap thread_kernel<{mode}, nslot={m.group(2)}, dims={m.group(3)}>"
    m = re.search(r"ws_kernel<(\d+), (\d+), (\d+), (\d+)>", name)
    if m:
        mode = {"0": "load", "1": "store", "2": "roundtrip"}[m.group(1)]
        return f"tmap ws_kernel<{mode}, stages={m.group(2)}, nslot={m.group(3)}, dims={m.group(4)}>"
    if "copyBuffer" in name:
        return "hip copyBuffer (torch d2d copy)"
    return (name[:60] + "...") if len(name) > 63 else name


def cmd_stats(a):
    rows = list(csv.DictReader(open(a.csv)))
    out = ["# rocprofv3 kernel statistics", "", f"command: `{a.cmd}`", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or ""
        calls = int(r.get("Calls", 0))
        avg = float(r.get("AverageNs", 0)) / 1e3
        mn = float(r.get("MinNs", 0)) / 1e3
        mx = float(r.get("MaxNs", 0)) / 1e3
        pct = float(r.get("Percentage", 0))
        out.append(f"| {short(name)} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f}% |")
    if a.trace:
        # the bench times its last `steps` launches (after the warm-up, whose
        # first launches run while the clocks settle): average those alone
        tr = [r for r in csv.DictReader(open(a.trace)) if is_copy_kernel(r["Kernel_Name"])]
        tr.sort(key=lambda r: int(r["Start_Timestamp"]))
        last = tr[-a.last:]
        us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in last]
        if us:
            out += ["", f"copy kernel, last {len(us)} launches (the bench's timed steps): "
                        f"average {sum(us) / len(us):.1f} us, median {sorted(us)[len(us) // 2]:.1f} us"]
        if a.list:
            every = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr]
            out += ["", f"every copy-kernel launch in order ({len(every)}, us): "
                        + ", ".join(f"{x:.1f}" for x in every)]
    open(a.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def per_dispatch(path, counter):
    rows = list(csv.DictReader(open(path)))
    agg = defaultdict(float)
    names = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        agg[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return [(d, names[d], agg[d]) for d in sorted(agg)]


def timed_kernel(names):
    """The copy kernel the bench times: the one dispatched most often (a
    store's bench first fills its packed images with one load)."""
    counts = defaultdict(int)
    for n in names:
        if is_copy_kernel(n):
            counts[n] += 1
    return max(counts, key=counts.get) if counts else None


def cmd_traffic(a):
    from tiled_tensor_bulk_amd import inputs
    w = inputs.WORKLOADS[a.workload]
    known_kib = w.alloc_bytes / 1024.0                 # the reference copy reads and writes this much
    res = {}
    for counter, path in (("FETCH_SIZE", a.fetch), ("WRITE_SIZE", a.write)):
        d = per_dispatch(path, counter)
        copies = [v for (_, n, v) in d if "copyBuffer" in n and v > 0.25 * known_kib]
        timed = timed_kernel(n for (_, n, _) in d)
        kern = [v for (_, n, v) in d if n == timed]
        if not copies or not kern:
            sys.exit(f"{path}: no reference copy or copy kernel dispatches with {counter}")
        factor = known_kib / (sum(copies) / len(copies))
        res[counter] = (sum(kern) / len(kern), factor)
    fetch_kib, ff = res["FETCH_SIZE"]
    write_kib, wf = res["WRITE_SIZE"]
    hbm = (fetch_kib * ff + write_kib * wf) * 1024.0
    lines = [
        f"# HBM traffic of the copy kernel, {a.workload} {a.op} (rocprofv3 --pmc, one counter per run)",
        f"# command (FETCH_SIZE): {a.cmd}",
        f"# command (WRITE_SIZE): same with --pmc WRITE_SIZE",
        f"# scale: the same process copies the whole {w.alloc_bytes}-byte tensor with torch (hip copyBuffer);",
        f"# each counter is multiplied by known_bytes / counter_reading for that copy.",
        f"kernel_source_sha: {kernel_source_sha()}",
        f"fetch_kib_per_dispatch_raw: {fetch_kib:.1f}",
        f"fetch_scale: {ff:.4f}",
        f"write_kib_per_dispatch_raw: {write_kib:.1f}",
        f"write_scale: {wf:.4f}",
        f"hbm_read_bytes_per_launch: {fetch_kib * ff * 1024.0:.0f}",
        f"hbm_write_bytes_per_launch: {write_kib * wf * 1024.0:.0f}",
        f"hbm_bytes_per_launch: {hbm:.0f}",
    ]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_counters(a):
    rows = list(csv.DictReader(open(a.csv)))
    agg = defaultdict(float)
    disp = set()
    timed = timed_kernel({int(r["Dispatch_Id"]): r["Kernel_Name"] for r in rows}.values())
    for r in rows:
        if r["Kernel_Name"] != timed:
            continue
        disp.add(int(r["Dispatch_Id"]))
        agg[r["Counter_Name"]] += float(r["Counter_Value"])
    if not disp:
        sys.exit(f"{a.csv}: no copy kernel dispatches")
    lines = [f"# rocprofv3 counters of the copy kernel, {a.workload} {a.op}, averaged over {len(disp)} dispatches",
             f"# command: {a.cmd}",
             f"kernel_source_sha: {kernel_source_sha()}"]
    lines += [f"{k}: {v / len(disp):.0f}" for k, v in sorted(agg.items())]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--workload", required=True)
    c.add_argument("--op", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--out", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--trace", help="the run's kernel trace csv (adds the average of the last launches)")
    s.add_argument("--last", type=int, default=100)
    s.add_argument("--list", action="store_true", help="also list every copy-kernel launch duration in order")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--op", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    a = ap.parse_args()
    sys.path.insert(0, ROOT)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.what](a)


if __name__ == "__main__":
    main()
