"""Build libtmap.so (gfx950) in-tree with hipcc.

    python -m tiled_tensor_bulk_amd.build [--jobs N]

Each translation unit is compiled in parallel into tiled_tensor_bulk_amd/_build
and linked into tiled_tensor_bulk_amd/libtmap.so.  Cross-compiles without a GPU.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtmap.so")
ROOT = os.path.dirname(PKG)

SOURCES = (["tmap_host.cpp"] + [f"tmap_{m}_r{r}.hip" for m in ("load", "store", "roundtrip") for r in (2, 5)]
           + [f"tmap_band_{m}.hip" for m in ("load", "store", "roundtrip")]
           + [f"tmap_corner_{m}.hip" for m in ("load", "store", "roundtrip")]
           + [f"tmap_corner4_{m}.hip" for m in ("load", "store", "roundtrip")] + ["tmap_noalloc.hip"])
ARCH = "gfx950"


def hipcc() -> str:
    for p in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if p and os.path.exists(p):
            return p
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            # packed fp32 instructions are kept out of every device build
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


def build(jobs: int = 7, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every translation unit (or, with incremental=True, only those
    older than a source or header) and link libtmap.so."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    t0 = time.time()
    newest_hdr = max(os.path.getmtime(os.path.join(d, f)) for d in (CSRC, os.path.join(ROOT, "include"))
                     for f in os.listdir(d) if f.endswith(".h"))
    pending = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        if (incremental and os.path.exists(obj)
                and os.path.getmtime(obj) > max(newest_hdr, os.path.getmtime(os.path.join(CSRC, src)))):
            objs.append(obj)
        else:
            pending.append(src)
    running = []
    while pending or running:
        while pending and len(running) < max(1, jobs):
            src = pending.pop(0)
            obj = os.path.join(BUILD, src + ".o")
            objs.append(obj)
            cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            running.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        src, p = running.pop(0)
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature name: harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            sys.stderr.write("\n".join(lines) + "\n")
            raise RuntimeError(f"compiling {src} failed")
        if verbose and lines:
            print("\n".join(lines))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=7)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--incremental", action="store_true", help="recompile only out-of-date units")
    a = ap.parse_args()
    build(jobs=a.jobs, verbose=a.verbose, incremental=a.incremental)


if __name__ == "__main__":
    main()
