"""Instruction selection in the built library (CPU only; our own gfx950 code).

The gfx950 code objects embedded in tiled_tensor_bulk_amd/libtmap.so are
extracted and disassembled with ROCm's llvm-objdump, and checked kernel by
kernel:
  - every kernel of the staged copy (the shared ring, wave-per-box and
    producer-wave variants) moves tile data with 16-byte direct-to-LDS
    buffer loads (`buffer_load_dwordx4 ... lds`); the thread-copy variant,
    the register path, has none;
  - the corner kernels in 4-byte lanes load from the tensor with 4-byte
    direct-to-LDS loads (`buffer_load_dword ... lds`), fetch each slot's
    row offset across lanes (`ds_bpermute_b32`) and store to the tensor in
    4-byte stores, with 1- and 2-byte accesses for the words the tensor's
    edge cuts;
  - no kernel uses a matrix instruction (there is no contraction);
  - no kernel writes through the scalar data cache (scalar stores, scalar
    atomics, scalar cache write-back): every store is a vector store.
"""
import os
import re
import shutil
import subprocess

import pytest

from tiled_tensor_bulk_amd import tmap as T

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
SCALAR_WRITE = re.compile(r"\b(s_store_|s_buffer_store|s_atomic_|s_buffer_atomic|s_dcache_wb|s_scratch_store)")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not available")
    if not os.path.exists(T.LIB_PATH):
        from tiled_tensor_bulk_amd import build
        build.build()
    d = tmp_path_factory.mktemp("isa")
    lib = d / "libtmap.so"
    shutil.copy(T.LIB_PATH, lib)
    # writes libtmap.so.<i>.<target> beside the copy, one per embedded bundle
    subprocess.run([OBJDUMP, "--offloading", str(lib)], cwd=d, check=True, capture_output=True)
    objs = sorted(p for p in os.listdir(d) if p.endswith("gfx950"))
    assert objs, "no gfx950 code object in the library"
    out = {}
    for o in objs:
        text = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(d / o)], check=True, capture_output=True,
                              text=True).stdout
        cur = None
        for line in text.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.+)>:", line)
            if m:
                cur = m.group(1)
                out[cur] = []
            elif cur is not None and line.strip():
                out[cur].append(line)
    return out


def _family(name):
    m = re.search(r"(copy|wave|thread|ws|band|corner4|corner)_kernel", name)
    return m.group(0) if m else None


def test_every_variant_is_present(kernels):
    fams = {_family(k) for k in kernels}
    assert {"copy_kernel", "wave_kernel", "thread_kernel", "ws_kernel", "band_kernel", "corner_kernel",
            "corner4_kernel"} <= fams
    assert len(kernels) >= 200


def test_staged_kernels_load_tiles_straight_into_lds(kernels):
    for name, body in kernels.items():
        fam = _family(name)
        lds_dma = sum(1 for l in body if "buffer_load_dwordx4" in l and re.search(r"\blds\b", l))
        if fam in ("copy_kernel", "wave_kernel", "ws_kernel", "band_kernel", "corner_kernel"):
            assert lds_dma > 0, name
        elif fam == "thread_kernel":
            assert lds_dma == 0, name


def test_corner4_kernels_move_4_byte_lanes(kernels):
    seen = set()
    for name, body in kernels.items():
        if _family(name) != "corner4_kernel":
            continue
        mode = int(re.search(r"corner4_kernelILi(\d)E", name).group(1))
        seen.add(mode)
        dword_dma = sum(1 for l in body if re.search(r"buffer_load_dword\s", l) and re.search(r"\blds\b", l))
        wide_dma = sum(1 for l in body if "buffer_load_dwordx4" in l and re.search(r"\blds\b", l))
        stores4 = sum(1 for l in body if re.search(r"buffer_store_dword\s", l))
        bperm = sum(1 for l in body if "ds_bpermute_b32" in l)
        assert bperm > 0, name
        # words the tensor's x edge cuts (1- and 2-byte elements) move element by element
        narrow_loads = {k for k in ("buffer_load_ubyte", "buffer_load_ushort") if any(k in l for l in body)}
        narrow_stores = {k for k in ("buffer_store_byte", "buffer_store_short") if any(k in l for l in body)}
        if mode == 1:       # store: packed images in 16-byte lanes, the tensor in 4-byte ones
            assert wide_dma > 0 and dword_dma == 0 and stores4 > 0, name
        else:               # load and round trip read the tensor in 4-byte lanes
            assert dword_dma > 0 and wide_dma == 0, name
            assert (stores4 > 0) == (mode == 2), name
        assert len(narrow_loads) == (0 if mode == 1 else 2), (name, narrow_loads)
        assert len(narrow_stores) == (0 if mode == 0 else 2), (name, narrow_stores)
    assert seen == {0, 1, 2}


def test_no_matrix_instructions(kernels):
    for name, body in kernels.items():
        assert not any("v_mfma" in l or "v_smfmac" in l for l in body), name


def test_no_scalar_cache_writes(kernels):
    for name, body in kernels.items():
        bad = [l for l in body if SCALAR_WRITE.search(l)]
        assert not bad, (name, bad[:3])
