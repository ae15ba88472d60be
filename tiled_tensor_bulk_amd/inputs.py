"""Seeded synthetic workloads for the tiled bulk copy.

This module holds only workload descriptions and seeded random generators.
It computes nothing the copy computes (no tile counts, no addresses, no
swizzle, no bounds), so the HIP path and the CPU oracle can both take their
inputs from it without sharing any of the method's arithmetic.

Shapes follow the pages' examples:
  * a 64x64 fp32 tile of 16384 bytes ("Day 76: TMA", "An exact round trip"),
  * a row-major fp16 matrix cut into 64x256 boxes walked as 132 row strips of
    7 column tiles with the identity swizzle (0,4,3) ("Understanding TMA loads
    in CuTe DSL", "The work assigned to each block"),
and three larger synthetic cases: a ragged bf16 sweep with a 128-byte XOR
swizzle, a padded 5-D fp32 tensor read at random (partly out-of-bounds)
corners and swept whole, and a 2 GiB byte tensor swept with a 128-byte
swizzle.
All dims, boxes and coordinates are innermost dimension first.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

# element size in bytes per dtype name (matches the library's dtype enum names)
ELEM_SIZE = {"u8": 1, "i8": 1, "u16": 2, "f16": 2, "bf16": 2, "u32": 4, "i32": 4,
             "f32": 4, "u64": 8, "f64": 8}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    dims: Tuple[int, ...]          # innermost first
    strides: Tuple[int, ...]       # bytes, dims 1..rank-1
    box: Tuple[int, ...]           # innermost first
    swizzle: Tuple[int, int, int]  # (B, M, S)
    coords: str                    # "sweep", "origin" or "random"
    n_random: int = 0
    stages: int = 4
    values: str = "u32"            # value recipe, see tensor_bytes()
    seed: int = 0

    @property
    def es(self) -> int:
        return ELEM_SIZE[self.dtype]

    @property
    def rank(self) -> int:
        return len(self.dims)

    @property
    def alloc_bytes(self) -> int:
        """Bytes of the backing allocation: outermost dim times its stride."""
        if self.rank == 1:
            return self.dims[0] * self.es
        return self.dims[-1] * self.strides[-1]


WORKLOADS = {
    # one 64x64 fp32 box at (0,0), no swizzle, load -> tile -> store round trip
    "tile64_f32": Workload("tile64_f32", "f32", (64, 64), (256,), (64, 64), (0, 0, 0),
                           "origin", stages=1, values="u32", seed=1),
    # fp16 8448 rows x 1792 cols, 64x256 boxes, identity swizzle (0,4,3), 2 stages
    "strips_f16": Workload("strips_f16", "f16", (1792, 8448), (3584,), (256, 64), (0, 4, 3),
                           "sweep", stages=2, values="normal_f16", seed=2),
    # bf16 16383 rows x 16320 cols, 64x64 boxes (128-byte rows), 128-byte swizzle
    "ragged_bf16": Workload("ragged_bf16", "bf16", (16320, 16383), (32640,), (64, 64), (3, 3, 3),
                            "sweep", stages=4, values="normal_bf16", seed=3),
    # 5-D fp32 (7,13,33,65,129) outermost first, innermost padded to 132 elements
    "pad5d_f32": Workload("pad5d_f32", "f32", (129, 65, 33, 13, 7),
                          (528, 528 * 65, 528 * 65 * 33, 528 * 65 * 33 * 13),
                          (32, 8, 4, 2, 1), (0, 0, 0), "random", n_random=100_000,
                          stages=4, values="u32", seed=4),
    # 2 GiB byte tensor 32768 rows x 65536 cols, 128x128 boxes, 128-byte swizzle
    "sweep2g_u8": Workload("sweep2g_u8", "u8", (65536, 32768), (65536,), (128, 128), (3, 4, 3),
                           "sweep", stages=4, values="bytes", seed=5),
    # the same padded 5-D fp32 tensor swept whole: 5 x 9 x 9 x 7 x 7 boxes,
    # ragged in every dimension but the outermost
    "pad5d_sweep_f32": Workload("pad5d_sweep_f32", "f32", (129, 65, 33, 13, 7),
                                (528, 528 * 65, 528 * 65 * 33, 528 * 65 * 33 * 13),
                                (32, 8, 4, 2, 1), (0, 0, 0), "sweep", stages=1, values="u32", seed=7),
    # the round-trip program's 64x64 fp32 boxes over a 1 GiB matrix (16384 x 16384),
    # 128-byte swizzle, for the fused +1.0f update
    "plus1_f32": Workload("plus1_f32", "f32", (16384, 16384), (65536,), (64, 64), (3, 2, 3),
                          "sweep", stages=4, values="normal_f32", seed=6),
}


def tensor_bytes(w: Workload, seed: Optional[int] = None, nbytes: Optional[int] = None) -> np.ndarray:
    """Seeded contents of the whole allocation (padding included) as uint8.

    Recipes: "u32" uniform 32-bit patterns (NaN/Inf bit patterns included),
    "normal_f16" normal(0,1) rounded to fp16 by numpy, "normal_bf16" normal(0,1)
    fp32 rounded to bf16 with round-to-nearest-even on the bit pattern,
    "bytes" uniform bytes.  Generator: numpy PCG64 seeded with `seed`.
    """
    seed = w.seed if seed is None else seed
    n = w.alloc_bytes if nbytes is None else nbytes
    rng = np.random.default_rng(seed)
    if w.values == "bytes":
        return np.frombuffer(rng.bytes(n), dtype=np.uint8).copy()
    if w.values == "u32":
        assert n % 4 == 0
        return rng.integers(0, 2**32, size=n // 4, dtype=np.uint32).view(np.uint8)
    if w.values == "normal_f16":
        assert n % 2 == 0
        return rng.standard_normal(n // 2, dtype=np.float32).astype(np.float16).view(np.uint8)
    if w.values == "normal_f32":
        assert n % 4 == 0
        return rng.standard_normal(n // 4, dtype=np.float32).view(np.uint8)
    if w.values == "normal_bf16":
        assert n % 2 == 0
        u = rng.standard_normal(n // 2, dtype=np.float32).view(np.uint32).astype(np.uint64)
        b = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        return b.view(np.uint8)
    raise ValueError(w.values)


def device_bytes(w: Workload, device, seed: Optional[int] = None, nbytes: Optional[int] = None,
                 values: Optional[str] = None):
    """Seeded contents of the allocation generated on `device` with torch's
    counter-based Philox generator (fast at gigabyte sizes).  Same recipes as
    tensor_bytes(); the values differ from the numpy ones, so a check against
    the oracle hands the oracle a host copy of these very bytes.  Returns a
    uint8 torch tensor."""
    import torch
    seed = w.seed if seed is None else seed
    n = w.alloc_bytes if nbytes is None else nbytes
    values = w.values if values is None else values
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    if values in ("bytes", "u32"):
        n8 = (n + 7) // 8
        x = torch.randint(-(2**63), 2**63 - 1, (n8,), dtype=torch.int64, generator=g, device=device)
        return x.view(torch.uint8)[:n].contiguous() if n8 * 8 != n else x.view(torch.uint8)
    if values == "normal_f16":
        assert n % 2 == 0
        return torch.randn(n // 2, generator=g, device=device, dtype=torch.float32).to(torch.float16).view(torch.uint8)
    if values == "normal_f32":
        assert n % 4 == 0
        return torch.randn(n // 4, generator=g, device=device, dtype=torch.float32).view(torch.uint8)
    if values == "normal_bf16":
        assert n % 2 == 0
        f = torch.randn(n // 2, generator=g, device=device, dtype=torch.float32)
        u = f.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
        b = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).to(torch.int32).to(torch.int16)
        return b.view(torch.uint8)
    raise ValueError(values)


def sentinel_bytes(n: int, seed: int) -> np.ndarray:
    """Seeded uniform bytes used to pre-fill destinations, so that a byte the
    copy never wrote is told apart from one it wrote."""
    return np.frombuffer(np.random.default_rng(seed).bytes(n), dtype=np.uint8).copy()


def random_corners(dims, box, n: int, seed: int) -> np.ndarray:
    """[n][rank] int32 box corners.  The first ones are fixed: every corner
    that keeps exactly one in-bounds slice per dimension (each c_d is
    -box_d+1 or dims_d-1), then all -box_d (wholly before the tensor), all
    dims_d (wholly past its end) and all 0.  The rest are uniform in
    [-box_d, dims_d] per dimension (numpy PCG64, `seed`)."""
    rank = len(dims)
    fixed = []
    for mask in range(1 << rank):
        fixed.append([(dims[d] - 1) if (mask >> d) & 1 else (-box[d] + 1) for d in range(rank)])
    fixed.append([-box[d] for d in range(rank)])
    fixed.append([dims[d] for d in range(rank)])
    fixed.append([0] * rank)
    fixed = np.array(fixed[:n], dtype=np.int64).reshape(-1, rank)
    rng = np.random.default_rng(seed)
    m = n - fixed.shape[0]
    rand = np.stack([rng.integers(-box[d], dims[d] + 1, size=m, dtype=np.int64) for d in range(rank)],
                    axis=1) if m > 0 else np.zeros((0, rank), dtype=np.int64)
    return np.ascontiguousarray(np.concatenate([fixed, rand], axis=0).astype(np.int32))


def random_map(rng: np.random.Generator, max_rank: int = 5, es_choices=(1, 2, 4, 8)):
    """A small random valid-looking map for fuzz cases: returns a dict with
    es, dims, strides (bytes, dims 1..), box, swizzle and alloc_bytes.  Rows are
    padded by a random multiple of 16 bytes; box rows are whole 16-byte chunks."""
    rank = int(rng.integers(1, max_rank + 1))
    es = int(rng.choice(es_choices))
    k = 16 // es                              # elements per 16-byte chunk
    box0 = k * int(rng.integers(1, 5))
    box = [box0] + [int(rng.integers(1, 5)) for _ in range(rank - 1)]
    dims = [int(rng.integers(1, 3 * box0 + 3))] + [int(rng.integers(1, 9)) for _ in range(rank - 1)]
    strides = []
    run = -(-(dims[0] * es) // 16) * 16 + 16 * int(rng.integers(0, 3))
    for d in range(1, rank):
        strides.append(run)
        run = run * dims[d] + 16 * int(rng.integers(0, 2))
    alloc = run if rank > 1 else dims[0] * es
    alloc = max(alloc, 16)
    n_elems = int(np.prod(box))
    swz = (0, 0, 0)
    choice = int(rng.integers(0, 3))
    if choice:
        # a swizzle whose tile period divides the box
        for _ in range(20):
            b = int(rng.integers(1, 4))
            m = int(rng.integers(0, 5))
            s = int(rng.integers(b, 5))
            if n_elems % (1 << (m + b)) == 0:
                swz = (b, m, s)
                break
    return dict(es=es, dims=dims, strides=strides, box=box, swizzle=swz, alloc_bytes=alloc)
