"""The pins are strong enough to catch a wrong oracle (CPU only).

Each mutant is a copy of oracle/oracle.c with one plausible mistake planted:
a dropped term, a wrong sign, bound or index, a transposed operand, a missed
step.  tests/test_oracle_pins.py, which pins the oracle to the pages' worked
values, closed forms, invariants and an independent numpy formulation, is run
against each mutant and must fail.  The unmutated source, through the same
harness, must pass.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "oracle.c")).read()

# (name, text in oracle.c, planted replacement); the first occurrence is replaced
MUTANTS = [
    ("swizzle_target_bits", "return e ^ (field << (uint64_t)m);", "return e ^ (field << (uint64_t)(m + 1));"),
    ("swizzle_source_bits", "field = (e >> (uint64_t)(m + s))", "field = (e >> (uint64_t)s)"),
    ("swizzle_field_width", "((1ull << (uint64_t)b) - 1ull)", "((1ull << (uint64_t)(b - 1)) - 1ull)"),
    ("validator_box_limit", "if (box[d] > 256u) return OR_BOX_MAX;", "if (box[d] > 257u) return OR_BOX_MAX;"),
    ("validator_stride_16", "if (strides_1[d - 1] % 16u != 0) return OR_STRIDE_16;",
     "if (strides_1[d - 1] % 8u != 0) return OR_STRIDE_16;"),
    ("validator_base_16", "if (base % 16u != 0) return OR_BASE_16;", "if (base % 4u != 0) return OR_BASE_16;"),
    ("validator_rank_0", "if (rank < 1 || rank > OR_MAX_RANK) return OR_RANK;",
     "if (rank < 0 || rank > OR_MAX_RANK) return OR_RANK;"),
    ("validator_swizzle_tile", "(n_elems % (1ull << (m + b))) != 0", "(n_elems % (1ull << m)) != 0"),
    ("sweep_floor", "n *= (int64_t)((mp->dims[d] + mp->box[d] - 1) / mp->box[d]);",
     "n *= (int64_t)(mp->dims[d] / mp->box[d]);"),
    ("sweep_corner_unscaled", "coords[d] = (int32_t)((t % nt) * (int64_t)mp->box[d]);",
     "coords[d] = (int32_t)(t % nt);"),
    ("sweep_outer_fastest", "int64_t nt = (int64_t)((mp->dims[d] + mp->box[d] - 1) / mp->box[d]);",
     "int64_t nt = (int64_t)((mp->dims[mp->rank - 1 - d] + mp->box[mp->rank - 1 - d] - 1)"
     " / mp->box[mp->rank - 1 - d]);"),
    ("bounds_upper_inclusive", "(uint64_t)g >= mp->dims[d]) inb = 0;", "(uint64_t)g > mp->dims[d]) inb = 0;"),
    # (loosening only `g < 0` would be an equivalent mutant: the unsigned
    # comparison that follows rejects negative coordinates too)
    ("bounds_lower_off_by_one", "if (g < 0 || (uint64_t)g >= mp->dims[d]) inb = 0;",
     "if (g < -1 || g >= (int64_t)mp->dims[d]) inb = 0;"),
    ("box_radix_uses_dims", "int64_t i = (int64_t)(rest % mp->box[d]);", "int64_t i = (int64_t)(rest % mp->dims[d]);"),
    ("stride_index_shifted", "else o += (uint64_t)g * mp->stride[d];",
     "else o += (uint64_t)g * mp->stride[d > 1 ? d - 1 : d];"),
    ("load_unswizzled", "uint8_t *dst = tile + oracle_swizzle(e, mp->swz_b, mp->swz_m, mp->swz_s) * es;",
     "uint8_t *dst = tile + e * es;"),
    ("load_fill_nonzero", "memset(dst, 0, es);", "memset(dst, 0xFF, es);"),
    ("store_unswizzled", "tile + oracle_swizzle(e, mp->swz_b, mp->swz_m, mp->swz_s) * es, es);",
     "tile + e * es, es);"),
    ("roundtrip_stores_through_src_map", "if (store_one_tile(dst_map, dst, dst_len, c, tile_scratch)) return -1;",
     "if (store_one_tile(src_map, dst, dst_len, c, tile_scratch)) return -1;"),
    ("addend_sign", "f = f + addend;", "f = f - addend;"),
    ("bulk_copy_short", "for (i = 0; i < bytes; ++i) dst[i] = src[i];",
     "for (i = 0; i + 1 < bytes; ++i) dst[i] = src[i];"),
    ("inbounds_count_short", "for (e = 0; e < nb; ++e) total +=", "for (e = 1; e < nb; ++e) total +="),
    ("box_bytes_elements", "return box_elems(mp) * (uint64_t)mp->es;", "return box_elems(mp);"),
]


def _run_pins(src_path):
    env = dict(os.environ, TMAP_ORACLE_SRC=src_path, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


def _write(tmp_path, name, text):
    d = tmp_path / name
    d.mkdir()
    p = d / "oracle.c"
    p.write_text(text)
    return str(p)


def test_pins_kill_every_planted_mistake(tmp_path):
    jobs = {"unmutated": _write(tmp_path, "unmutated", SRC)}
    for name, old, new in MUTANTS:
        assert old in SRC, f"{name}: the text to mutate is not in oracle.c"
        jobs[name] = _write(tmp_path, name, SRC.replace(old, new, 1))
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 2)) as ex:
        results = dict(zip(jobs, ex.map(_run_pins, jobs.values())))
    rc, out = results.pop("unmutated")
    assert rc == 0, "the pins fail on the unmutated oracle:\n" + out
    survivors = [name for name, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"mutants the pins did not catch: {survivors}"
