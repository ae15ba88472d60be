"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The CPU oracle and the host half of libtmap (encode, queries, schedule
choice, launch planning, argument checks, the device gate) are compiled with
gcc/g++ and -fsanitize=address,undefined, and driven over seeded random and
arbitrary parameters by tests/sanitize/*_driver.*: any out-of-bounds access,
use after free, signed overflow, oversized shift or misaligned access stops
the driver with a report.  No device code is built here; the kernel
launchers are stubbed, and with no GPU every copy stops at the device gate.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def _run(exe, tmp_path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], cwd=tmp_path, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-std=c11", *SAN, "-o", exe, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")],
                   check=True, capture_output=True)
    assert "maps exercised" in _run(exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"),
                    reason="g++ or the HIP runtime library not available")
@pytest.mark.skipif(_has_gpu(), reason="drives the host half on a machine without a GPU")
def test_host_half_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
                    "-I" + os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tiled_tensor_bulk_amd", "csrc", "tmap_host.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe],
                   check=True, capture_output=True)
    assert "0 unexpected results" in _run(exe, tmp_path)
