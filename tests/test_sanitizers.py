"""CPU runs of the host code under AddressSanitizer and UBSan.

- The C oracle (gcc -fsanitize=address,undefined) on a ragged grouped shape
  with an initial state and a state trace, cross-checked against its own
  decode step token by token (tests/sanitize/oracle_check.c).
- The C ABI's host side: ssd_api.hip (every argument check and the workspace
  layout) built with the sanitizers on the host pass only, linked against the
  built libssd.so for the launch code, driven through every entry point's
  failing checks and the workspace queries on extreme shapes
  (tests/sanitize/abi_check.cpp). No GPU is touched: every call returns before
  anything is enqueued.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
LIBDIR = os.path.join(ROOT, "ssd_sequence_mixing_amd")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout[-2000:]}\n{p.stderr[-4000:]}"
    return p


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-std=c11", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", os.path.join(HERE, "oracle_check.c"),
          os.path.join(ROOT, "oracle", "ssd_oracle.c"), "-o", exe, "-lm"])
    out = _run([exe], env=SAN_ENV).stdout
    assert "step vs forward" in out


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libssd.so")):
        pytest.skip("libssd.so is not built")
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(LIBDIR, "csrc")]
    # sanitizers on the host pass only (the device code of ssd_api.hip is two fill kernels)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "abi_check.o")
    exe = str(tmp_path / "abi_check")
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", *inc,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
          "-c", os.path.join(LIBDIR, "csrc", "ssd_api.hip"), "-o", api])
    _run([hipcc, "--offload-host-only", "-O1", "-g", "-std=c++17", *inc, *san,
          "-c", os.path.join(HERE, "abi_check.cpp"), "-o", drv])
    _run([hipcc, "--offload-arch=gfx950", *san, drv, api, "-L" + LIBDIR, "-lssd",
          "-Wl,-rpath," + LIBDIR, "-o", exe])
    # leak checking off: the HIP runtime's own start-up allocations are not ours
    env = dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    out = _run([exe], env=env).stdout
    assert "abi checks passed" in out
