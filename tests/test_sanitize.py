"""Sanitizer leg of the CPU suite (no GPU).

1. The oracle, built into one program with the driver oracle/sanitize_check.c
   under AddressSanitizer and UndefinedBehaviorSanitizer (gcc, leak detection
   on, any report fatal), over seeded random small corpora in every mode:
   every plan, cycle, batch, padding-free row, digest and export call, with
   output buffers of exact sizes.
2. The C ABI's host-side checks (every error returned before device work),
   in a copy of the library built with host-only sanitizers (hipcc
   -Xarch_host), driven by tests/sanitize/abi_host_check.c.  Leak detection
   is off for this one: the HIP runtime's own static allocations are not the
   library's.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:verify_asan_link_order=0:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _reports(text):
    return [ln for ln in text.splitlines() if "AddressSanitizer" in ln or "runtime error" in ln
            or "LeakSanitizer" in ln]


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "sanitize_check")
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
                    os.path.join(ROOT, "oracle", "sanitize_check.c")], check=True)
    r = subprocess.run([exe, "192"], capture_output=True, text=True, timeout=600, env={**os.environ, **SAN_ENV})
    assert r.returncode == 0 and not _reports(r.stderr), r.stdout + r.stderr[-4000:]
    m = re.search(r"(\d+) cases, (\d+) with unexpected errors; (\d+) plans, (\d+) cycles, (\d+) batch calls",
                  r.stdout)
    assert m, r.stdout
    cases, failed, plans, cycles, batches = map(int, m.groups())
    assert cases == 192 and failed == 0
    assert plans >= 300 and cycles >= 600 and batches >= 1000, m.group(0)  # the calls did run


def test_abi_host_checks_under_address_and_undefined_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("hipcc / ROCm clang not available")
    src = os.path.join(ROOT, "deterministic_packing_amd", "csrc")
    lib = str(tmp_path / "libdpack_san.so")
    hips = sorted(os.path.join(src, f) for f in os.listdir(src) if f.endswith(".hip"))
    # sanitizers on the host code only (the device code is built as usual)
    subprocess.run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-I", os.path.join(ROOT, "include"), "-I", src, *hips, "-o", lib],
                   check=True, capture_output=True)
    exe = str(tmp_path / "abi_host_check")
    subprocess.run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_host_check.c"), lib,
                    "-Wl,-rpath," + str(tmp_path), "-o", exe], check=True)
    env = {**os.environ, **SAN_ENV, "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0"}
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and not _reports(r.stderr), r.stdout + r.stderr[-4000:]
    assert "abi host checks: ok" in r.stdout
