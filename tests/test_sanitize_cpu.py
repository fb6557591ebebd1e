"""Host sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer).

* The oracle's C source is built with -fsanitize=address,undefined and every
  oracle pin (tests/test_oracle_pins.py) runs against that build in a child
  process, so any out-of-bounds access, use after free or undefined arithmetic
  in the oracle aborts the pins.
* The C ABI's validation unit (abi.cpp) is built host-only with g++ under the
  same sanitizers, with the kernel launchers replaced by recording stubs
  (tests/abi_sanitize_check.cpp), and every entry point is driven through
  valid, invalid and extreme arguments.

Both builds use the host compiler only; no GPU code is built with a sanitizer.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no host gcc")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@needs_gcc
def test_oracle_pins_under_asan_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    os.makedirs(OUT, exist_ok=True)
    so = os.path.join(OUT, "liblinattn_oracle_asan.so")
    subprocess.check_call(["gcc", *SAN, "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
                           os.path.join(ROOT, "oracle", "linattn_oracle.c"), "-o", so, "-lm"])
    env = dict(os.environ)
    env.update(LINATTN_ORACLE_LIB=so, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = res.stdout + res.stderr
    assert res.returncode == 0, log[-4000:]
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert " passed" in log


@needs_gcc
def test_abi_validation_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_sanitize_check")
    csrc = os.path.join(ROOT, "weight_recurrences_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", csrc,
                           "-I", os.path.join(ROOT, "include"), os.path.join(csrc, "abi.cpp"),
                           os.path.join(ROOT, "tests", "abi_sanitize_check.cpp"), "-o", exe])
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1"))
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all cases passed" in res.stdout
