"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

- The oracle (oracle/engram_oracle.c) is built with -fsanitize=address,undefined
  and the oracle pins run against that build in a child process (the sanitizer
  runtime preloaded, leak checking off for the interpreter's own allocations).
- The library's host layout code (csrc/layout.cpp: prime draw, floor fit, guards,
  segment geometry) is built with g++ into a stand-alone driver
  (tests/sanitize/layout_driver.cpp) that creates, checks and destroys a few
  thousand layouts, with leak checking on.
Both builds use gcc / g++ only; nothing here runs device code.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _need(tool):
    path = shutil.which(tool)
    if path is None:
        pytest.skip(f"{tool} not available")
    return path


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc = _need("gcc")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run([gcc, "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", *SAN, "-o", str(lib), os.path.join(ROOT, "oracle", "engram_oracle.c"),
                    "-lm"], check=True)
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = dict(os.environ, ORACLE_LIB=str(lib), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (out.stdout + out.stderr)[-3000:]
    assert out.returncode == 0, tail
    assert "passed" in out.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail


def test_layout_host_code_under_asan_ubsan(tmp_path):
    gxx = _need("g++")
    if not os.path.isdir("/opt/rocm/include"):
        pytest.skip("the ROCm headers are not available")
    exe = tmp_path / "layout_driver"
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "sanitize", "layout_driver.cpp"),
                    os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd", "csrc", "layout.cpp"),
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                                  UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"))
    assert out.returncode == 0, (out.stdout + out.stderr)[-3000:]
    assert "layout driver ok" in out.stdout
