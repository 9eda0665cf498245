"""Host code under the address and undefined-behaviour sanitizers (no GPU).

* The C ABI layer (sparse_attention_kv_ds_amd/csrc/api.cpp) is built with g++
  against host stand-ins for the HIP runtime and the kernel launchers
  (tests/abi_host/fake_hip.cpp) and driven through every status path of
  include/ds_indexer.h by tests/abi_host/abi_host_check.cpp: each rejected
  call must return the status the header promises and launch nothing, each
  accepted call must run exactly the expected launchers, and destroy must
  free every allocation.
* The CPU oracle (oracle/oracle.c) is built with the same sanitizers and every
  pin of tests/oracle_pins.py is run against that build, in a child Python
  with the sanitizer runtime preloaded.

Any sanitizer report fails the test (reports abort the process).
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "sparse_attention_kv_ds_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(f"{name} not available")
    return p


def test_abi_status_paths_under_sanitizers():
    _need("g++")
    with tempfile.TemporaryDirectory(prefix="abi_host_") as tmp:
        exe = os.path.join(tmp, "abi_host_check")
        cmd = ["g++", "-std=c++17", *SAN, "-w", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(TESTS, "abi_host"),
               os.path.join(CSRC, "api.cpp"), os.path.join(TESTS, "abi_host", "fake_hip.cpp"),
               os.path.join(TESTS, "abi_host", "abi_host_check.cpp"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"build failed:\n{r.stderr[-3000:]}"
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out[-4000:]
        assert "0 failed" in out and "Sanitizer" not in out and "runtime error" not in out, out


def test_oracle_pins_under_sanitizers():
    _need("gcc")
    asan = _runtime("libasan.so")
    with tempfile.TemporaryDirectory(prefix="oracle_san_") as tmp:
        so = os.path.join(tmp, "liboracle_san.so")
        cmd = ["gcc", "-std=c11", *SAN, "-Wall", "-shared", "-fPIC", "-pthread",
               "-o", so, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"build failed:\n{r.stderr[-3000:]}"
        # (the interpreter itself is not instrumented; its own allocations are
        # not leak-checked)
        env = dict(os.environ, LD_PRELOAD=asan,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([sys.executable, os.path.join(TESTS, "oracle_pins.py"), so],
                           capture_output=True, text=True, timeout=900, env=env, cwd=TESTS)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out[-4000:]
        assert "FAIL" not in out and "Sanitizer" not in out and "runtime error" not in out, out
