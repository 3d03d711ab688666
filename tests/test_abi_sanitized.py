"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library sources with the sanitizers on the host side only (each
-fsanitize= follows -Xarch_host; device code is built as usual) together with
tests/native/abi_host_checks.cpp, a host program that drives every entry
point's validation, size queries and host-side planning with ragged and
extreme inputs, and runs it.  Any sanitizer report fails the test.  No GPU is
used: without one the planning paths stop at the first HIP call, and with one
the program runs its validation cases only.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

import pytest

from compressed_composable_kv_amd import build_lib as B

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "native", "abi_host_checks.cpp")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = [f"--offload-arch={B.ARCH}", "-xhip", "-O1", "-g", "-std=c++17", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{B.INCLUDE}", f"-I{B.CSRC}"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("abi_san")
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [DRIVER]
    objs = [str(out / (os.path.splitext(os.path.basename(s))[0] + ".o")) for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, [[B.HIPCC, *FLAGS, *SAN, "-c", s, "-o", o] for s, o in zip(srcs, objs)]))
    exe = str(out / "abi_host_checks")
    _run([B.HIPCC, f"--offload-arch={B.ARCH}", *SAN[:4], *objs, "-o", exe, "-Wl,-rpath,/opt/rocm/lib"])
    return exe


def test_abi_host_code_is_sanitizer_clean(sanitized_driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert r.returncode == 0, report
    assert "checks passed" in r.stdout and "FAILED" not in r.stdout, report
