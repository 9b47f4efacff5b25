"""Host AddressSanitizer / UndefinedBehaviorSanitizer builds (CPU, no GPU):

* the fp64 oracle (oracle/gla_oracle.c) under a C driver that runs every oracle
  function on small shapes, all scan orders, one and several threads and ragged
  chunks, and checks that recurrence, quadratic form and chunked form agree;
* the C ABI layer (csrc/gtr_gla_api.cpp: validation, planning glue, workspace
  bookkeeping) under a C++ driver that calls every validating entry point with
  valid, invalid and extreme arguments, the kernel-launch layer and the HIP
  runtime calls replaced by stand-ins (tests/sanitize/abi_stubs.cpp).

Both are built with g++/gcc (host code only) and must exit cleanly.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "chunkwise_gated_recurrence_amd", "csrc")
FLAGS = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-pthread", *FLAGS, "-o", exe,
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "gla_oracle.c"),
          "-lm"], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV)
    assert r.returncode == 0 and "0 failures" in r.stdout, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *FLAGS, "-o", exe,
          os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "abi_stubs.cpp"),
          os.path.join(CSRC, "gtr_gla_api.cpp")], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV)
    assert r.returncode == 0 and "0 failures" in r.stdout, r.stdout + r.stderr
