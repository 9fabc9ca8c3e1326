"""The C-ABI host code (abi.cpp, validate.cpp) built with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer, against host stand-ins of the HIP runtime and of the
kernel launchers (tests/host_stub).  The driver calls every entry point with every
argument error (each must return its status before any launch) and with valid shapes
of every path; the stand-in launchers write each output's full extent, so an
undersized workspace plan or an output placed past a caller's buffer is reported by
the sanitizer.  No GPU and no HIP compiler are involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_sparse_attention_hca_amd", "csrc")
STUB = os.path.join(ROOT, "tests", "host_stub")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_host_paths_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_host"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-Wall",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", STUB, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "validate.cpp"),
           os.path.join(STUB, "launch_stub.cpp"), os.path.join(STUB, "driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ABI checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
