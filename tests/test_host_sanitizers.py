"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU only).

* The fp64 oracle (``oracle/hetattn_oracle.c``) with a C driver that runs
  every oracle function on small inputs and checks their invariants.
* The C ABI layer (``csrc/api.cpp``: argument checks, marshalling, the
  workspace carving of the backward and the allocation-free forward) built
  with the host compiler against stand-ins for the device launchers and the
  two HIP device queries, with a driver that calls every entry point of
  ``include/hetattn.h`` with valid and invalid arguments.

Both are built with -fsanitize=address,undefined -fno-sanitize-recover=all
(g++/gcc only: no device code is built here) and must run clean.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "uncertainty_routed_heterogeneous_amd", "csrc")
FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def run_clean(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c11", "-fopenmp", *FLAGS, "-I", os.path.join(ROOT, "oracle"),
                           os.path.join(ROOT, "oracle", "hetattn_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
                           "-o", exe, "-lm"])
    assert "oracle driver ok" in run_clean(exe)


@pytest.mark.skipif(not os.path.isdir("/opt/rocm/include/hip"), reason="HIP headers not installed")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    subprocess.check_call(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *FLAGS, "-I", "/opt/rocm/include",
                           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "api.cpp"),
                           os.path.join(SAN, "api_stubs.cpp"), os.path.join(SAN, "api_driver.cpp"), "-o", exe])
    assert "api driver ok" in run_clean(exe)
