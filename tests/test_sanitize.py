"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two programs are built with gcc/g++ (host code only, no device code) and
run:

* the C ABI layer (``csrc/abi.cpp``) and the host sizes and plans
  (``csrc/layout.cpp``), linked against recording stand-ins of the kernel
  launchers (``tests/asan/launch_stubs.cpp``) and driven through every entry
  point's checks by ``tests/asan/abi_driver.cpp``;
* the CPU oracle (``oracle/osm_oracle.c``), driven through its edge cases by
  ``tests/asan/oracle_driver.c``.

Any sanitizer report aborts the program (``-fno-sanitize-recover=all``)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_online_softmax_amd", "csrc")
ASAN = os.path.join(ROOT, "tests", "asan")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{' '.join(cmd)}\n{r.stderr}"
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    return out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_host_code_sanitized(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "layout.cpp"),
           os.path.join(ASAN, "launch_stubs.cpp"), os.path.join(ASAN, "abi_driver.cpp"), "-o", exe]
    assert "all expectations hold" in _build_and_run(cmd, exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", *SAN, "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           os.path.join(ROOT, "oracle", "osm_oracle.c"), os.path.join(ASAN, "oracle_driver.c"),
           "-o", exe, "-lm"]
    assert "all expectations hold" in _build_and_run(cmd, exe)
