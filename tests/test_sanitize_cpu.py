"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two standalone drivers under tests/sanitize/, built here into a temporary
directory:

* oracle_checks: the fp64 oracle's C source with the sanitizers, checked
  on malloc'd buffers of exact size against closed forms (single-sample
  ramp, k = 0 sum, adjointness, thread-count independence);
* abi_checks: libfhd.so's host code compiled with the sanitizers (the
  device code as usual), driven through the C ABI on calls that are
  refused or return before any device access, so no GPU is needed.

Each driver exits 0 when its checks hold; a sanitizer report aborts it.
"""
import os
import shutil
import subprocess

import pytest

from non_cartesian_mri_fhd_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
         "-fno-sanitize-recover=all"]


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    run(["gcc", "-std=c11", "-ffp-contract=off", *FLAGS, os.path.join(ROOT, "oracle", "fhd_oracle.c"),
         os.path.join(SAN, "oracle_checks.c"), "-o", exe, "-lm", "-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    assert "passed" in run([exe], env=env).stdout


@pytest.mark.skipif(not os.path.exists(CLANG), reason="needs the ROCm clang")
def test_abi_host_code_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libfhd_san.so")
    srcs = [os.path.join(build.CSRC, s) for s in build.LIBRARIES["libfhd.so"]]
    # the sanitizers instrument the host code only
    run([build.HIPCC, "--offload-arch=" + build.ARCH, "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + build.INCLUDE, "-o", lib, *srcs])
    exe = str(tmp_path / "abi_checks")
    run([CLANG, *FLAGS, "-I" + build.INCLUDE, os.path.join(SAN, "abi_checks.c"), "-L" + str(tmp_path),
         "-lfhd_san", "-Wl,-rpath," + str(tmp_path), "-o", exe])
    # the HIP runtime keeps allocations for the process's life: leaks off
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    assert "passed" in run([exe], env=env).stdout
