"""Host code under AddressSanitizer and UBSan, on the CPU.

* The C ABI layer (csrc/api.hip, host side instrumented, device side the
  usual gfx950 build) linked with stand-ins for the kernel launchers
  (tests/sanitize/abi_stubs.cpp) and driven through every entry point with
  valid, invalid and extreme arguments (tests/sanitize/abi_driver.cpp): each
  call returns its documented status and a failing call launches nothing.
* The C oracle (oracle/dsa_oracle.c) driven over small decode and prefill
  cases and its error paths (tests/sanitize/oracle_driver.c).
Any sanitizer report aborts the driver, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_attention_indexer_amd", "csrc")
INC = os.path.join(ROOT, "include")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm compilers not installed")
def test_abi_layer_under_asan_ubsan(build_dir):
    # The host pass of hipcc gets the sanitizers (each flag behind -Xarch_host);
    # the plain C++ parts and the link use clang++ directly.
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer",
          "-std=c++17", *host_san, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INC, "-I", CSRC, "-c", os.path.join(CSRC, "api.hip"), "-o", "api.o"], build_dir)
    _run([CLANGXX, "-O1", "-g", "-std=c++17", *san, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", INC, "-I", CSRC, "-c",
          os.path.join(SAN, "abi_stubs.cpp"), "-o", "stubs.o"], build_dir)
    _run([CLANGXX, "-O1", "-g", "-std=c++17", *san, "-I", INC, "-c",
          os.path.join(SAN, "abi_driver.cpp"), "-o", "driver.o"], build_dir)
    _run([CLANGXX, *san, "api.o", "stubs.o", "driver.o", "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", "abi_driver"], build_dir)
    r = subprocess.run([os.path.join(build_dir, "abi_driver")], capture_output=True, text=True,
                       timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(build_dir):
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "dsa_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
          "-o", "oracle_driver", "-lm"], build_dir)
    r = subprocess.run([os.path.join(build_dir, "oracle_driver")], capture_output=True,
                       text=True, timeout=300, env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
