"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code, CPU only:
the C oracle (gcc) and the host side of libsvla (hipcc, sanitizers on the
host pass only; the device code is built unoptimised, since none of it runs),
each driven by a small C program under tests/sanitize/ that reaches every
branch the CPU can reach.  The first invalid access or undefined operation
aborts the driver, and the test fails with its report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(SAN, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "bin", "amdclang")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, timeout=600, env=None):
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    return p.returncode, p.stdout + p.stderr


def test_oracle_under_sanitizers():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_san")
    rc, log = _run(["gcc", "-O1", "-g", "-std=c99", "-Wall", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", os.path.join(SAN, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "svla_oracle.c"), "-lm", "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe], env=ENV)
    assert rc == 0 and "clean" in log, log


def test_library_host_code_under_sanitizers():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libsvla_host_san.so")
    src = os.path.join(ROOT, "block_causal_linear_relu_amd", "csrc", "svla.hip")
    inc = os.path.join(ROOT, "include")
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
                    "-Xarch_host", "-O1", "-Xarch_host", "-g", "-Xarch_device", "-O0",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I" + inc, src, "-o", lib])
    assert rc == 0, log
    exe = os.path.join(OUT, "abi_san")
    rc, log = _run([CLANG, "-O1", "-g", "-std=c99", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I" + inc, os.path.join(SAN, "abi_driver.c"),
                    "-L" + OUT, "-lsvla_host_san", "-Wl,-rpath," + OUT,
                    "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe], env=ENV)
    assert rc == 0 and "clean" in log, log
