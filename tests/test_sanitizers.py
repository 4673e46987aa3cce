"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C-ABI front end (argument validation, error reporting) is built for the host alone, with the
kernel launchers replaced by stand-ins that report an error (tests/sanitize/host_stubs.cpp), and
the oracle's C is built as it is; both instrumented.  The host ABI tests and the oracle pins then
run against those builds in a child process with the sanitizer runtime preloaded: any invalid
access or undefined behaviour aborts the run.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="no host compiler")
def test_abi_validation_and_oracle_under_sanitizers(tmp_path):
    te_lib = str(tmp_path / "libte_fp8_host_san.so")
    or_lib = str(tmp_path / "liboracle_san.so")
    csrc = os.path.join(ROOT, "fp8_linear_layer_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"), "-o", te_lib], check=True)
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", *SAN,
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", or_lib], check=True)
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    env = dict(os.environ, LD_PRELOAD=libasan, TE_FP8_TEST_LIB=te_lib, ORACLE_TEST_LIB=or_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
