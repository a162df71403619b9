"""The C ABI's host code under address and undefined-behaviour sanitizers.

Builds every library source with the sanitizers on the host code only (the
device code is compiled as usual) together with tests/abi_sanitize/abi_check.cpp,
which calls each entry point with invalid arguments (and, on a host without a
GPU, valid ones that stop at the device check) and checks every status.  No
kernel is launched.  A sanitizer report fails the run.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ternary_bitlinear_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OUT = os.path.join(ROOT, "ternary_bitlinear_amd", "_build", "sanitize")

# Sanitizers for the host pass only, each -fsanitize= right after -Xarch_host.
HOST_SAN = ["-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_host_sanitizers():
    from ternary_bitlinear_amd.build import FLAGS, SOURCES
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_check")
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [
        os.path.join(ROOT, "tests", "abi_sanitize", "abi_check.cpp")]
    flags = [f for f in FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC, *flags, *HOST_SAN, "-x", "hip", *srcs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "abi_check ok" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
