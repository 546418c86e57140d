"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

abi.hip is compiled as plain host C++ against the HIP headers, with host stubs for the kernel
launchers and the HIP device queries (tests/sanitize/host_stubs.cpp): no device code and no HIP
runtime are linked, and nothing is launched. tests/sanitize/abi_validation.c then calls every entry
point with valid arguments, with each invalid argument the header names, and with sizes up to
INT64_MAX; every call must return the status include/pf8.h promises, and any sanitizer report
(memory error, signed overflow, misaligned access, ...) fails the run. The oracle is plain numpy and
has no native code of its own to check this way."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_block_scaled_pf8_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIP_INCLUDE = "/opt/rocm/include"
FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]


def _tool(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not available")
    return path


def test_abi_validation_clean_under_asan_and_ubsan(tmp_path):
    gxx, gcc = _tool("g++"), _tool("gcc")
    if not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")):
        pytest.skip("HIP headers not available")
    cxx = [gxx, "-x", "c++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + HIP_INCLUDE, "-I" + CSRC, *FLAGS, "-c"]
    objs = []
    for src, obj in ((os.path.join(CSRC, "abi.hip"), "abi.o"), (os.path.join(SAN, "host_stubs.cpp"), "stubs.o")):
        out = str(tmp_path / obj)
        r = subprocess.run(cxx + [src, "-o", out], capture_output=True, text=True, timeout=300)
        if r.returncode != 0 and "asan" in (r.stderr or "").lower():
            pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
        assert r.returncode == 0, r.stderr
        objs.append(out)
    exe = str(tmp_path / "abi_validation")
    r = subprocess.run([gcc, "-std=c11", "-I" + os.path.join(ROOT, "include"), *FLAGS,
                        os.path.join(SAN, "abi_validation.c"), *objs, "-lstdc++", "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert out.strip().startswith("ok ") and int(out.split()[1]) >= 80, out
