"""The host half of the C ABI (argument checks, frequency tables, workspace
sizing, the decode plan) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through every entry point in a child
process (CPU only; the device side is stubbed, see tests/sanitize/)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "yarn_scaled_rope_amd", "csrc")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "freqs.cpp", "decode_plan.cpp")]


def _gxx():
    return shutil.which("g++")


@pytest.mark.skipif(_gxx() is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libyarnattn_host_san.so")
    cmd = [_gxx(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include", *HOST_SOURCES,
           os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    asan = subprocess.run([_gxx(), "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = dict(os.environ)
    env.update({"LD_PRELOAD": asan, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "abi_calls.py"),
                        lib], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert "no report" in r.stdout
