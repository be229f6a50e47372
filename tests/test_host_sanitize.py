"""The host half of the library (packer, unpacker, calibration, the C ABI's
argument checks) built with AddressSanitizer and UndefinedBehaviorSanitizer
by g++ and run on random weights of small, ragged shapes in every precision
mode (tests/sanitize/host_driver.cpp); the device functions are stand-ins
that abort if reached (tests/sanitize/device_stubs.cpp).  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_memory_bound_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path / "host_driver")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I" + os.path.join(ROCM, "include"),
           "-D__HIP_PLATFORM_AMD__"]
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "pack.cpp"),
            os.path.join(HERE, "host_driver.cpp"), os.path.join(HERE, "device_stubs.cpp")]
    cmd = [gxx] + flags + inc + srcs + ["-o", exe, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                                        "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "OK (0 failed checks)" in r.stdout, out[-4000:]
