"""The C ABI's host validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).  tests/abi_sanitize/validation.cpp is
linked against the real validation layer (moe_abi.cpp, plan.cpp) and
launchers that abort if reached, built with g++ (host code only), and run:
every rejected call must return its status, launch nothing and write
nothing, and no size computation over the shape domain may overflow."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
HIPLIB = os.path.join(ROCM, "lib", "libamdhip64.so")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(HIPLIB),
                                reason="needs g++ and the HIP runtime library")


def test_validation_battery_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "sparse_moe_routed_amd", "csrc")
    here = os.path.join(ROOT, "tests", "abi_sanitize")
    srcs = [os.path.join(here, "validation.cpp"), os.path.join(here, "stub_launch.cpp"),
            os.path.join(csrc, "moe_abi.cpp"), os.path.join(csrc, "plan.cpp")]
    exe = str(tmp_path / "validation")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), *srcs, "-o", exe,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all passed" in r.stdout
