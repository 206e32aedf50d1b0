"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_check.cpp links the library's own validation and planning sources
(fa_api.cpp, fa_plan.cpp) against stub launchers and drives every status
code; it is built here with g++ (host code only: no GPU code is involved and
no HIP runtime call is made) with -fsanitize=address,undefined and no
recovery, so an out-of-bounds access, an integer overflow in the size
arithmetic or any other undefined behaviour fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("g++ or the HIP headers are not installed")
    exe = str(tmp_path / "abi_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           os.path.join(ROOT, "tests", "abi_check.cpp"), os.path.join(CSRC, "fa_api.cpp"),
           os.path.join(CSRC, "fa_plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # (verify_asan_link_order=0: the environment may preload other libraries)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all expectations hold" in r.stdout
