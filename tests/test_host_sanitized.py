"""The library's host code (planner, work lists, C-ABI argument handling)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run
on the CPU (tests/host/wsp_host_check.cpp: stub kernel launchers, no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_dit_window_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.timeout(600)
def test_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "wsp_host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-Wall",
           # the two HIP-compiler macros abi.cpp uses, for a host-only compiler
           "-D__align__(x)=__attribute__((aligned(x)))", "-DHIP_SYMBOL(X)=X",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "wsp_host_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "abi.cpp"), "-o", exe, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "host build failed:\n" + r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               LSAN_OPTIONS="suppressions=" + os.path.join(ROOT, "tests", "host", "lsan.supp"))
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=500)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, "sanitized host check failed:\n" + r.stderr[-4000:]
    assert "host check: ok" in r.stdout
