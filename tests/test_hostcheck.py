"""The C ABI's host code (argument validation, workspace layout, dispatch) built for the CPU with
AddressSanitizer and UndefinedBehaviorSanitizer, the kernel launchers replaced by stubs that
check every workspace pointer against the workspace (tests/hostcheck).  The driver calls every
entry point on every dispatch path with valid and invalid arguments; any sanitizer report,
workspace pointer out of range or unexpected status fails it.  Needs only g++ and the ROCm
headers."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "hostcheck")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_hostcheck"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "coreset_head_rpcholesky_amd", "csrc", "wc_api.cpp"),
           os.path.join(HERE, "stub_launch.cpp"), os.path.join(HERE, "abi_driver.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "hostcheck ok" in run.stdout
