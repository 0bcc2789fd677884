"""The host code of the C ABI (validation, planner, workspace layout) built
with AddressSanitizer and UndefinedBehaviorSanitizer by the host compiler and
driven through random and extreme shapes and every validation path.  The
kernel launches are stubs: no GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_14_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "fd_host_checks"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "fd_api.cpp"), os.path.join(CSRC, "fd_select.cpp"),
           os.path.join(ROOT, "tests", "sanitize_host_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize_host_driver.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "host checks ok" in r.stdout
