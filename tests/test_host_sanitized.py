"""CPU: libattnres's host-side validation and dispatch planning under
AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code only; no HIP
call is made).  See tests/native/host_checks.cpp."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_residual_rmsnorm_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-I", CSRC, os.path.join(ROOT, "tests", "native", "host_checks.cpp"),
           os.path.join(CSRC, "attnres_host.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
