"""The per-matrix update coefficients of the finalise kernel
(csrc/update_math.h: the Hyperball closed form of Eq. (1), and the Eq. (3)
and Eq. (5) modes), compiled with the host compiler and checked on the CPU
against the exact norm R sqrt(1 - 2 eta c + eta^2), including eta and c near
and at 1 where the closed form cancels."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="g++ or the ROCm headers are missing")
def test_update_coefficients_on_the_host(tmp_path):
    exe = tmp_path / "update_coeffs"
    cmd = ["g++", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "pretraining_optimizer_amd", "csrc"),
           os.path.join(HERE, "host_math", "update_coeffs.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "all checks passed" in r.stdout
