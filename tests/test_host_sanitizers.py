"""The library's host code (planner, validation, schedule helpers, AdamW
host side) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
and driven through the C ABI with no device (CPU only; kernel launches are
stubbed, and never reached).  A sanitizer report or a failed check fails."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "pretraining_optimizer_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _have_toolchain() -> bool:
    return shutil.which("g++") is not None and os.path.exists(os.path.join(ROCM, "include", "hip"))


@pytest.mark.skipif(not _have_toolchain(), reason="g++ or the ROCm headers are missing")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_driver"
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    srcs = [os.path.join(CSRC, "muonh.cpp"), os.path.join(CSRC, "adamw.cpp"),
            os.path.join(HERE, "host_sanitize", "launch_stubs.cpp"),
            os.path.join(HERE, "host_sanitize", "driver.cpp")]
    cmd = ["g++", *flags, *srcs, "-o", str(exe), "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    # Leak checking covers the library's own allocations (the failing init
    # paths must free their plan and handle); the HIP runtime's are suppressed.
    supp = tmp_path / "lsan.supp"
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:libdrm\nleak:librocprofiler\n")
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["LSAN_OPTIONS"] = f"suppressions={supp}"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "all checks passed" in out
    assert "runtime error" not in out and "Sanitizer" not in out, out[-4000:]
