"""The planner's grouped-GEMM tile lists, checked on the host (CPU only):
every output tile of every Newton-Schulz product listed exactly once, each
unit of row panels on one XCD, longest contractions first within an XCD, and
the executed-FLOP count consistent with the lists (tests/host_plan/)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _have_toolchain() -> bool:
    return shutil.which("g++") is not None and os.path.exists(os.path.join(ROCM, "include", "hip"))


@pytest.mark.skipif(not _have_toolchain(), reason="g++ or the ROCm headers are missing")
def test_tile_lists_cover_every_tile_once(tmp_path):
    exe = tmp_path / "tile_lists"
    cmd = ["g++", "-std=c++17", "-O1", "-Wno-subobject-linkage", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "host_plan", "tile_lists.cpp"),
           os.path.join(HERE, "host_sanitize", "launch_stubs.cpp"),
           "-o", str(exe), "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = {k: v for k, v in os.environ.items() if k != "MUONH_GEMM_TILE"}
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "all checks passed" in out, out[-4000:]
