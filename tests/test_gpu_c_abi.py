"""The library driven from C through include/muonh.h alone (no Python
binding, no torch): tests/c_abi/one_step.c, built with the host compiler
against the in-tree libmuonh.so, runs one step on the MI355X and checks the
Hyperball identities itself."""

import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LIBDIR = os.path.join(ROOT, "pretraining_optimizer_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_one_step_from_c(tmp_path):
    assert os.path.exists(os.path.join(LIBDIR, "libmuonh.so")), "build the library first"
    exe = tmp_path / "one_step"
    cmd = ["gcc", "-std=c11", "-O1", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "one_step.c"), "-o", str(exe),
           "-L", LIBDIR, "-lmuonh", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + LIBDIR + ":" + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    print("running the C driver", flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
