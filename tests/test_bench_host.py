"""Host-side checks of bench.py (CPU only): the one-GPU guard, its work
model against the library's own plan, and the key that ties the recorded
GEMM traffic to the kernel sources."""

import os
import shutil
import subprocess
import sys

import pytest

import bench
import inputs
import pretraining_optimizer_amd as pm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_work_model_matches_plan():
    wl = inputs.workload("qwen3_1.7b")
    f, b, params = bench.per_kernel_work(wl.shapes, 5, 2, 2)
    info = pm.plan_query(wl.shapes)
    assert sum(f.values()) == pytest.approx(info.ns_dense_flops, rel=1e-12)
    assert params == wl.params()
    assert info.elem_bytes == pytest.approx(18.0 * params)   # G in, M and W in and out
    assert b["update"] == pytest.approx(10.0 * params)       # W in and out, bf16 u in
    # momentum: G (2) + M in and out (8) per element, X_0 (2) per padded
    # element; every dim of this set is a multiple of 256, so no padding
    assert b["momentum"] == pytest.approx(12.0 * params)
    # a ragged shape pads X_0: (300, 200) -> 256 x 512 in NS orientation
    _, b2, p2 = bench.per_kernel_work([(300, 200)], 5, 2, 2)
    assert b2["momentum"] == pytest.approx(10.0 * p2 + 2.0 * 256 * 512)


def _copy_sources(dst):
    src = os.path.join(ROOT, "pretraining_optimizer_amd", "csrc")
    out = os.path.join(dst, "pretraining_optimizer_amd", "csrc")
    os.makedirs(out)
    for f in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(src, f), out)
    return out


def test_traffic_key_ignores_comments_only(tmp_path, monkeypatch):
    ref = bench.kernel_source_sha()
    csrc = _copy_sources(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_sha() == ref
    p = os.path.join(csrc, "gemm.hip")
    text = open(p).read()
    open(p, "w").write("// a new comment\n\n/* and a block\n   comment */\n" + text.replace("\n", "  // note\n", 3))
    assert bench.kernel_source_sha() == ref
    open(p, "w").write(text + "\nstatic int unused_marker = 0;\n")
    assert bench.kernel_source_sha() != ref


def test_traffic_is_none_when_the_key_does_not_match(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 64)
    assert bench.traffic_for("ns_apply") is None
