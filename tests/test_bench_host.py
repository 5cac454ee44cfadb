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


def test_executed_and_floor_flop_models_match_the_plan(monkeypatch):
    """bench.py splits the plan's executed MFMA FLOP per product; the split
    must add up to what the library plans, on both GEMM paths."""
    for name, ns in (("qwen3_1.7b", pm.MUONH_BF16), ("stress", pm.MUONH_BF16),
                     ("stress", pm.MUONH_F32), ("diag170m", pm.MUONH_BF16)):
        wl = inputs.workload(name)
        tsize = 2 if ns == pm.MUONH_BF16 else 4
        info = pm.plan_query(wl.shapes, pm.default_options(ns_dtype=ns))
        ex = bench.plan_exec_flops(wl.shapes, 5, tsize, info.ns_exec_flops)
        assert sum(ex.values()) == pytest.approx(info.ns_exec_flops, rel=1e-12)
    # the single 256 x 128 matrix runs on the 64 x 64 path
    info = pm.plan_query([(256, 128)], pm.default_options(ns_dtype=pm.MUONH_F32), g_dtype=pm.MUONH_F32)
    assert sum(bench.exec_flops([(256, 128)], 5, 4, True).values()) == pytest.approx(info.ns_exec_flops)
    # ... and bench names the kernel of the path the plan took
    assert bench.plan_gemm_path([(256, 128)], 5, 4, info.ns_exec_flops)[1] is True
    wl = inputs.workload("qwen3_1.7b")
    big = pm.plan_query(wl.shapes, pm.default_options(ns_dtype=pm.MUONH_BF16))
    assert bench.plan_gemm_path(wl.shapes, 5, 2, big.ns_exec_flops)[1] is False
    monkeypatch.setenv("MUONH_GEMM_TILE", "256")
    info = pm.plan_query([(256, 128)], pm.default_options(ns_dtype=pm.MUONH_F32), g_dtype=pm.MUONH_F32)
    assert sum(bench.exec_flops([(256, 128)], 5, 4, False).values()) == pytest.approx(info.ns_exec_flops)
    # aligned 1.7B shapes: the floor is 3 m^2 n + m^3 per iteration; the
    # executed count lies between it and the dense one (the diagonal tiles)
    wl = inputs.workload("qwen3_1.7b")
    f, _, _ = bench.per_kernel_work(wl.shapes, 5, 2, 2)
    floor = bench.floor_flops(wl.shapes, 5)
    assert floor == pytest.approx(f["ns_gram"] / 2 + f["ns_poly"] / 2 + f["ns_apply"], rel=1e-12)
    info = pm.plan_query(wl.shapes)
    assert floor < info.ns_exec_flops < sum(f.values())


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
    assert bench.traffic_for("ns_apply", "qwen3_1.7b", "bf16") is None


def test_traffic_belongs_to_its_kernel_workload_and_type():
    """The committed counter profile covers the bf16 B'X launch of the 1.7B
    set only: another workload, Newton-Schulz type or kernel gets None."""
    t = bench.traffic_for("ns_apply", "qwen3_1.7b", "bf16")
    assert t is not None and t > 0
    assert bench.traffic_for("ns_apply", "diag170m", "bf16") is None
    assert bench.traffic_for("ns_apply", "qwen3_1.7b", "f32") is None
    assert bench.traffic_for("ns_gram", "qwen3_1.7b", "bf16") is None


def test_data_label_follows_the_workload():
    assert "N(0,1) grads" in bench.synthetic_data_label(inputs.workload("qwen3_1.7b"))
    assert "fan_in" in bench.synthetic_data_label(inputs.workload("diag170m"))
    assert "rank-8" in bench.synthetic_data_label(inputs.workload("stress"))
