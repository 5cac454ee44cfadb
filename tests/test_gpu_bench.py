"""bench.py end to end on a small workload (MI355X only): the one JSON line
its contract defines, with the roofline and CPU-baseline objects, and values
consistent with each other."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_on_the_170m_set():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "diag170m",
           "--steps", "3", "--warmup", "1", "--cpu-mats", "2", "--no-hbm-ceiling"]
    print("[gpu-test] bench.py on the 170M set, 3 steps", flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "steps/s" and d["higher_is_better"] is True
    assert d["value"] > 0 and d["value"] == pytest.approx(1000.0 / d["ms_per_step"], rel=1e-6)
    assert d["config"]["workload"].startswith("diag170m")
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2500.0
    assert 0 < rl["achieved"] < rl["peak"]
    assert rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], rel=1e-9)
    # the traffic figure is recorded for the 1.7B launch only
    assert rl["traffic"] is None
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert "2 of 84 matrices" in cb["sample"] or "2 matrices" in cb["sample"], cb["sample"]
    assert d["norm_invariant_max_dev"] < 1e-5
