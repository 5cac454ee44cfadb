"""The C ABI on the host (CPU only): the library loads, exports every entry
point the header declares, plans and validates without a device, and its
LR helpers agree with the oracle's schedules."""

import ctypes
import json
import os
import re

import pytest

import inputs
import oracle
import pretraining_optimizer_amd as pm
from pretraining_optimizer_amd import muonh as mb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muonh.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muonh_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = pm.load_library()
    names = _declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
    bound = {n for n, _, _ in mb._SIGNATURES}
    assert set(names) == bound


def test_default_options():
    o = pm.default_options()
    assert o.beta == pytest.approx(0.95)
    assert o.ns_steps == 5
    assert (o.ns_a, o.ns_b, o.ns_c) == pytest.approx(oracle.NS_COEFFS_QUINTIC)
    assert o.ns_eps == pytest.approx(1e-7)
    assert o.ns_dtype == pm.MUONH_BF16 and o.mode == pm.MUONH_MODE_HYPERBALL and o.symmetric == 1
    assert o.deterministic == 1
    # the flag sits in what was padding before the workspace pointer
    assert mb.muonh_options.workspace.offset == 48 and ctypes.sizeof(mb.muonh_options) == 64
    # 0 is accepted (the path is deterministic either way)
    assert pm.plan_query([(8, 8)], pm.default_options(deterministic=0)).n_matrices == 1


def _tiles(m_pad, n_pad, sym=True):
    mt, nt = m_pad // 256, n_pad // 256
    gram = mt * (mt + 1) // 2 if sym else mt * mt
    return gram, gram, mt * nt


def test_plan_qwen3_17b_buckets_tiles_and_flops():
    wl = inputs.workload("qwen3_1.7b")
    info = pm.plan_query(wl.shapes)
    assert info.n_matrices == 196 and info.n_buckets == 3
    expect = [0, 0, 0]
    for r, c in wl.shapes:
        t = _tiles(min(r, c), max(r, c))
        expect = [a + b for a, b in zip(expect, t)]
    assert list(info.gemm_tiles) == expect
    dense = sum(oracle.muonh.ns_dense_flops(r, c) for r, c in wl.shapes)
    assert info.ns_dense_flops == pytest.approx(dense, rel=1e-12)
    assert info.ns_dense_flops == pytest.approx(6.795e13, rel=1e-3)
    # momentum blocks: 64 x 128 tiles for tall matrices (their X_0 is packed
    # transposed), 1024-column row segments otherwise (bf16 plan)
    assert info.mom_tiles == sum((r // 64) * (c // 128) if r > c else r * -(-c // 1024)
                                 for r, c in wl.shapes)
    f32 = pm.plan_query(wl.shapes, pm.default_options(ns_dtype=pm.MUONH_F32))
    assert f32.mom_tiles == sum(r * c for r, c in wl.shapes) // 8192
    assert info.elem_bytes == pytest.approx(18.0 * wl.params())


def test_plan_pads_ragged_shapes(monkeypatch):
    shapes = [(1, 1), (300, 200), (129, 4096)]
    monkeypatch.setenv("MUONH_GEMM_TILE", "256")
    info = pm.plan_query(shapes, pm.default_options(symmetric=0))
    assert info.n_buckets == 3
    # (1,1) -> 256x256; (300,200) -> 256x512 (tall: m=200, n=300); (129,4096) -> 256x4096
    assert list(info.gemm_tiles) == [3, 3, 1 + 2 + 16]
    # The same plan on the small-problem path: 64 x 64 tiles over the valid
    # dims only, every tile listed: m = 1, 200, 129 -> 1, 4, 3 row tiles;
    # n = 1, 300, 4096 -> 1, 5, 64 column tiles.
    monkeypatch.setenv("MUONH_GEMM_TILE", "64")
    small = pm.plan_query(shapes, pm.default_options(symmetric=0))
    assert list(small.gemm_tiles) == [1 + 16 + 9, 1 + 16 + 9, 1 + 20 + 192]
    # The path is chosen by the big-tile count of B'X when not forced: 19 < 64.
    monkeypatch.delenv("MUONH_GEMM_TILE")
    assert list(pm.plan_query(shapes, pm.default_options(symmetric=0)).gemm_tiles) == list(small.gemm_tiles)
    assert info.flat_chunks == 1 + 4 + 33


def test_plan_gemm_path_threshold(monkeypatch):
    monkeypatch.delenv("MUONH_GEMM_TILE", raising=False)
    # 2048 x 2048 has 8 x 8 = 64 big B'X tiles: the big path; 63 of them in
    # 63 matrices of 256 x 256: the small path (one 64-tile grid of 4 x 4 each).
    assert list(pm.plan_query([(2048, 2048)]).gemm_tiles)[2] == 64
    assert list(pm.plan_query([(256, 256)] * 63).gemm_tiles)[2] == 63 * 16
    assert list(pm.plan_query([(256, 256)] * 64).gemm_tiles)[2] == 64


def test_workspace_size_matches_plan():
    shapes = inputs.workload("diag170m").shapes
    assert pm.workspace_size(shapes) == pm.plan_query(shapes).workspace_bytes
    f32 = pm.workspace_size(shapes, pm.default_options(ns_dtype=pm.MUONH_F32))
    assert f32 > pm.workspace_size(shapes)


@pytest.mark.parametrize("bad", [
    dict(shapes=[(0, 5)]), dict(shapes=[(5, -1)]), dict(shapes=[(70000, 8)]),
    dict(opts=dict(ns_steps=0)), dict(opts=dict(ns_steps=17)), dict(opts=dict(ns_dtype=7)),
    dict(opts=dict(mode=9)), dict(opts=dict(nesterov=2)), dict(opts=dict(ns_eps=-1.0)),
    dict(opts=dict(deterministic=2)), dict(g_dtype=5),
])
def test_invalid_arguments_are_rejected(bad):
    shapes = bad.get("shapes", [(8, 8)])
    opts = pm.default_options(**bad.get("opts", {}))
    with pytest.raises(pm.MuonHError) as ei:
        pm.plan_query(shapes, opts, g_dtype=bad.get("g_dtype", pm.MUONH_BF16))
    assert ei.value.status == mb.MUONH_EINVAL
    assert pm.load_library().muonh_last_error()


def test_null_and_empty_arguments():
    lib = pm.load_library()
    o = pm.default_options()
    n = ctypes.c_size_t()
    assert lib.muonh_workspace_size(None, 1, ctypes.byref(o), ctypes.byref(n)) == mb.MUONH_EINVAL
    assert lib.muonh_workspace_size(mb.shape_descs([(4, 4)]), 0, ctypes.byref(o), ctypes.byref(n)) == mb.MUONH_EINVAL
    assert lib.muonh_init(None, mb.shape_descs([(4, 4)]), 1, ctypes.byref(o), None) == mb.MUONH_EINVAL
    h = ctypes.c_void_p()
    # radius <= 0 with no weights to measure it from
    assert lib.muonh_init(ctypes.byref(h), mb.shape_descs([(4, 4)], radius=0.0), 1,
                          ctypes.byref(o), None) == mb.MUONH_EINVAL
    assert not h.value
    assert lib.muonh_step(None, None, 0, None, None) == mb.MUONH_EINVAL
    assert lib.muonh_destroy(None) == mb.MUONH_OK
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert lib.muonh_status_str(code)


def test_lr_helpers_match_oracle_schedules():
    lib = pm.load_library()
    for s in (0.0, 10.0, 123.4, 500.0, 900.0):
        assert lib.muonh_lr_linear(1.04e-3, 1e-5, s, 500.0) == pytest.approx(
            oracle.lr_linear(1.04e-3, 1e-5, s, 500.0), rel=1e-15)
    for k in (0.0, 250.0, 1000.0, 1001.0, 69751.7, 2e5):
        assert lib.muonh_lr_power(k, 5e-3, 5e-4, 1000.0, 1000.0, 0.5) == pytest.approx(
            oracle.lr_phase1_power(k), rel=1e-14)
    for k in (0, 2, 5, 7.5, 10):
        assert lib.muonh_lr_wsd(k, 0.024, 10.0, 0.5, 0.0, 0.0) == pytest.approx(
            oracle.lr_wsd(k, 0.024, 10, 0.5), rel=1e-14, abs=1e-18)


def test_hold_cosine_and_multiplier_helpers():
    lib = pm.load_library()
    sched = lambda s: oracle.lr_linear(1.04e-3, 1e-5, s, 500.0)
    for s in (0.0, 100.0, 300.0, 301.0, 450.0, 600.0):
        assert lib.muonh_lr_linear_hold(1.04e-3, 1e-5, s, 500.0, 300.0) == pytest.approx(
            oracle.lr_constant_hold(s, 300.0, sched), rel=1e-15)
    for k in (0.0, 5.0, 10.0, 37.0, 50.0, 99.0, 100.0, 150.0):
        assert lib.muonh_lr_cosine(k, 100.0, 1e-5, 1e-7, 10.0) == pytest.approx(
            oracle.lr_cosine(k, 100.0, 1e-5, 1e-7, warmup=10.0), rel=1e-14)
    assert lib.muonh_elr_from_base(1.04e-3, 10.0) == pytest.approx(oracle.hyperball_lr(1.04e-3))


def test_cma_hold_value_printed_on_the_pages():
    """The held LR of the constant-LR continuation, through the C helpers:
    Phase-1 end of Eq. (10), then Eq. (11) frozen at the hold step."""
    pins = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "schedule_pins.json")))
    lib = pm.load_library()
    tps = pins["tokens_per_step"]
    eta0 = lib.muonh_lr_power(pins["phase1_end"]["tokens"] / tps, 5e-3, 5e-4, 1000.0, 1000.0, 0.5)
    h = pins["cma_hold"]
    S = h["run_last_step"] - h["phase2_start_step"]
    for k in (h["hold_step"], 220000, h["run_last_step"]):
        v = lib.muonh_lr_linear_hold(eta0, h["eta_min"], k - h["phase2_start_step"], S,
                                     h["hold_step"] - h["phase2_start_step"])
        assert float(f"{v:.3g}") == h["printed_base_lr"]
        assert float(f"{lib.muonh_elr_from_base(v, 10.0):.3g}") == h["printed_hyperball_lr"]


def test_adamw_defaults_and_host_validation():
    lib = pm.load_library()
    o = mb.muonh_adamw_options()
    lib.muonh_adamw_default_options(ctypes.byref(o))
    assert (o.beta1, o.beta2, o.weight_decay) == pytest.approx((0.9, 0.95, 0.1))
    assert o.eps == pytest.approx(1e-12)
    h = ctypes.c_void_p()
    t = (mb.muonh_adamw_tensor * 2)()
    for i in range(2):
        t[i].numel, t[i].g_dtype = 1000, mb.MUONH_BF16
    assert lib.muonh_adamw_init(None, t, 2, None) == mb.MUONH_EINVAL
    assert lib.muonh_adamw_init(ctypes.byref(h), None, 2, None) == mb.MUONH_EINVAL
    assert lib.muonh_adamw_init(ctypes.byref(h), t, 0, None) == mb.MUONH_EINVAL
    t[1].numel = 0
    assert lib.muonh_adamw_init(ctypes.byref(h), t, 2, None) == mb.MUONH_EINVAL
    t[1].numel, t[1].g_dtype = 5, 7
    assert lib.muonh_adamw_init(ctypes.byref(h), t, 2, None) == mb.MUONH_EINVAL
    t[1].g_dtype, t[1].reserved = mb.MUONH_F32, 1
    assert lib.muonh_adamw_init(ctypes.byref(h), t, 2, None) == mb.MUONH_EINVAL
    t[1].reserved = 0
    for bad in (dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(weight_decay=-1.0)):
        ob = mb.muonh_adamw_options()
        lib.muonh_adamw_default_options(ctypes.byref(ob))
        for k, v in bad.items():
            setattr(ob, k, v)
        assert lib.muonh_adamw_init(ctypes.byref(h), t, 2, ctypes.byref(ob)) == mb.MUONH_EINVAL
        assert lib.muonh_last_error()
    assert not h.value
    assert lib.muonh_adamw_step(None, t, 2, 1e-3, 1, None) == mb.MUONH_EINVAL
    assert lib.muonh_adamw_destroy(None) == mb.MUONH_OK


def test_noalloc_step_host_side_errors():
    """muonh_step_noalloc rejects, before touching any device: a radius that
    is not given, a caller workspace, and a plan larger than its static
    buffer (MUONH_ENOMEM naming both sizes)."""
    lib = pm.load_library()
    assert mb.NOALLOC_MAX_WORKSPACE == 64 << 20
    o = pm.default_options()
    args = mb.muonh_step_args()
    args.elr = 0.01
    d = mb.shape_descs([(64, 96)], radius=0.0)
    assert lib.muonh_step_noalloc(d, 1, ctypes.byref(o), ctypes.byref(args), None) == mb.MUONH_EINVAL
    assert b"radius" in lib.muonh_last_error()
    d = mb.shape_descs([(64, 96)], radius=3.0)
    ow = pm.default_options()
    ow.workspace = 256
    assert lib.muonh_step_noalloc(d, 1, ctypes.byref(ow), ctypes.byref(args), None) == mb.MUONH_EINVAL
    big = [(2048, 2048)] * 2
    assert pm.workspace_size(big) > mb.NOALLOC_MAX_WORKSPACE
    d = mb.shape_descs(big, radius=3.0)
    assert lib.muonh_step_noalloc(d, 2, ctypes.byref(o), ctypes.byref(args), None) == mb.MUONH_ENOMEM
    err = lib.muonh_last_error().decode()
    assert str(pm.workspace_size(big)) in err and str(mb.NOALLOC_MAX_WORKSPACE) in err
    assert lib.muonh_step_noalloc(None, 1, ctypes.byref(o), ctypes.byref(args), None) == mb.MUONH_EINVAL
    assert lib.muonh_step_noalloc(d, 2, None, ctypes.byref(args), None) == mb.MUONH_EINVAL
