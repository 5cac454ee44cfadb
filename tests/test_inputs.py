"""Host-side checks of the synthetic workloads (CPU only)."""

import math

import torch

import inputs


def test_workload_param_counts():
    assert inputs.workload("single").params() == 256 * 128
    assert inputs.workload("diag170m").params() == 12 * (4 * 768 * 768 + 3 * 2048 * 768)
    assert len(inputs.workload("qwen3_0.6b").shapes) == 196
    assert inputs.workload("qwen3_0.6b").params() == 28 * (2048 * 1024 + 2 * 1024 * 1024 + 1024 * 2048 + 3 * 3072 * 1024)
    w = inputs.workload("qwen3_1.7b")
    assert len(w.shapes) == 196
    assert w.params() == 28 * (2 * 2048 * 2048 + 2 * 1024 * 2048 + 3 * 6144 * 2048)


def test_fused_workload_has_the_split_parameters():
    split = inputs.workload("qwen3_1.7b")
    fused = inputs.workload("qwen3_1.7b_fused")
    assert len(fused.shapes) == 28 * 4
    assert fused.params() == split.params()
    assert fused.shapes[:4] == [(4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144)]


def test_stress_shapes():
    shapes = inputs.workload("stress").shapes
    assert len(shapes) == 64
    for i, (r, c) in enumerate(shapes):
        s, l = min(r, c), max(r, c)
        assert 128 <= s <= l <= 4096
        assert l / s <= 8.0 + 1e-9
        if s != l:
            assert (r < c) == (i % 2 == 0)
    odd = sum(1 for r, c in shapes for d in (r, c) if d % 16)
    assert odd > 64


def test_weights_are_seeded_and_on_radius():
    wl = inputs.workload("diag170m")
    a = inputs.make_weight(wl, 5)
    b = inputs.make_weight(wl, 5)
    assert torch.equal(a, b)
    assert abs(torch.linalg.vector_norm(a.double()).item() / math.sqrt(a.shape[0]) - 1.0) < 1e-6
    g1 = inputs.make_grad(wl, 0, 5)
    g2 = inputs.make_grad(wl, 1, 5)
    assert g1.dtype == torch.bfloat16 and not torch.equal(g1, g2)


def test_single_workload_radius():
    wl = inputs.workload("single")
    w = inputs.make_weight(wl, 0)
    assert abs(torch.linalg.vector_norm(w.double()).item() - 16.0) < 1e-5


def test_lowrank_grad_spectrum():
    wl = inputs.workload("stress")
    g = inputs.to_numpy64(inputs.make_grad(wl, 0, 0))
    import numpy as np
    s = np.linalg.svd(g, compute_uv=False)
    noise = math.sqrt(1e-3) * (math.sqrt(g.shape[0]) + math.sqrt(g.shape[1]))
    assert s[8] <= 1.2 * noise


def test_adamw_group_sizes():
    g = inputs.adamw_group("qwen3_1.7b")
    assert g.params() == 2 * 151936 * 2048 + 28 * (2 * 2048 + 2 * 128) + 2048
    total = g.params() + inputs.workload("qwen3_1.7b").params()
    assert 1.95e9 < total < 2.1e9          # "about 2B parameters", untied
    r = inputs.adamw_group("ragged_f32")
    p = inputs.make_adamw_param(r, 0)
    assert p.dtype == torch.float32 and p.numel() == r.numels()[0]
    assert inputs.make_adamw_grad(r, 1, 3).dtype == torch.float32
    assert torch.equal(inputs.make_adamw_grad(r, 1, 3), inputs.make_adamw_grad(r, 1, 3))
    assert not torch.equal(inputs.make_adamw_grad(r, 1, 3), inputs.make_adamw_grad(r, 2, 3))
