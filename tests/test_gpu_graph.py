"""Steps through muonh_step_graph (the step's launches recorded once into a
HIP graph and replayed) against ordinary muonh_step calls and the oracle,
on the MI355X.

The graph reads the step size and the pointer table from device memory, so
replays with a different learning rate, per-matrix scales or new gradient
buffers must give bitwise the results of the ordinary path (same kernels,
same order).  Between replays the test runs unrelated eager work and
synchronises, and it checks every replay, not only the last.
"""

import math

import pytest
import torch

import pretraining_optimizer_amd as pm
from parity import TOL_BF16, TOL_F32, announce, check_reports, run_parity

pytestmark = pytest.mark.gpu

SHAPES = [(300, 200), (128, 640), (515, 515), (1000, 260), (64, 64)]
ETAS = [0.02, 0.011, 0.017, 0.005, 0.013]
SCALES = [None, [1.0, 0.5, 2.0, 0.25, 1.5], None, [0.75, 1.25, 1.0, 0.5, 2.0], None]


def _fns(shapes, gdt, seed):
    def make_w(i):
        g = torch.Generator().manual_seed(seed * 1000 + i)
        r, c = shapes[i]
        w = torch.randn((r, c), generator=g)
        return w * (math.sqrt(r) / torch.linalg.vector_norm(w.double()).item())

    def make_g(k, i):
        g = torch.Generator().manual_seed(seed * 1000 + 100000 * (k + 1) + i)
        return torch.randn(shapes[i], generator=g).to(gdt)

    return make_w, make_g


def _trajectory(ns, graph, mode=pm.MUONH_MODE_HYPERBALL):
    gdt = torch.bfloat16 if ns == "bf16" else torch.float32
    mw, mg = _fns(SHAPES, gdt, seed=11)
    ws = [mw(i).cuda() for i in range(len(SHAPES))]
    ms = [torch.zeros_like(w) for w in ws]
    opt = pm.MuonH(ws, ms, grad_dtype=gdt, mode=mode, weight_decay=0.1,
                   ns_dtype=pm.MUONH_BF16 if ns == "bf16" else pm.MUONH_F32)
    snaps = []
    for k, eta in enumerate(ETAS):
        gs = [mg(k, i).cuda() for i in range(len(SHAPES))]   # new buffers every step
        opt.step(gs, eta, elr_scale=SCALES[k], step=k, graph=graph)
        if graph:
            # unrelated eager work and a synchronisation between replays
            x = torch.randn(1 << 20, device="cuda")
            assert torch.isfinite(x.sum()).item()
        torch.cuda.synchronize()
        snaps.append(([w.clone() for w in ws], [m.clone() for m in ms], opt.stats()))
    opt.close()
    return snaps


@pytest.mark.parametrize("tile", ["auto", "256"])
@pytest.mark.parametrize("ns", ["bf16", "f32"])
@pytest.mark.parametrize("mode", [pm.MUONH_MODE_HYPERBALL, pm.MUONH_MODE_MUON_WD,
                                  pm.MUONH_MODE_ELR_ALIGNED])
def test_graph_replays_match_ordinary_steps(ns, mode, tile, monkeypatch):
    """On the plan's own GEMM path (small-problem, for these shapes) and on
    the 256 x 256 one."""
    if tile != "auto":
        monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"graph replays vs ordinary steps, ns {ns}, mode {mode}, GEMM tile {tile}")
    a = _trajectory(ns, graph=False, mode=mode)
    b = _trajectory(ns, graph=True, mode=mode)
    for k, ((wa, ma, sa), (wb, mb, sb)) in enumerate(zip(a, b)):
        for i, (x, y) in enumerate(zip(wa + ma, wb + mb)):
            assert torch.equal(x, y), (k, i)
        assert sa == sb, k


def test_graph_steps_against_oracle():
    announce("graph steps vs oracle, bf16")
    mw, mg = _fns(SHAPES, torch.bfloat16, seed=12)
    etas = [0.02, 0.01, 0.015]
    reps = run_parity(SHAPES, mw, mg, etas, check=list(range(len(SHAPES))), ns="bf16",
                      graph=True)
    check_reports(reps, TOL_BF16, etas)
    mw, mg = _fns(SHAPES, torch.float32, seed=13)
    reps = run_parity(SHAPES, mw, mg, etas, check=list(range(len(SHAPES))), ns="f32",
                      elr_scale=[1.0, 0.5, 2.0, 0.25, 1.5], graph=True)
    check_reports(reps, TOL_F32, etas)


def test_graph_and_ordinary_steps_interleave():
    """Ordinary and recorded steps on one handle share its state."""
    announce("graph and ordinary steps interleaved")
    outs = []
    for pattern in ((False, False, False, False), (True, False, True, True)):
        mw, mg = _fns(SHAPES, torch.bfloat16, seed=14)
        ws = [mw(i).cuda() for i in range(len(SHAPES))]
        ms = [torch.zeros_like(w) for w in ws]
        opt = pm.MuonH(ws, ms, grad_dtype=torch.bfloat16)
        for k, g in enumerate(pattern):
            opt.step([mg(k, i).cuda() for i in range(len(SHAPES))], ETAS[k], graph=g)
        torch.cuda.synchronize()
        outs.append([w.clone() for w in ws] + [m.clone() for m in ms])
        opt.close()
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_graph_step_refuses_timing():
    announce("graph step with timing on")
    ws = [torch.randn(256, 128, device="cuda")]
    opt = pm.MuonH(ws, [torch.zeros_like(ws[0])], grad_dtype=torch.float32)
    opt.set_timing(True)
    with pytest.raises(pm.MuonHError):
        opt.step([torch.randn(256, 128, device="cuda")], 0.01, graph=True)
    opt.set_timing(False)
    opt.step([torch.randn(256, 128, device="cuda")], 0.01, graph=True)
    torch.cuda.synchronize()
    assert abs(torch.linalg.vector_norm(ws[0].double()).item() / opt.radii()[0] - 1.0) < 1e-5
    opt.close()
