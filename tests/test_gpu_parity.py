"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle on
identical seeded inputs (MI355X only).

Gates: per-matrix relative Frobenius error of u_hat <= 2e-2 (bf16
Newton-Schulz) / 1e-4 (fp32), ||W|| = R to 1e-5 on every matrix after every
step, momentum to 1e-6.
"""

import math

import numpy as np
import pytest
import torch

import inputs
import oracle
import pretraining_optimizer_amd as pm
from parity import (TOL_BF16, TOL_F32, TOL_NORM, announce, check_reports, rel, run_parity,
                    summarize, unit, workload_fns)

pytestmark = pytest.mark.gpu


def _gauss_fns(shapes, gdt, seed=0, gscale=1.0):
    def make_w(i):
        g = torch.Generator().manual_seed(seed * 1000 + i)
        r, c = shapes[i]
        w = torch.randn((r, c), generator=g)
        return w * (math.sqrt(r) / torch.linalg.vector_norm(w.double()).item())

    def make_g(k, i):
        g = torch.Generator().manual_seed(seed * 1000 + 100000 * (k + 1) + i)
        return (gscale * torch.randn(shapes[i], generator=g)).to(gdt)

    return make_w, make_g


@pytest.mark.parametrize("tile", ["auto", "256"])
def test_single_fp32_trajectory(tile, monkeypatch):
    """256x128 fp32, 3 steps, eta 0.01, fp32 Newton-Schulz; on the plan's own
    GEMM path (the small-problem one: a single big tile) and forced onto the
    256 x 256 path."""
    if tile != "auto":
        monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"single fp32 256x128, 3 steps, GEMM tile {tile}")
    wl = inputs.workload("single")
    etas = [wl.eta(k) for k in range(wl.steps)]
    mw, mg = workload_fns(wl)
    reps = run_parity(wl.shapes, mw, mg, etas, check=[0], ns="f32")
    summarize(f"single fp32, tile {tile}", reps)
    check_reports(reps, TOL_F32, etas)


RAGGED = [(300, 200), (128, 640), (1, 37), (37, 1), (515, 515), (257, 1031), (1000, 260), (64, 64)]


@pytest.mark.parametrize("tile", ["64", "256"])
@pytest.mark.parametrize("ns,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_ragged_shapes(ns, tol, tile, monkeypatch):
    """Shapes that span several tiles, ragged tails, vectors, tall and wide, on
    both GEMM paths (64 x 64 tiles over the valid dims; 256 x 256 tiles)."""
    monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"ragged shapes, ns {ns}, GEMM tile {tile}")
    mw, mg = _gauss_fns(RAGGED, torch.bfloat16 if ns == "bf16" else torch.float32, seed=1)
    etas = [0.02, 0.015]
    reps = run_parity(RAGGED, mw, mg, etas, check=list(range(len(RAGGED))), ns=ns)
    summarize(f"ragged {ns}, tile {tile}", reps)
    check_reports(reps, tol, etas)


# Thin SVDs of the stress set's first Newton-Schulz inputs (Y = M_1 = G_0),
# shared by the fp32 and bf16 runs of the stress tests.
_STRESS_SVD = {}


def _stress_svd(i, y):
    if i not in _STRESS_SVD:
        _STRESS_SVD[i] = np.linalg.svd(y, full_matrices=False)
    return _STRESS_SVD[i]


@pytest.mark.parametrize("ns,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_stress_set_trajectory(ns, tol):
    """All 64 stress matrices (aspect 1:1 to 1:8, sides 128-4096, rank-8
    signal with singular values 10^U(-3,1) plus noise) in one grouped launch,
    3 steps at eta 0.02, every matrix followed by the oracle at every step.
    The first step also measures how well u_hat keeps the singular vectors
    of the Newton-Schulz input (off-diagonal energy of U^T u_hat V from the
    SVD of Y): the library's value is gated like u_hat itself, the oracle's
    must vanish to fp64 rounding."""
    announce(f"stress set, ns {ns}, 3 steps, all 64 matrices")
    wl = inputs.workload("stress")
    mw, mg = workload_fns(wl)
    etas = [wl.eta(k) for k in range(wl.steps)]
    reps = run_parity(wl.shapes, mw, mg, etas, check=list(range(len(wl.shapes))), ns=ns,
                      svd_of=_stress_svd)
    out = summarize(f"stress {ns}, 3 steps", reps)
    check_reports(reps, tol, etas)
    sv = reps[0].sv_err
    assert len(sv) == len(wl.shapes)
    for i, (lib, ora) in sv.items():
        assert lib <= tol, (i, lib)
        assert ora <= 1e-11, (i, ora)
    announce(f"stress {ns}: singular-vector agreement max {out['sv_lib']:.3e} "
             f"(oracle {out['sv_oracle']:.1e}) over {len(sv)} matrices")


@pytest.mark.parametrize("ns,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_stress_set_small_gemm_path(ns, tol, monkeypatch):
    """The 64 stress matrices (dims 128-4096, ragged) forced onto the
    small-problem GEMM path, one step, every matrix checked."""
    monkeypatch.setenv("MUONH_GEMM_TILE", "64")
    announce(f"stress set on the 64 x 64 GEMM path, ns {ns}, 1 step")
    wl = inputs.workload("stress")
    mw, mg = workload_fns(wl)
    reps = run_parity(wl.shapes, mw, mg, [wl.eta(0)], check=list(range(len(wl.shapes))), ns=ns)
    summarize(f"stress {ns}, 64-tile path", reps)
    check_reports(reps, tol, [wl.eta(0)])


@pytest.mark.parametrize("ns,tol,tile", [("bf16", TOL_BF16, "256"), ("f32", TOL_F32, "256"),
                                         ("bf16", TOL_BF16, "64")])
def test_maximum_dimension(ns, tol, tile, monkeypatch):
    """Matrices at the largest supported side, 65536 (tall and wide): a
    contraction of 1024 K stages and 256 (1024 small) column tiles."""
    monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"maximum dimension 65536, ns {ns}, GEMM tile {tile}")
    shapes = [(65536, 96), (100, 65536)]
    mw, mg = _gauss_fns(shapes, torch.bfloat16 if ns == "bf16" else torch.float32, seed=21)
    reps = run_parity(shapes, mw, mg, [0.02], check=[0, 1], ns=ns)
    summarize(f"max dimension {ns}, tile {tile}", reps)
    check_reports(reps, tol, [0.02])


@pytest.mark.parametrize("tile", ["64", "256"])
@pytest.mark.parametrize("ns", ["f32", "bf16"])
def test_rank_one_gradient_gives_its_outer_product(ns, tile, monkeypatch):
    """A rank-1 gradient G = x y^T has one singular value, so the
    Newton-Schulz output is a multiple of x y^T and u_hat = x y^T / (|x||y|):
    a closed form checked on the GPU path directly, not through the oracle.
    x and y are small integers, so G is exactly rank 1 in fp32 and bf16.

    Each B'X product keeps an iterate rank 1, but rounding it to the
    operand type adds full-rank noise, and the remaining iterations multiply
    small singular values by about 3.4 each (the iteration is built to grow
    them).  In fp32 that leaves |u_hat - x y^T| below 1e-3.  In bf16 the
    first rounding (2^-9) grows into spurious singular values of 0.08-0.12
    next to the main one (0.7), on either GEMM path: the bf16 iteration
    orthogonalises its own rounding error on an exactly rank-deficient input
    (measured cosines 0.977 and 0.991 for these shapes).  What is checked
    there is that the rank-1 direction dominates (cosine >= 0.95)."""
    monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"rank-1 gradient, ns {ns}, GEMM tile {tile}")
    gen = torch.Generator().manual_seed(31)
    for r, c in [(512, 384), (300, 1000)]:
        x = torch.randint(-8, 9, (r, 1), generator=gen).double()
        y = torch.randint(-8, 9, (c, 1), generator=gen).double()
        x[0, 0], y[0, 0] = 5.0, -3.0   # never all zero
        g = (x @ y.T).float()           # |entries| <= 64: exact in fp32 and bf16
        w = torch.randn(r, c, generator=gen)
        w = (w * (math.sqrt(r) / w.norm())).cuda()
        m = torch.zeros_like(w)
        gdt = torch.bfloat16 if ns == "bf16" else torch.float32
        opt = pm.MuonH([w], [m], grad_dtype=gdt,
                       ns_dtype=pm.MUONH_BF16 if ns == "bf16" else pm.MUONH_F32)
        opt.step([g.to(gdt).cuda()], 0.01)
        u = opt.copy_update(0).double().cpu()
        torch.cuda.synchronize()
        opt.close()
        uh, v = u / u.norm(), (x @ y.T) / (x.norm() * y.norm())
        if ns == "f32":
            assert (uh - v).norm().item() <= 1e-3, (r, c)
        else:
            assert (uh * v).sum().item() >= 0.95, (r, c)


def test_diag170m_trajectory():
    """170M-class set (84 matrices, bf16 grads scaled by 1/sqrt(fan_in)), all 20
    steps of the linear ELR decay; the oracle checks every matrix at the first
    step and follows layers 0 and 11 through all 20."""
    announce("diag170m, 20 steps")
    wl = inputs.workload("diag170m")
    mw, mg = workload_fns(wl)
    etas = [wl.eta(k) for k in range(wl.steps)]
    check = list(range(7)) + list(range(77, 84))
    reps = run_parity(wl.shapes, mw, mg, etas, check=check, ns="bf16",
                      check_first=range(len(wl.shapes)))
    summarize("diag170m bf16, 20 steps", reps)
    check_reports(reps, TOL_BF16, etas)
    assert len(reps[0].u_err) == 84


def test_qwen3_06b_trajectory():
    """Qwen3-0.6B set (196 matrices), all 10 steps of the linear decay from
    0.024; the oracle checks all 196 matrices at the first step and follows
    the seven of layer 0 through all 10."""
    announce("qwen3-0.6b set, 10 steps")
    wl = inputs.workload("qwen3_0.6b")
    mw, mg = workload_fns(wl)
    etas = [wl.eta(k) for k in range(wl.steps)]
    reps = run_parity(wl.shapes, mw, mg, etas, check=list(range(7)), ns="bf16",
                      check_first=range(len(wl.shapes)))
    summarize("qwen3_0.6b bf16, 10 steps", reps)
    check_reports(reps, TOL_BF16, etas)
    assert len(reps[0].u_err) == 196


def test_qwen3_17b_full_size():
    """The benchmarked configuration (196 Qwen3-1.7B matrices, bf16 NS) in the
    same launch configuration the benchmark times, all 10 steps; the oracle
    follows all seven matrices of layer 0 and q, k, v, o of layers 13 and 27
    (each an exact check, matrices being independent), and the norm
    invariant is checked on all 196 matrices after every step.  Every other
    matrix is checked at the first step by test_qwen3_17b_every_matrix."""
    announce("qwen3-1.7b full set, 10 steps")
    wl = inputs.workload("qwen3_1.7b")
    mw, mg = workload_fns(wl)
    etas = [wl.eta(k) for k in range(wl.steps)]
    check = list(range(7)) + [7 * l + j for l in (13, 27) for j in range(4)]
    reps = run_parity(wl.shapes, mw, mg, etas, check=check, ns="bf16")
    summarize("qwen3_1.7b bf16, 10 steps, followed subset", reps)
    check_reports(reps, TOL_BF16, etas)
    for rep in reps:
        assert len(rep.norm_err) == 196


@pytest.mark.parametrize("layers", [(0, 7), (7, 14), (14, 21), (21, 28)])
def test_qwen3_17b_every_matrix(layers):
    """The first step of the benchmarked 1.7B set (all 196 matrices in one
    grouped launch per product, as the benchmark runs it), with the oracle
    checking every matrix of seven layers: together the four cases cover
    all 196, including gate, up and down beyond layer 0 (whose tiles sit at
    other positions of the tile lists and other partial-slot offsets)."""
    l0, l1 = layers
    announce(f"qwen3-1.7b full set, first step, layers {l0}-{l1 - 1}")
    wl = inputs.workload("qwen3_1.7b")
    mw, mg = workload_fns(wl)
    reps = run_parity(wl.shapes, mw, mg, [wl.eta(0)], check=[], ns="bf16",
                      check_first=range(7 * l0, 7 * l1))
    summarize(f"qwen3_1.7b bf16, first step, layers {l0}-{l1 - 1}", reps)
    check_reports(reps, TOL_BF16, [wl.eta(0)])
    assert len(reps[0].u_err) == 7 * (l1 - l0) and len(reps[0].norm_err) == 196


def test_qwen3_17b_fp32_newton_schulz():
    """The benchmarked 1.7B set with the fp32 Newton-Schulz path (fp32 MFMA,
    X and X^T both stored), all 10 steps; the oracle follows the seven
    matrices of layers 0 and 27 to the fp32 tolerance and the norm invariant
    is checked on all 196 matrices."""
    announce("qwen3-1.7b full set, fp32 Newton-Schulz, 10 steps")
    wl = inputs.workload("qwen3_1.7b")
    mw, mg = workload_fns(wl)
    etas = [wl.eta(k) for k in range(wl.steps)]
    reps = run_parity(wl.shapes, mw, mg, etas, check=list(range(7)) + list(range(189, 196)), ns="f32")
    summarize("qwen3_1.7b fp32, 10 steps, layers 0 and 27", reps)
    check_reports(reps, TOL_F32, etas)
    for rep in reps:
        assert len(rep.norm_err) == 196


def test_qwen3_17b_fused_projections():
    """Qwen3-1.7B dims with fused qkv (4096 x 2048) and gate_up (12288 x 2048)
    matrices: wider Newton-Schulz problems (n up to 12288) in the same grouped
    launches; the oracle checks the four matrices of layers 0 and 27."""
    announce("qwen3-1.7b fused projections, 1 step")
    wl = inputs.workload("qwen3_1.7b_fused")
    mw, mg = workload_fns(wl)
    etas = [wl.eta(0)]
    reps = run_parity(wl.shapes, mw, mg, etas, check=list(range(4)) + list(range(108, 112)), ns="bf16")
    summarize("qwen3_1.7b_fused bf16, first step, layers 0 and 27", reps)
    check_reports(reps, TOL_BF16, etas)
    for rep in reps:
        assert len(rep.norm_err) == 112


def test_stats_match_oracle_diagnostics():
    announce("stats vs oracle diagnostics")
    shapes = [(256, 512), (700, 300)]
    mw, mg = _gauss_fns(shapes, torch.float32, seed=2)
    reps = run_parity(shapes, mw, mg, [0.03], check=[0, 1], ns="f32")
    rep = reps[0]
    for i, (u, d) in enumerate(rep.oracle_diag):
        s = rep.stats[i]
        assert s["nonfinite"] == 0
        assert s["u_norm"] == pytest.approx(np.linalg.norm(u), rel=1e-4)
        assert s["elr"] == pytest.approx(0.03, rel=1e-5)
        assert s["c"] == pytest.approx(d.c, abs=1e-4)
        assert s["angle"] == pytest.approx(d.angle, rel=1e-4)
        assert s["wt_norm"] == pytest.approx(d.wt_norm, rel=1e-5)


def test_zero_gradient_projects_only():
    announce("zero gradient")
    dev = torch.device("cuda")
    w = torch.randn(96, 160, device=dev)
    w0 = w.clone()
    m = torch.zeros_like(w)
    opt = pm.MuonH([w], [m], grad_dtype=torch.float32, radii=[5.0])
    opt.step([torch.zeros_like(w)], 0.05)
    s = opt.stats()[0]
    assert s["u_norm"] == 0.0 and s["nonfinite"] == 0
    expect = 5.0 * w0.double() / torch.linalg.vector_norm(w0.double())
    assert torch.allclose(w.double(), expect, rtol=1e-5, atol=1e-6)
    assert opt.radii()[0] == 5.0
    opt.close()


def test_nonfinite_gradient_propagates_and_is_flagged():
    announce("non-finite gradient")
    dev = torch.device("cuda")
    ws = [torch.randn(128, 256, device=dev), torch.randn(64, 64, device=dev)]
    ms = [torch.zeros_like(w) for w in ws]
    opt = pm.MuonH(ws, ms, grad_dtype=torch.bfloat16)
    gs = [torch.randn(128, 256, device=dev).bfloat16(), torch.randn(64, 64, device=dev).bfloat16()]
    gs[0][3, 7] = float("nan")
    opt.step(gs, 0.01)
    st = opt.stats()
    assert st[0]["nonfinite"] == 1 and torch.isnan(ws[0]).all()
    assert st[1]["nonfinite"] == 0 and torch.isfinite(ws[1]).all()
    opt.close()


@pytest.mark.parametrize("tile", ["256", "64"])
def test_bitwise_deterministic(tile, monkeypatch):
    """Two runs give bitwise the same W and M, on either GEMM path."""
    monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"determinism, GEMM tile {tile}")
    wl = inputs.workload("diag170m")
    outs = []
    for _ in range(2):
        ws = [inputs.make_weight(wl, i, "cuda") for i in range(14)]
        ms = [torch.zeros_like(w) for w in ws]
        opt = pm.MuonH(ws, ms, grad_dtype=torch.bfloat16)
        for k in range(2):
            opt.step([inputs.make_grad(wl, k, i, "cuda") for i in range(14)], wl.eta(k))
        torch.cuda.synchronize()
        outs.append(([w.clone() for w in ws], [m.clone() for m in ms]))
        opt.close()
    for a, b in zip(outs[0][0] + outs[0][1], outs[1][0] + outs[1][1]):
        assert torch.equal(a, b)


def test_symmetric_and_full_tiles_agree(monkeypatch):
    monkeypatch.setenv("MUONH_GEMM_TILE", "256")   # the option belongs to the 256 x 256 path
    announce("symmetric vs full Gram tiles")
    shapes = [(512, 768), (1024, 300)]
    mw, mg = _gauss_fns(shapes, torch.bfloat16, seed=3)
    a = run_parity(shapes, mw, mg, [0.02], check=[0, 1], ns="bf16", symmetric=1)
    b = run_parity(shapes, mw, mg, [0.02], check=[0, 1], ns="bf16", symmetric=0)
    check_reports(a, TOL_BF16, [0.02])
    check_reports(b, TOL_BF16, [0.02])


@pytest.mark.parametrize("tile", ["auto", "256"])
@pytest.mark.parametrize("ns,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
@pytest.mark.parametrize("mode", [pm.MUONH_MODE_MUON_WD, pm.MUONH_MODE_ELR_ALIGNED])
def test_other_update_modes(mode, ns, tol, tile, monkeypatch):
    """Ordinary Muon with decoupled weight decay (Eq. 3) and ELR-aligned Muon
    (Eq. 5), with fp32 and bf16 Newton-Schulz, on the plan's own GEMM path
    and on the 256 x 256 one.  Both updates are linear in u, so W's error is
    at most the step size times u's (plus fp32 rounding of W)."""
    if tile != "auto":
        monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"mode {mode}, ns {ns}, GEMM tile {tile}")
    shapes = [(256, 384), (640, 256)]
    gdt = torch.float32 if ns == "f32" else torch.bfloat16
    mw, mg = _gauss_fns(shapes, gdt, seed=4)
    etas = [0.02, 0.01]
    reps = run_parity(shapes, mw, mg, etas, check=[0, 1], ns=ns, mode=mode, weight_decay=0.1)
    summarize(f"mode {mode} {ns}, tile {tile}", reps)
    acc = 0.0
    for rep in reps:
        acc += etas[rep.step]
        assert max(rep.u_err) <= tol
        # Eq. (3): W moves by eta u, |u| = ||u^|| sqrt(rows) scale; Eq. (5):
        # by eta ||W|| u^.  Relative to ||W|| both are O(eta) times u^'s error.
        assert max(rep.w_err) <= 2.0 * acc * tol + 1e-5, (rep.step, rep.w_err)
        if mode == pm.MUONH_MODE_ELR_ALIGNED:
            for s, eta in zip(rep.stats, etas):
                assert s["elr"] == pytest.approx(etas[rep.step], rel=1e-5)


@pytest.mark.parametrize("mode", [pm.MUONH_MODE_MUON_WD, pm.MUONH_MODE_ELR_ALIGNED])
def test_other_modes_zero_gradient_beside_a_live_one(mode):
    """A zero gradient in the Eq. (3) and Eq. (5) modes, in the same step as a
    matrix with a live gradient: u = 0 leaves only the decay (Eq. 3) or W
    unchanged with eta_t = 0 (Eq. 5), the other matrix follows the oracle, and
    nothing is flagged non-finite."""
    announce(f"zero gradient beside a live one, mode {mode}")
    eta, lam = 0.02, 0.1
    shapes = [(96, 160), (192, 128)]
    mw, mg = _gauss_fns(shapes, torch.float32, seed=9)
    w0 = [mw(i) for i in range(2)]
    g = [torch.zeros(shapes[0]), mg(0, 1)]
    ws = [w.cuda() for w in w0]
    ms = [torch.zeros_like(w) for w in ws]
    opt = pm.MuonH(ws, ms, grad_dtype=torch.float32, ns_dtype=pm.MUONH_F32, mode=mode,
                   weight_decay=lam)
    opt.step([x.cuda() for x in g], eta)
    st = opt.stats()
    u1 = opt.copy_update(1).cpu().double().numpy()
    torch.cuda.synchronize()
    opt.close()
    assert all(x["nonfinite"] == 0 for x in st)
    assert st[0]["u_norm"] == 0.0 and st[0]["elr"] == 0.0
    y1 = oracle.ns_input(oracle.momentum_update(np.zeros(shapes[1]), g[1].numpy(), 0.95),
                         g[1].numpy(), 0.95, False)
    u1_ref = oracle.newton_schulz(y1)
    assert rel(unit(u1), unit(u1_ref)) <= TOL_F32
    if mode == pm.MUONH_MODE_MUON_WD:
        ref = [oracle.muon_wd_update(w0[0].numpy(), np.zeros(shapes[0]), eta, lam),
               oracle.muon_wd_update(w0[1].numpy(), u1_ref, eta, lam)]
    else:
        ref = [oracle.elr_aligned_update(w0[0].numpy(), np.zeros(shapes[0]), eta)[0],
               oracle.elr_aligned_update(w0[1].numpy(), u1_ref, eta)[0]]
        assert torch.equal(ws[0].cpu(), w0[0])
        assert st[1]["elr"] == pytest.approx(eta, rel=1e-5)
    for w, r in zip(ws, ref):
        assert rel(w.cpu().double().numpy(), r) <= 1e-5


@pytest.mark.parametrize("tile", ["auto", "256"])
def test_nesterov_and_elr_scale_and_resume_radius(tile, monkeypatch):
    if tile != "auto":
        monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"nesterov + per-matrix elr scale + given radii, GEMM tile {tile}")
    shapes = [(256, 256), (300, 512)]
    mw, mg = _gauss_fns(shapes, torch.float32, seed=5)
    reps = run_parity(shapes, mw, mg, [0.02, 0.02], check=[0, 1], ns="f32",
                      oracle_opts=oracle.OracleOptions(nesterov=True),
                      elr_scale=[1.0, 0.5], radii=[10.0, 7.5])
    check_reports(reps, TOL_F32, [0.02, 0.02])


@pytest.mark.parametrize("ns,steps,coeffs,beta", [
    ("f32", 1, "quintic", 0.95), ("bf16", 1, "quintic", 0.95),
    ("f32", 2, "quintic", 0.95), ("bf16", 3, "quintic", 0.95),
    ("bf16", 6, "quintic", 0.95), ("f32", 5, "classical", 0.9),
    ("bf16", 4, "classical", 0.9),
])
@pytest.mark.parametrize("tile", ["auto", "256"])
def test_iteration_count_and_coefficients(ns, steps, coeffs, beta, tile, monkeypatch):
    """The options the ABI takes beside the defaults: other Newton-Schulz
    iteration counts (one iteration makes a single B'X launch both the first,
    which applies the normalisation, and the last, which writes u and the
    update statistics; odd and even counts end in different iterate
    buffers), the classical cubic-equivalent coefficients (15/8, -10/8, 3/8)
    and another momentum coefficient, against the oracle with the same
    options (a plain reading of the iteration the arXiv page's Section 3.3
    update wraps, whatever its length)."""
    if tile != "auto":
        monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"{steps} NS steps, {coeffs} coefficients, beta {beta}, {ns} NS, GEMM tile {tile}")
    shapes = [(300, 512), (640, 256), (256, 256), (129, 1000)]
    mw, mg = _gauss_fns(shapes, torch.bfloat16 if ns == "bf16" else torch.float32, seed=17 + steps)
    oo = oracle.OracleOptions(
        beta=beta, ns_steps=steps,
        ns_coeffs=oracle.NS_COEFFS_QUINTIC if coeffs == "quintic" else oracle.NS_COEFFS_CLASSICAL)
    etas = [0.03, 0.02]
    reps = run_parity(shapes, mw, mg, etas, check=list(range(len(shapes))), ns=ns, oracle_opts=oo)
    summarize(f"{steps} NS steps, {coeffs}, beta {beta}, {ns}, tile {tile}", reps)
    check_reports(reps, TOL_BF16 if ns == "bf16" else TOL_F32, etas)


@pytest.mark.parametrize("tile", ["auto", "256"])
def test_resume_from_saved_state_is_bitwise(tile, monkeypatch):
    """All state is the caller's (W, M) plus the radii: 3 steps, a new handle
    built from the saved W, M and R (muonh_get_radii passed back as the
    descriptors' radius), 2 more steps -- bitwise the same as 5 steps on one
    handle."""
    if tile != "auto":
        monkeypatch.setenv("MUONH_GEMM_TILE", tile)
    announce(f"resume from saved state, GEMM tile {tile}")
    shapes = [(300, 200), (128, 640), (515, 515)]
    mw, mg = _gauss_fns(shapes, torch.bfloat16, seed=41)
    etas = [0.02, 0.015, 0.012, 0.01, 0.008]

    def run(split):
        ws = [mw(i).cuda() for i in range(len(shapes))]
        ms = [torch.zeros_like(w) for w in ws]
        opt = pm.MuonH(ws, ms, grad_dtype=torch.bfloat16)
        for k, eta in enumerate(etas):
            if k == split:
                radii = opt.radii()
                saved_w = [w.clone() for w in ws]
                saved_m = [m.clone() for m in ms]
                opt.close()
                del ws, ms
                torch.cuda.synchronize()
                ws, ms = saved_w, saved_m
                opt = pm.MuonH(ws, ms, grad_dtype=torch.bfloat16, radii=radii)
            opt.step([mg(k, i).cuda() for i in range(len(shapes))], eta, step=k)
        torch.cuda.synchronize()
        out = [w.clone() for w in ws] + [m.clone() for m in ms]
        opt.close()
        return out

    for a, b in zip(run(split=None), run(split=3)):
        assert torch.equal(a, b)


def test_step_list_mismatch_is_rejected():
    announce("mismatch errors")
    dev = torch.device("cuda")
    ws = [torch.randn(64, 64, device=dev)]
    opt = pm.MuonH(ws, [torch.zeros_like(ws[0])], grad_dtype=torch.float32)
    with pytest.raises(ValueError):
        opt.step([torch.randn(64, 32, device=dev)], 0.01)
    import ctypes
    from pretraining_optimizer_amd import muonh as mb
    lib = pm.load_library()
    d = (mb.muonh_matrix_desc * 1)()
    d[0].w = ws[0].data_ptr(); d[0].g = ws[0].data_ptr(); d[0].m = ws[0].data_ptr()
    d[0].rows, d[0].cols, d[0].g_dtype = 64, 65, mb.MUONH_F32
    args = mb.muonh_step_args(); args.elr = 0.01
    assert lib.muonh_step(opt._h, d, 1, ctypes.byref(args), None) == mb.MUONH_EMISMATCH
    d[0].cols = 64
    assert lib.muonh_step(opt._h, d, 2, ctypes.byref(args), None) == mb.MUONH_EMISMATCH
    d[0].g = ws[0].data_ptr() + 4   # misaligned
    assert lib.muonh_step(opt._h, d, 1, ctypes.byref(args), None) == mb.MUONH_EINVAL
    opt.close()


def test_iterate_beyond_2gib_signed_permutation():
    """A 32768 x 33024 matrix, so the bf16 iterate X (2.17 GB) spans more than
    2^31 bytes and the operand walking X along K must rebase its addresses.
    G is a signed permutation of the first 32768 columns (the rest zero): its
    rows are orthogonal with equal norms, so X X^T, A A and B' are multiples
    of I at every iteration, every product keeps X proportional to G and each
    bf16 rounding is a uniform scaling.  Hence u^ = G/||G|| to fp32 rounding
    at any size (the polynomial acts on one repeated singular value), the
    zero columns stay exactly zero, and W follows the Hyperball closed form
    with ||W|| = R."""
    announce("iterate > 2 GiB: 32768 x 33024 signed permutation")
    dev = torch.device("cuda")
    r, c = 32768, 33024
    gen = torch.Generator(device=dev).manual_seed(7)
    perm = torch.randperm(r, generator=gen, device=dev)
    sign = torch.randint(0, 2, (r,), generator=gen, device=dev).to(torch.bfloat16) * 2 - 1
    g = torch.zeros((r, c), device=dev, dtype=torch.bfloat16)
    g[torch.arange(r, device=dev), perm] = sign
    w = torch.randn((r, c), generator=gen, device=dev)
    m = torch.zeros_like(w)
    R = float(torch.linalg.vector_norm(w, dtype=torch.float64))
    eta = 0.02
    opt = pm.MuonH([w], [m], grad_dtype=torch.bfloat16)
    assert abs(opt.radii()[0] / R - 1.0) < 1e-6
    w_tilde = w.double()                       # W_0 in fp64; the step updates w in place
    opt.step([g], eta)
    u = opt.copy_update(0)
    torch.cuda.synchronize()
    assert torch.equal(m, g.float())           # M = beta * 0 + G
    assert bool((u[:, r:] == 0).all())
    uhat = u / torch.linalg.vector_norm(u, dtype=torch.float64).item()
    ghat = g.float() / float(r) ** 0.5
    err = torch.linalg.vector_norm((uhat - ghat).double()).item()
    announce(f"u^ error {err:.3e}")
    assert err <= 1e-5, err
    del uhat, u
    w_tilde.sub_(ghat.double(), alpha=eta * R)
    w_exp = w_tilde.mul_(R / torch.linalg.vector_norm(w_tilde).item())
    werr = (torch.linalg.vector_norm(w.double() - w_exp) / R).item()
    wn = torch.linalg.vector_norm(w, dtype=torch.float64).item()
    announce(f"W error {werr:.3e}, |W|/R - 1 {wn / R - 1:.2e}")
    assert werr <= 1e-5 and abs(wn / R - 1.0) <= TOL_NORM
    assert opt.stats()[0]["nonfinite"] == 0
    opt.close()


def test_debug_sync_and_log_flags(monkeypatch, capfd):
    """MUONH_DEBUG_SYNC=1 (a synchronisation after every launch) gives
    bitwise the same steps as the asynchronous path, and MUONH_LOG=1 prints
    the plan at init."""
    announce("MUONH_DEBUG_SYNC / MUONH_LOG")
    shapes = [(300, 200), (128, 640)]
    mw, mg = _gauss_fns(shapes, torch.bfloat16, seed=6)
    outs = []
    for flags in ({}, {"MUONH_DEBUG_SYNC": "1", "MUONH_LOG": "1"}):
        for name in ("MUONH_DEBUG_SYNC", "MUONH_LOG"):
            monkeypatch.delenv(name, raising=False)
        for name, value in flags.items():
            monkeypatch.setenv(name, value)
        ws = [mw(i).cuda() for i in range(len(shapes))]
        ms = [torch.zeros_like(w) for w in ws]
        opt = pm.MuonH(ws, ms, grad_dtype=torch.bfloat16)
        for k in range(2):
            opt.step([mg(k, i).cuda() for i in range(len(shapes))], 0.02)
        torch.cuda.synchronize()
        opt.close()
        outs.append([w.clone() for w in ws] + [m.clone() for m in ms])
    err = capfd.readouterr().err
    assert "muonh: 2 matrices" in err, err
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_steps_on_a_side_stream():
    """Steps enqueued on a stream other than torch's current one, with each
    step's gradients dropped right after the call (the binding records them
    on that stream), give bitwise the results of the current-stream path."""
    announce("side stream")
    shapes = [(256, 384), (640, 256)]
    mw, mg = _gauss_fns(shapes, torch.bfloat16, seed=8)
    outs = []
    for side in (False, True):
        ws = [mw(i).cuda() for i in range(len(shapes))]
        ms = [torch.zeros_like(w) for w in ws]
        s = torch.cuda.Stream() if side else None
        if side:
            s.wait_stream(torch.cuda.current_stream())
        opt = pm.MuonH(ws, ms, grad_dtype=torch.bfloat16, stream=s)
        for k in range(3):
            gs = [mg(k, i).cuda() for i in range(len(shapes))]
            if side:
                s.wait_stream(torch.cuda.current_stream())
            opt.step(gs, 0.02, stream=s)
            del gs
        if side:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        opt.close()
        outs.append([w.clone() for w in ws] + [m.clone() for m in ms])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_init_on_a_side_stream_then_steps_on_the_current_one():
    """The handle orders its own work across streams: init (workspace
    clearing, radius kernels) enqueued on a side stream, then steps and
    copies of u on torch's current stream with no synchronisation in
    between, then a copy of u on the side stream after a step on the current
    one, give bitwise the results of doing everything on one stream."""
    announce("init on a side stream, steps on the current stream")
    shapes = [(512, 768), (1000, 260)]
    mw, mg = _gauss_fns(shapes, torch.bfloat16, seed=12)
    outs = []
    for mixed in (False, True):
        ws = [mw(i).cuda() for i in range(len(shapes))]
        ms = [torch.zeros_like(w) for w in ws]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())   # W and M are ready
        opt = pm.MuonH(ws, ms, grad_dtype=torch.bfloat16, stream=side if mixed else None)
        us = []
        for k in range(3):
            opt.step([mg(k, i).cuda() for i in range(len(shapes))], 0.02)
            if mixed and k == 1:
                u = opt.copy_update(0, stream=side)   # ordered after the step by the library
                torch.cuda.current_stream().wait_stream(side)
            else:
                u = opt.copy_update(0)
            us.append(u)
        torch.cuda.synchronize()
        R = opt.radii()
        opt.close()
        outs.append([w.clone() for w in ws] + [m.clone() for m in ms] + us + [torch.tensor(R)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
