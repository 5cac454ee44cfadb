"""GPU parity of the AdamW step (the parameters MuonH does not wrap) through
the C ABI against the fp64 oracle, on identical seeded inputs (MI355X only).

Tolerance, from the fp32 arithmetic of the kernel (a handful of roundings per
element and step, unit roundoff 2^-24): after K steps, elementwise
  |W - W_oracle| <= K (2.4e-7 |W_oracle| + 3e-6 lr_max)
  |m - m_oracle| <= K 2.4e-7 (|m_oracle| + 0.1 max|g|),  v likewise with 0.05 g^2.
|m_hat| / (sqrt(v_hat) + eps) is at most a few units for these betas, so an
error in the update rule (a missing bias correction, eps inside the square
root, decay after the step) is orders of magnitude above the bound.
"""

import numpy as np
import pytest
import torch

import inputs
import oracle
import pretraining_optimizer_amd as pm
from parity import announce

pytestmark = pytest.mark.gpu

OPTS = oracle.AdamWOptions(beta1=0.9, beta2=0.95, eps=1e-12, weight_decay=0.1)


def _check(w, m, v, w_ref, m_ref, v_ref, gmax, steps, lr_max, what):
    tol_w = steps * (2.4e-7 * np.abs(w_ref) + 3e-6 * lr_max)
    tol_m = steps * 2.4e-7 * (np.abs(m_ref) + 0.1 * gmax)
    tol_v = steps * 2.4e-7 * (np.abs(v_ref) + 0.05 * gmax * gmax)
    for name, a, b, t in (("w", w, w_ref, tol_w), ("m", m, m_ref, tol_m), ("v", v, v_ref, tol_v)):
        err = np.abs(a - b)
        bad = err > t
        assert not bad.any(), (f"{what}: {name} off at {int(bad.sum())} of {a.size} elements, "
                               f"worst {float((err - t).max()):.3e} over the bound")


def _run_group(grp, steps, dev):
    n = len(grp.tensors)
    ws = [inputs.make_adamw_param(grp, i, dev) for i in range(n)]
    w0 = [w.clone() for w in ws]
    ms = [torch.zeros_like(w) for w in ws]
    vs = [torch.zeros_like(w) for w in ws]
    opt = pm.AdamW(ws, ms, vs, grad_dtype=grp.g_dtype)
    grads = []
    for k in range(steps):
        gs = [inputs.make_adamw_grad(grp, k, i, dev) for i in range(n)]
        opt.step(gs, grp.lr(k), k + 1)
        grads.append(gs)
    torch.cuda.synchronize()
    opt.close()
    return w0, ws, ms, vs, grads


@pytest.mark.parametrize("name", ["ragged_bf16", "ragged_f32"])
def test_ragged_tensors_every_element(name):
    """Sizes 1 .. 70001 (not multiples of 4, one chunk and several), 4 steps of a
    decaying LR; every element against the oracle."""
    announce(f"adamw {name}, 4 steps")
    grp = inputs.adamw_group(name)
    dev = torch.device("cuda")
    w0, ws, ms, vs, grads = _run_group(grp, grp.steps, dev)
    lrs = [grp.lr(k) for k in range(grp.steps)]
    for i in range(len(grp.tensors)):
        g64 = [inputs.to_numpy64(gs[i]) for gs in grads]
        w_ref, m_ref, v_ref = oracle.adamw_trajectory(inputs.to_numpy64(w0[i]), g64, lrs, OPTS)
        gmax = max(float(np.abs(g).max()) for g in g64)
        _check(inputs.to_numpy64(ws[i]), inputs.to_numpy64(ms[i]), inputs.to_numpy64(vs[i]),
               w_ref, m_ref, v_ref, gmax, grp.steps, max(lrs), f"{name} tensor {i}")


def test_qwen3_17b_group_full_size_sampled():
    """The whole AdamW group of the untied Qwen3-1.7B model (0.62 G params,
    embedding and LM head 311 M each) in one launch per step, 2 steps; the
    oracle checks 65536 sampled elements of each large tensor and every
    element of the normalisation weights (elements are independent)."""
    announce("adamw qwen3-1.7b group, 2 steps")
    grp = inputs.adamw_group("qwen3_1.7b")
    dev = torch.device("cuda")
    steps = 2
    w0, ws, ms, vs, grads = _run_group(grp, steps, dev)
    lrs = [grp.lr(k) for k in range(steps)]
    rng = np.random.default_rng(11)
    for i, (_, n, _) in enumerate(grp.tensors):
        idx = np.arange(n) if n <= 65536 else np.unique(np.concatenate(
            [rng.integers(0, n, 65536 - 2), [0, n - 1]]))
        ti = torch.from_numpy(idx).to(dev)
        pick = lambda t: inputs.to_numpy64(t.index_select(0, ti))
        g64 = [pick(gs[i]) for gs in grads]
        w_ref, m_ref, v_ref = oracle.adamw_trajectory(pick(w0[i]), g64, lrs, OPTS)
        gmax = max(float(np.abs(g).max()) for g in g64)
        _check(pick(ws[i]), pick(ms[i]), pick(vs[i]), w_ref, m_ref, v_ref, gmax, steps, max(lrs),
               f"qwen3_1.7b {grp.tensors[i][0]}")


def test_adamw_argument_errors():
    announce("adamw argument errors")
    dev = torch.device("cuda")
    w = torch.zeros(1024, device=dev)
    m, v = torch.zeros_like(w), torch.zeros_like(w)
    opt = pm.AdamW([w], [m], [v], grad_dtype=torch.float32)
    with pytest.raises(pm.MuonHError):
        opt.step([torch.zeros(1024, device=dev)], 1e-3, 0)          # step count starts at 1
    with pytest.raises(pm.MuonHError):
        opt.step([torch.zeros(1024, device=dev)], float("nan"), 1)
    opt.close()
    base = torch.zeros(1025, device=dev)
    wv, mv, vv = base[1:], torch.zeros(1024, device=dev), torch.zeros(1024, device=dev)
    opt = pm.AdamW([wv], [mv], [vv], grad_dtype=torch.float32)
    with pytest.raises(pm.MuonHError):                                   # w misaligned by 4 bytes
        opt.step([torch.zeros(1024, device=dev)], 1e-3, 1)
    opt.close()
    torch.cuda.synchronize()
