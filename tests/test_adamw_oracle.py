"""Pins of the AdamW oracle (CPU): closed forms the update rule implies and
PyTorch's own AdamW (an independent implementation) in fp64."""

import numpy as np
import pytest
import torch

import oracle

OPTS = oracle.AdamWOptions(beta1=0.9, beta2=0.95, eps=1e-12, weight_decay=0.1)


def _rng(seed):
    return np.random.default_rng(seed)


def test_first_step_is_decay_plus_sign_step():
    """t = 1: bias correction makes m_hat = g, v_hat = g^2, so the step is
    lr * g / (|g| + eps) after the decoupled decay.  Gradients near eps
    separate eps outside the square root from eps inside it."""
    r = _rng(0)
    w = r.standard_normal(64)
    g = r.standard_normal(64)
    g[:8] = np.array([1e-13, -3e-13, 1e-12, -2e-12, 5e-12, 1e-11, -1e-10, 0.0])
    lr = 0.3
    w1, m1, v1 = oracle.adamw_step(w, g, np.zeros(64), np.zeros(64), 1, lr, OPTS)
    expect = w * (1 - lr * OPTS.weight_decay) - lr * g / (np.abs(g) + OPTS.eps)
    np.testing.assert_allclose(w1, expect, rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=4e-15)
    np.testing.assert_allclose(v1, 0.05 * g * g, rtol=4e-15)


def test_constant_gradient_closed_form():
    r = _rng(1)
    w0 = r.standard_normal(33)
    g = r.standard_normal(33)
    lr = 0.05
    w, m, v = oracle.adamw_trajectory(w0, [g] * 7, [lr] * 7, OPTS)
    np.testing.assert_allclose(w, oracle.constant_gradient_closed_form(w0, g, lr, 7, OPTS),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(m, (1 - 0.9 ** 7) * g, rtol=1e-13)
    np.testing.assert_allclose(v, (1 - 0.95 ** 7) * g * g, rtol=1e-13)


def test_zero_gradient_is_pure_decay():
    w0 = np.linspace(-2, 2, 17)
    w, m, v = oracle.adamw_trajectory(w0, [np.zeros(17)] * 5, [0.1] * 5, OPTS)
    np.testing.assert_allclose(w, (1 - 0.1 * 0.1) ** 5 * w0, rtol=1e-15)
    assert not m.any() and not v.any()


@pytest.mark.parametrize("wd,eps", [(0.1, 1e-12), (0.0, 1e-8), (0.3, 1e-6)])
def test_matches_torch_adamw_fp64(wd, eps):
    """Ten steps with changing gradients and a changing LR against
    torch.optim.AdamW on the CPU in float64."""
    opts = oracle.AdamWOptions(beta1=0.9, beta2=0.95, eps=eps, weight_decay=wd)
    r = _rng(2)
    w0 = r.standard_normal((7, 13))
    grads = [r.standard_normal((7, 13)) * (0.1 + k) for k in range(10)]
    grads[3][0, :] = 0.0
    lrs = [1e-2 * (1 - k / 10) + 1e-4 for k in range(10)]
    w, m, v = oracle.adamw_trajectory(w0, grads, lrs, opts)
    p = torch.nn.Parameter(torch.tensor(w0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lrs[0], betas=(0.9, 0.95), eps=eps, weight_decay=wd)
    for g, lr in zip(grads, lrs):
        opt.param_groups[0]["lr"] = lr
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    np.testing.assert_allclose(w, p.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-16)


def test_step_count_starts_at_one():
    with pytest.raises(ValueError):
        oracle.adamw_step(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), 0, 0.1)


def test_bytes_per_element():
    assert oracle.adamw_bytes_per_element(2) == 26
    assert oracle.adamw_bytes_per_element(4) == 28
