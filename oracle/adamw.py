"""fp64 NumPy oracle of the AdamW step of the non-MuonH parameter group
(test infrastructure only).

The pages train every parameter that MuonH does not wrap -- embeddings,
normalisation layers, the LM head and the rest -- with AdamW at weight decay
0.1 on the base LR schedule [arXiv §3.3; App. C, Tab. 8 and the production
run setup], and give Adam's betas (0.9, 0.95) and epsilon 1e-12 for the
post-training runs [arXiv App. E].  They do not print the update rule.  The
reading taken is the standard AdamW with decoupled weight decay and bias
correction, in this order, for step t = 1, 2, ... and LR eta:

    W <- W (1 - eta * lambda)
    m <- beta1 m + (1 - beta1) g
    v <- beta2 v + (1 - beta2) g^2
    W <- W - eta * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)

m and v start at zero.  Every tensor is updated element by element, so the
step of a list of tensors is the step of each one.
"""

from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class AdamWOptions:
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-12
    weight_decay: float = 0.1


def adamw_step(w: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, t: int,
               lr: float, opts: AdamWOptions = AdamWOptions()):
    """One AdamW step at step count t (>= 1); returns new (w, m, v) in fp64."""
    if t < 1:
        raise ValueError("the step count starts at 1")
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    w = w * (1.0 - lr * opts.weight_decay)
    m = opts.beta1 * m + (1.0 - opts.beta1) * g
    v = opts.beta2 * v + (1.0 - opts.beta2) * g * g
    m_hat = m / (1.0 - opts.beta1 ** t)
    v_hat = v / (1.0 - opts.beta2 ** t)
    w = w - lr * m_hat / (np.sqrt(v_hat) + opts.eps)
    return w, m, v


def adamw_trajectory(w0, grads, lrs, opts: AdamWOptions = AdamWOptions()):
    """Steps 1..K from zero moments; returns (w, m, v) after the last step."""
    w = np.asarray(w0, dtype=np.float64)
    m = np.zeros_like(w)
    v = np.zeros_like(w)
    for k, (g, lr) in enumerate(zip(grads, lrs)):
        w, m, v = adamw_step(w, g, m, v, k + 1, lr, opts)
    return w, m, v


def adamw_bytes_per_element(g_bytes: int) -> int:
    """HBM bytes one element moves: g read, W / m / v (fp32) read and written."""
    return g_bytes + 3 * 2 * 4


def first_step_direction(g: np.ndarray, eps: float) -> np.ndarray:
    """At t = 1 the bias corrections give m_hat = g and v_hat = g^2, so the
    update direction is g / (|g| + eps), i.e. sign(g) up to eps."""
    g = np.asarray(g, dtype=np.float64)
    return g / (np.abs(g) + eps)


def constant_gradient_closed_form(w0, g, lr: float, steps: int, opts: AdamWOptions):
    """A constant gradient keeps m_hat = g and v_hat = g^2 at every step, so
    W_t = a^t W_0 - lr s (1 + a + ... + a^(t-1)) with a = 1 - lr lambda and
    s = g / (|g| + eps)."""
    a = 1.0 - lr * opts.weight_decay
    s = first_step_direction(g, opts.eps)
    geo = float(steps) if a == 1.0 else (1.0 - a ** steps) / (1.0 - a)
    return (a ** steps) * np.asarray(w0, dtype=np.float64) - lr * s * geo

