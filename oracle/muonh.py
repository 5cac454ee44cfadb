"""fp64 NumPy oracle of the MuonH step (test infrastructure only).

What one MuonH step does to each wrapped 2-D matrix W (shape r x c), in the
order the pages give it:

1. momentum accumulation of the gradient G into M;
2. the Muon update u: Newton-Schulz orthogonalisation of the momentum;
3. the Hyperball step [arXiv §3.3, Eq. (1); notes §2.5]:
       u_hat = u / ||u||_F
       W~    = W - eta * R * u_hat
       W'    = R * W~ / ||W~||_F          with R = ||W_0||_F fixed per matrix.

The pages name the momentum and the Newton-Schulz iteration ("the Muon
update") but define neither.  The readings taken here:

* momentum is heavy-ball, M <- beta*M + G, zero-initialised; an EMA form
  (1-beta)*G differs only by the constant factor (1-beta) on M, which the
  Newton-Schulz normalisation and u_hat both cancel;
* Nesterov is off unless asked for (then the iterate is G + beta*M);
* Newton-Schulz is the quintic iteration of the published Muon method,
      X_0 = Y / (||Y||_F + eps)
      A = X X^T,  B = b A + c A A,  X <- a X + B X      (5 times)
  with (a, b, c) = (3.4445, -4.7750, 2.0315) and eps = 1e-7;
* the iteration runs in the orientation with the short side first (a tall
  matrix is transposed, iterated, transposed back).  This is exact:
  q(X X^T) X = X q(X^T X) for every polynomial q;
* weight decay is zero for the MuonH group [arXiv App. C, Tab. 8];
* an all-zero update (||u|| = 0) gives u_hat = 0, so the step is the
  projection alone; non-finite inputs propagate (no masking).

Everything is computed in float64 from inputs that are upcast exactly from
their stored dtype (bf16 and fp32 values are exact in fp64).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional, Sequence

import numpy as np

# Quintic coefficients of the published Muon method (Jordan et al., 2024).
# The pages do not print them (a reading); newton_schulz itself is pinned for
# any coefficients by the SVD closed form and the classical polar limit.
NS_COEFFS_QUINTIC = (3.4445, -4.7750, 2.0315)
# Classical Newton-Schulz polar iteration written in the same quintic form:
# p(x) = (15 x - 10 x^3 + 3 x^5) / 8, with p(1) = 1 and p'(1) = 0, whose
# fixed point on singular values in (0, sqrt(3)) is 1: the polar factor.
NS_COEFFS_CLASSICAL = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def fro(a) -> float:
    """Frobenius norm ||a||_F, summed in fp64."""
    a = _f64(a)
    return float(np.sqrt(np.sum(a * a)))


def radius(w0) -> float:
    """Hyperball radius R = ||W_0||_F, fixed per matrix [arXiv §3.3]."""
    return fro(w0)


def momentum_update(m, g, beta: float) -> np.ndarray:
    """Heavy-ball momentum M <- beta*M + G (reading of the Muon update)."""
    return beta * _f64(m) + _f64(g)


def ns_input(m_new, g, beta: float, nesterov: bool) -> np.ndarray:
    """The matrix handed to Newton-Schulz: M, or G + beta*M with Nesterov."""
    if nesterov:
        return _f64(g) + beta * _f64(m_new)
    return _f64(m_new)


def newton_schulz(y, steps: int = 5, coeffs=NS_COEFFS_QUINTIC,
                  eps: float = 1e-7, orient: bool = True) -> np.ndarray:
    """Quintic Newton-Schulz orthogonalisation of y (the Muon update u).

    X_0 = y / (||y||_F + eps); then `steps` times
    A = X X^T, B = b*A + c*(A A), X = a*X + B X.
    With `orient`, a tall y (rows > cols) is transposed first and the result
    transposed back, so the Gram matrix A is min(r,c) square.
    """
    a, b, c = (float(v) for v in coeffs)
    y = _f64(y)
    if y.ndim != 2:
        raise ValueError("newton_schulz expects a 2-D matrix")
    tall = orient and y.shape[0] > y.shape[1]
    x = y.T if tall else y
    x = x / (fro(x) + eps)
    for _ in range(steps):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x.T.copy() if tall else x


@dataclasses.dataclass
class HyperballDiag:
    """Per-matrix diagnostics of one Hyperball step (cf. [arXiv App. D, Fig. 15])."""
    u_norm: float          # ||u||_F of the raw Muon update
    w_norm: float          # ||W_t||_F before the step
    inner: float           # <W_t, u_hat>
    c: float               # <W_t, u_hat> / R
    wt_norm: float         # ||W~||_F before projection
    elr: float             # ||W~ - W_t||_F / ||W_t||_F   (= eta when ||W_t|| = R)
    angle: float           # angle between W_t and W_{t+1}, from the closed form
    nonfinite: bool


def hyperball_update(w, u, eta: float, R: float):
    """Hyperball step of [arXiv §3.3, Eq. (1)] on one matrix.

    Returns (W_{t+1}, HyperballDiag).  ||W~|| is computed directly from W~.
    """
    w = _f64(w)
    u = _f64(u)
    un = fro(u)
    u_hat = u / un if un != 0.0 else np.zeros_like(u)   # NaN propagates
    w_tilde = w - eta * R * u_hat
    wt_norm = fro(w_tilde)
    w_new = R * w_tilde / wt_norm
    w_norm = fro(w)
    inner = float(np.sum(w * u_hat))
    c = inner / R
    diag = HyperballDiag(
        u_norm=un, w_norm=w_norm, inner=inner, c=c, wt_norm=wt_norm,
        elr=fro(w_tilde - w) / w_norm,
        angle=closed_form_angle(eta, c),
        nonfinite=not (np.all(np.isfinite(u)) and np.all(np.isfinite(w))),
    )
    return w_new, diag


def muon_wd_update(w, u, eta: float, lam: float) -> np.ndarray:
    """Ordinary Muon with decoupled weight decay [arXiv §3.3.1, Eq. (3)]:
    W <- (1 - lam*eta) W - eta u."""
    return (1.0 - lam * eta) * _f64(w) - eta * _f64(u)


def elr_aligned_update(w, u, rho: float):
    """Effective-LR-aligned Muon [arXiv §3.3.1, Eq. (5)]: the scalar LR is
    eta_t = rho * ||W_t|| / ||u_t|| and there is no projection, so the
    effective LR of Eq. (4), eta_t ||u_t|| / ||W_t||, equals rho.
    Returns (W_{t+1}, eta_t); an all-zero u leaves W unchanged (eta_t = 0)."""
    w = _f64(w)
    u = _f64(u)
    un = fro(u)
    eta_t = rho * fro(w) / un if un != 0.0 else 0.0
    return w - eta_t * u, eta_t


def chord_angle(w0, w1, R: float) -> float:
    """Angle between two points of the radius-R sphere from their chord:
    theta = 2 asin(||W1 - W0|| / (2R))."""
    return 2.0 * math.asin(min(1.0, fro(_f64(w1) - _f64(w0)) / (2.0 * R)))


def closed_form_angle(eta: float, c: float) -> float:
    """Angle turned by one Hyperball step.  With ||W|| = R and c = <W,u_hat>/R,
    W~ = W - eta R u_hat has ||W~||^2 = R^2 (1 - 2 eta c + eta^2), and the
    angle between W and W~ (hence W_{t+1}) satisfies
    tan(theta) = eta sqrt(1 - c^2) / (1 - eta c)."""
    c = max(-1.0, min(1.0, c))
    return math.atan2(eta * math.sqrt(max(0.0, 1.0 - c * c)), 1.0 - eta * c)


@dataclasses.dataclass
class OracleOptions:
    beta: float = 0.95
    ns_steps: int = 5
    ns_coeffs: tuple = NS_COEFFS_QUINTIC
    ns_eps: float = 1e-7
    nesterov: bool = False
    orient: bool = True


@dataclasses.dataclass
class OracleMatrixState:
    w: np.ndarray            # fp64 weights
    m: np.ndarray            # fp64 momentum
    R: float                 # fixed radius

    @staticmethod
    def from_arrays(w0, m0=None, R: Optional[float] = None) -> "OracleMatrixState":
        w = _f64(w0).copy()
        m = np.zeros_like(w) if m0 is None else _f64(m0).copy()
        return OracleMatrixState(w=w, m=m, R=radius(w) if R is None else float(R))


def muonh_step(states: Sequence[OracleMatrixState], grads: Sequence, eta: float,
               opts: OracleOptions = OracleOptions(),
               elr_scale: Optional[Sequence[float]] = None):
    """One MuonH step over a list of matrices, in place on `states`.

    Matrices are independent: each one runs momentum, Newton-Schulz and the
    Hyperball step of [arXiv §3.3, Eq. (1)] with effective LR eta (times the
    optional per-matrix factor).  Returns (list of u, list of HyperballDiag,
    list of ||M||_F after the momentum update).
    """
    if len(states) != len(grads):
        raise ValueError("states and grads differ in length")
    us, diags, mnorms = [], [], []
    for i, (st, g) in enumerate(zip(states, grads)):
        g = _f64(g)
        if g.shape != st.w.shape:
            raise ValueError(f"matrix {i}: grad shape {g.shape} != {st.w.shape}")
        st.m = momentum_update(st.m, g, opts.beta)
        y = ns_input(st.m, g, opts.beta, opts.nesterov)
        u = newton_schulz(y, opts.ns_steps, opts.ns_coeffs, opts.ns_eps, opts.orient)
        e = eta * (1.0 if elr_scale is None else float(elr_scale[i]))
        st.w, d = hyperball_update(st.w, u, e, st.R)
        us.append(u)
        diags.append(d)
        mnorms.append(fro(st.m))
    return us, diags, mnorms


def muonh_trajectory(states: Sequence[OracleMatrixState], grad_steps: Iterable[Sequence],
                     etas: Sequence[float], opts: OracleOptions = OracleOptions()):
    """Run several MuonH steps; returns the per-step (us, diags, mnorms)."""
    out = []
    for grads, eta in zip(grad_steps, etas):
        out.append(muonh_step(states, grads, eta, opts))
    return out


def ns_dense_flops(rows: int, cols: int, steps: int = 5) -> float:
    """Dense FLOP of the Newton-Schulz products of one matrix: per iteration
    2 m^2 n (X X^T) + 2 m^3 (A A) + 2 m^2 n (B X), m = min, n = max."""
    m, n = min(rows, cols), max(rows, cols)
    return float(steps) * (4.0 * m * m * n + 2.0 * m * m * m)
