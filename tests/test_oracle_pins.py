"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: a closed
form evaluated through a different route (SVD + scalar iteration), a textbook
special case (the classical Newton-Schulz polar iteration), an invariant of
the Hyperball step [arXiv §3.3, Eq. (1)], or a value printed on the pages.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import muonh as om

HERE = os.path.dirname(os.path.abspath(__file__))
A, B, C = oracle.NS_COEFFS_QUINTIC


def _scalar_iter(x, steps=5, coeffs=oracle.NS_COEFFS_QUINTIC):
    a, b, c = coeffs
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def _svd_closed_form(y, steps=5, coeffs=oracle.NS_COEFFS_QUINTIC, eps=1e-7):
    """An odd matrix polynomial acts on singular values only:
    NS(Y) = U diag(p^(steps)(sigma / (||Y||_F + eps))) V^T."""
    u, s, vt = np.linalg.svd(y, full_matrices=False)
    scale = np.linalg.norm(y) + eps
    return (u * _scalar_iter(s / scale, steps, coeffs)) @ vt


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _with_singular_values(rng, r, c, s):
    u, _ = np.linalg.qr(rng.standard_normal((r, len(s))))
    v, _ = np.linalg.qr(rng.standard_normal((c, len(s))))
    return (u * np.asarray(s)) @ v.T


@pytest.mark.parametrize("shape", [(8, 5), (5, 8), (64, 16), (16, 64), (33, 33), (3, 40)])
def test_ns_matches_svd_closed_form(shape):
    rng = np.random.default_rng(1)
    y = rng.standard_normal(shape)
    got = oracle.newton_schulz(y)
    assert _rel(got, _svd_closed_form(y)) <= 1e-10


def test_ns_rank_deficient_and_repeated_sigma():
    rng = np.random.default_rng(2)
    y = _with_singular_values(rng, 12, 9, [3.0, 1.0, 0.2])           # rank 3
    assert _rel(oracle.newton_schulz(y), _svd_closed_form(y)) <= 1e-10
    y = _with_singular_values(rng, 10, 20, [2.0, 2.0, 2.0, 0.5, 0.5])  # repeated
    assert _rel(oracle.newton_schulz(y), _svd_closed_form(y)) <= 1e-10


def test_ns_singular_vectors_and_band():
    """Output shares the input's singular vectors, and every singular value
    whose normalised input is >= 2e-3 lands in the band the five-fold scalar
    quintic gives: [0.68183, 1.20237] (>= 5e-3: upper edge 1.15437)."""
    rng = np.random.default_rng(3)
    y = rng.standard_normal((48, 96))
    o = oracle.newton_schulz(y)
    u, s, vt = np.linalg.svd(y, full_matrices=False)
    core = u.T @ o @ vt.T
    off = core - np.diag(np.diag(core))
    assert np.linalg.norm(off) <= 1e-10 * np.linalg.norm(o)
    xs = np.geomspace(2e-3, 1.0, 200001)
    ys = _scalar_iter(xs)
    lo, hi = ys.min(), ys.max()
    assert abs(lo - 0.68183) < 1e-5 and abs(hi - 1.20237) < 1e-5
    sig_in = s / (np.linalg.norm(y) + 1e-7)
    sig_out = np.diag(core)
    mask = sig_in >= 2e-3
    assert mask.all()
    assert np.all(sig_out[mask] >= lo - 1e-12) and np.all(sig_out[mask] <= hi + 1e-12)


def test_ns_classical_coefficients_give_polar_factor():
    """Classical Newton-Schulz (15/8, -10/8, 3/8) converges to U V^T, the
    polar factor from the SVD, on a well-conditioned matrix."""
    rng = np.random.default_rng(4)
    y = _with_singular_values(rng, 7, 11, [5.0, 3.0, 2.0, 1.0, 0.6, 0.4, 0.2])
    o = oracle.newton_schulz(y, steps=40, coeffs=oracle.NS_COEFFS_CLASSICAL)
    u, _, vt = np.linalg.svd(y, full_matrices=False)
    assert _rel(o, u @ vt) <= 1e-12


def test_ns_orientation_is_exact():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((40, 9))
    assert _rel(oracle.newton_schulz(y, orient=True), oracle.newton_schulz(y, orient=False)) <= 1e-12


def test_rank_one_update_direction():
    """Y = s x y^T has one singular value, so u_hat = x y^T exactly and
    W~ = W - eta R x y^T."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal(13); x /= np.linalg.norm(x)
    z = rng.standard_normal(7); z /= np.linalg.norm(z)
    g = 4.0 * np.outer(x, z)
    w0 = rng.standard_normal((13, 7))
    st = oracle.OracleMatrixState.from_arrays(w0)
    us, diags, _ = oracle.muonh_step([st], [g], eta=0.05)
    u_hat = us[0] / np.linalg.norm(us[0])
    assert _rel(u_hat, np.outer(x, z)) <= 1e-12
    wt = w0 - 0.05 * st.R * np.outer(x, z)
    assert _rel(st.w, st.R * wt / np.linalg.norm(wt)) <= 1e-12


def test_momentum_closed_form():
    rng = np.random.default_rng(7)
    beta = 0.95
    gs = [rng.standard_normal((6, 4)) for _ in range(5)]
    st = oracle.OracleMatrixState.from_arrays(rng.standard_normal((6, 4)))
    for g in gs:
        oracle.muonh_step([st], [g], eta=0.01, opts=oracle.OracleOptions(beta=beta))
    t = len(gs) - 1
    expect = sum(beta ** (t - k) * gs[k] for k in range(len(gs)))
    assert _rel(st.m, expect) <= 1e-14


def test_nesterov_iterate():
    """With Nesterov the Newton-Schulz input is G + beta*M_new; on the first
    step (M_0 = 0) that is (1 + beta) G, the same direction as G."""
    rng = np.random.default_rng(8)
    g = rng.standard_normal((9, 5))
    st1 = oracle.OracleMatrixState.from_arrays(np.ones((9, 5)))
    st2 = oracle.OracleMatrixState.from_arrays(np.ones((9, 5)))
    u1, _, _ = oracle.muonh_step([st1], [g], 0.01, oracle.OracleOptions(nesterov=True, ns_eps=0.0))
    u2, _, _ = oracle.muonh_step([st2], [g], 0.01, oracle.OracleOptions(nesterov=False, ns_eps=0.0))
    assert _rel(u1[0], u2[0]) <= 1e-13
    g2 = rng.standard_normal((9, 5))
    u1, _, _ = oracle.muonh_step([st1], [g2], 0.01, oracle.OracleOptions(nesterov=True, ns_eps=0.0))
    y = g2 + 0.95 * (0.95 * g + g2)
    assert _rel(u1[0], _svd_closed_form(y, eps=0.0)) <= 1e-10


def test_hyperball_invariant_elr_and_angle():
    """||W_{t+1}|| = R after every step; the pre-projection displacement is
    eta R, so the effective LR is eta [arXiv §3.3.1]; the angle turned equals
    the chord angle 2 asin(||dW|| / 2R) and cos(theta) = <W_t, W_{t+1}> / R^2."""
    rng = np.random.default_rng(9)
    w0 = rng.standard_normal((24, 40))
    w0 *= math.sqrt(24) / np.linalg.norm(w0)
    st = oracle.OracleMatrixState.from_arrays(w0)
    for k in range(8):
        eta = 0.012 * (1 - k / 20)
        w_prev = st.w.copy()
        g = rng.standard_normal((24, 40)) + 0.3 * w_prev   # correlated with W: c != 0
        _, diags, _ = oracle.muonh_step([st], [g], eta)
        d = diags[0]
        assert abs(np.linalg.norm(st.w) / st.R - 1.0) <= 1e-14
        assert abs(d.elr - eta) <= 1e-12 * eta
        theta_chord = oracle.chord_angle(w_prev, st.w, st.R)
        cos_t = float(np.sum(w_prev * st.w)) / st.R ** 2
        assert abs(theta_chord - d.angle) <= 1e-9 * eta
        assert abs(math.acos(min(1.0, cos_t)) - d.angle) <= 1e-6 * eta
        assert abs(d.angle - eta) <= eta * (abs(d.c) + eta)


def test_scale_invariance():
    """Scaling every gradient of a matrix by a positive constant leaves the
    trajectory unchanged (exactly with eps = 0; the 1/sqrt(fan_in) scaling of
    the 170M workload is such a constant)."""
    rng = np.random.default_rng(10)
    w0 = rng.standard_normal((16, 48))
    gs = [rng.standard_normal((16, 48)) for _ in range(4)]
    for eps, tol in ((0.0, 1e-12), (1e-7, 1e-6)):
        opts = oracle.OracleOptions(ns_eps=eps)
        s1 = oracle.OracleMatrixState.from_arrays(w0)
        s2 = oracle.OracleMatrixState.from_arrays(w0)
        for g in gs:
            oracle.muonh_step([s1], [g], 0.02, opts)
            oracle.muonh_step([s2], [g / math.sqrt(48)], 0.02, opts)
        assert _rel(s2.w, s1.w) <= tol


def test_zero_gradient_is_projection_only():
    w0 = np.arange(12.0).reshape(3, 4) + 1.0
    st = oracle.OracleMatrixState.from_arrays(w0, R=5.0)
    us, diags, _ = oracle.muonh_step([st], [np.zeros((3, 4))], 0.1)
    assert np.all(us[0] == 0.0)
    assert _rel(st.w, 5.0 * w0 / np.linalg.norm(w0)) <= 1e-15


def test_nonfinite_propagates():
    g = np.ones((4, 4)); g[1, 2] = np.nan
    st = oracle.OracleMatrixState.from_arrays(np.eye(4))
    _, diags, _ = oracle.muonh_step([st], [g], 0.1)
    assert diags[0].nonfinite and np.isnan(st.w).all()


def test_muon_wd_and_elr_aligned():
    """Eq. (3): W_{t+1} + eta u = (1 - lambda eta) W_t.  Eq. (5): the aligned
    LR makes the measured relative displacement ||dW|| / ||W_t|| equal rho."""
    rng = np.random.default_rng(11)
    w = rng.standard_normal((10, 30))
    u = oracle.newton_schulz(rng.standard_normal((10, 30)))
    w1 = oracle.muon_wd_update(w, u, 0.02, 0.1)
    assert _rel(w1 + 0.02 * u, (1 - 0.002) * w) <= 1e-15
    w2, eta_t = oracle.elr_aligned_update(w, u, 0.013)
    assert abs(np.linalg.norm(w2 - w) / np.linalg.norm(w) - 0.013) <= 1e-14
    assert eta_t > 0


def test_dense_flops_formula():
    # 1.7B down projection 2048 x 6144: 5 x (4 m^2 n + 2 m^3)
    assert om.ns_dense_flops(2048, 6144) == 5 * (4 * 2048 ** 2 * 6144 + 2 * 2048 ** 3)
    assert om.ns_dense_flops(6144, 2048) == om.ns_dense_flops(2048, 6144)


# ---------------------------------------------------------------------------
# schedule values printed on the pages

with open(os.path.join(HERE, "golden", "schedule_pins.json")) as f:
    PINS = json.load(f)


def _printed_match(value, printed):
    """Equal at the printed precision (3 significant figures)."""
    return float(f"{value:.3g}") == printed


def test_phase1_power_schedule_end_and_peak():
    tps = PINS["tokens_per_step"]
    p = PINS["phase1_end"]
    k = p["tokens"] / tps
    v = oracle.lr_phase1_power(k)
    assert _printed_match(v, p["printed_base_lr"])
    assert _printed_match(oracle.hyperball_lr(v), p["printed_hyperball_lr"])
    w = PINS["phase1_warmup_peak"]
    assert oracle.lr_phase1_power(w["step"]) == pytest.approx(w["printed_base_lr"], rel=1e-15)
    assert oracle.lr_phase1_power(w["step"] + 1e-9) == pytest.approx(w["printed_base_lr"], rel=1e-9)
    assert oracle.lr_phase1_power(500) == pytest.approx(2.5e-3, rel=1e-15)


def test_phase2_linear_and_cma_hold():
    tps = PINS["tokens_per_step"]
    eta0 = oracle.lr_phase1_power(PINS["phase1_end"]["tokens"] / tps)
    h = PINS["cma_hold"]
    S = h["run_last_step"] - h["phase2_start_step"]

    def sched(k):
        return oracle.lr_linear(eta0, h["eta_min"], k - h["phase2_start_step"], S)

    v = oracle.lr_constant_hold(220000, h["hold_step"], sched)
    assert _printed_match(v, h["printed_base_lr"])
    assert _printed_match(oracle.hyperball_lr(v), h["printed_hyperball_lr"])
    assert sched(h["phase2_start_step"]) == eta0
    assert sched(h["run_last_step"]) == pytest.approx(h["eta_min"], rel=1e-12)
    w = PINS["cma_window"]
    assert round((h["run_last_step"] - h["hold_step"]) * tps / 1e9) == w["printed_last_tokens_B"]
    assert round((h["run_last_step"] - 222100) * tps / 1e9, 2) == w["printed_window_tokens_B"]
    assert h["run_last_step"] - 222100 == w["printed_window_steps"]
    assert round(w["printed_spacing_steps"] * tps / 1e9, 2) == w["printed_spacing_tokens_B"]


def test_wsd_and_cosine_shapes():
    assert oracle.lr_wsd(0, 0.024, 10, 1.0) == pytest.approx(0.024)
    assert oracle.lr_wsd(5, 0.024, 10, 1.0) == pytest.approx(0.012)
    assert oracle.lr_wsd(10, 0.024, 10, 1.0) == 0.0
    assert oracle.lr_wsd(3, 0.01, 10, 0.5) == 0.01
    assert oracle.lr_wsd(7.5, 0.01, 10, 0.5) == pytest.approx(0.005)
    assert oracle.lr_cosine(0, 100, 1e-5, 1e-7) == pytest.approx(1e-5)
    assert oracle.lr_cosine(50, 100, 1e-5, 1e-7) == pytest.approx(0.5 * (1e-5 + 1e-7))
    assert oracle.lr_cosine(100, 100, 1e-5, 1e-7) == pytest.approx(1e-7)


# ---------------------------------------------------------------------------
# Property tests over random small shapes, spectra and step sizes.

from hypothesis import given, settings, strategies as st  # noqa: E402

_SETTINGS = settings(max_examples=40, deadline=None, derandomize=True)


@_SETTINGS
@given(r=st.integers(1, 24), c=st.integers(1, 24), seed=st.integers(0, 2 ** 31 - 1),
       decades=st.floats(0.0, 3.0), steps=st.integers(1, 6))
def test_ns_closed_form_random_shapes_and_spectra(r, c, seed, decades, steps):
    """Any shape (1 x n, n x 1, square, tall, wide), singular values spread
    over up to three decades, any iteration count: the oracle's Newton-Schulz
    equals the SVD closed form U p^steps(sigma/(||Y||+eps)) V^T."""
    rng = np.random.default_rng(seed)
    k = min(r, c)
    s = 10.0 ** (-decades * rng.random(k))
    y = _with_singular_values(rng, r, c, s) if k > 1 else rng.standard_normal((r, c))
    got = oracle.newton_schulz(y, steps)
    assert _rel(got, _svd_closed_form(y, steps)) <= 1e-10


@_SETTINGS
@given(r=st.integers(1, 20), c=st.integers(1, 20), seed=st.integers(0, 2 ** 31 - 1),
       eta=st.floats(1e-4, 0.5))
def test_hyperball_invariants_random(r, c, seed, eta):
    """For any W, direction and step size: ||W_{t+1}|| = R, the pre-projection
    displacement is eta R (ELR = eta), and the new W is the projection of
    W - eta R u^ onto the sphere (positive multiple, unit cosine)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((r, c))
    R = float(np.linalg.norm(w)) * (0.5 + rng.random())
    w = w * (R / np.linalg.norm(w))
    u = rng.standard_normal((r, c))
    w1, _ = om.hyperball_update(w, u, eta, R)
    assert abs(np.linalg.norm(w1) / R - 1.0) <= 1e-12
    wt = w - eta * R * u / np.linalg.norm(u)
    assert abs(np.linalg.norm(wt - w) / R - eta) <= 1e-12
    cos = float(np.sum(w1 * wt)) / (np.linalg.norm(w1) * np.linalg.norm(wt))
    assert abs(cos - 1.0) <= 1e-12


# ---------------------------------------------------------------------------
# Direct pins of the remaining helpers.

def test_fro_and_radius_on_integer_triples():
    """Frobenius norms of integer matrices with known integer norms
    (3-4-12-84 chains: 3^2+4^2 = 5^2, 5^2+12^2 = 13^2, 13^2+84^2 = 85^2)."""
    assert om.fro(np.array([[3.0, 4.0]])) == 5.0
    assert om.fro(np.array([[3.0, 4.0], [12.0, 0.0]])) == 13.0
    assert om.radius(np.array([[3.0, 4.0, 12.0], [84.0, 0.0, 0.0]])) == 85.0
    assert om.fro(np.zeros((4, 5))) == 0.0


def test_momentum_and_nesterov_input_on_scalars():
    """Heavy-ball momentum with beta = 1/2 on a 1 x 1 matrix: gradients 4, 2, 8
    give M = 4, 4, 10; the Nesterov input after the last is G + beta M = 13,
    the plain input M = 10."""
    m = np.zeros((1, 1))
    for g, want in ((4.0, 4.0), (2.0, 4.0), (8.0, 10.0)):
        m = om.momentum_update(m, np.array([[g]]), 0.5)
        assert m[0, 0] == want
    g = np.array([[8.0]])
    assert om.ns_input(m, g, 0.5, True)[0, 0] == 13.0
    assert om.ns_input(m, g, 0.5, False)[0, 0] == 10.0


def test_closed_form_angle_matches_the_turned_angle():
    """For actual Hyperball steps the closed-form angle equals the angle
    between W_t and W_{t+1} measured as acos(<W_t, W_{t+1}> / R^2), and the
    chord angle; at c = 0 it is atan(eta), at c = 1 (moving straight to the
    centre, eta < 1) it is zero."""
    rng = np.random.default_rng(11)
    for eta in (1e-3, 0.02, 0.3):
        w = rng.standard_normal((20, 30))
        R = float(np.linalg.norm(w))
        u = rng.standard_normal((20, 30))
        w1, d = om.hyperball_update(w, u, eta, R)
        c = float(np.sum(w * u)) / (np.linalg.norm(u) * R)
        th = om.closed_form_angle(eta, c)
        measured = math.acos(max(-1.0, min(1.0, float(np.sum(w * w1)) / R ** 2)))
        assert abs(th - measured) <= 1e-9
        assert abs(om.chord_angle(w, w1, R) - measured) <= 1e-9
    assert abs(om.closed_form_angle(0.1, 0.0) - math.atan(0.1)) <= 1e-15
    assert om.closed_form_angle(0.5, 1.0) == 0.0


def test_trajectory_zero_gradients_keep_the_projection():
    """Zero gradients for several steps: M stays 0, u = 0, and W stays the
    projection R W_0 / ||W_0|| of its start (here already on the sphere, so
    W_t = W_0 to rounding) with ||W_t|| = R after every step."""
    rng = np.random.default_rng(12)
    w0 = rng.standard_normal((6, 9))
    st = oracle.OracleMatrixState.from_arrays(w0)
    grads = [[np.zeros((6, 9))] for _ in range(4)]
    out = om.muonh_trajectory([st], grads, [0.05, 0.04, 0.03, 0.02])
    assert len(out) == 4
    for us, _, _ in out:
        assert not np.any(us[0])
    assert not np.any(st.m)
    assert abs(np.linalg.norm(st.w) / st.R - 1.0) <= 1e-15
    assert np.allclose(st.w, w0, rtol=0, atol=1e-14)


def test_adamw_first_step_direction_is_the_sign_up_to_eps():
    """g/(|g| + eps): exactly +-1/(1 + eps/|g|), i.e. the sign of g for |g| >> eps,
    0 for g = 0, and half the sign at |g| = eps."""
    from oracle import adamw as oa
    g = np.array([3.0, -2.0, 0.0, 1e-8, -1e-8])
    d = oa.first_step_direction(g, 1e-8)
    assert d[0] == 3.0 / (3.0 + 1e-8) and d[1] == -2.0 / (2.0 + 1e-8) and d[2] == 0.0
    assert d[3] == 0.5 and d[4] == -0.5


def _exact_ns(y_rows, steps, coeffs):
    """The quintic iteration in exact rational arithmetic (fractions.Fraction),
    written out with explicit sums: X_0 = Y / ||Y||_F for a Y whose Frobenius
    norm is rational, then A = X X^T, B = b A + c A A, X = a X + B X."""
    from fractions import Fraction
    a, b, c = (Fraction(str(v)) for v in coeffs)
    y = [[Fraction(v) for v in row] for row in y_rows]
    n2 = sum(v * v for row in y for v in row)
    # the norm is rational: find it as an exact square root
    num, den = n2.numerator, n2.denominator
    rn, rd = math.isqrt(num), math.isqrt(den)
    assert rn * rn == num and rd * rd == den, "test matrix must have a rational Frobenius norm"
    norm = Fraction(rn, rd)
    x = [[v / norm for v in row] for row in y]
    m, n = len(x), len(x[0])
    for _ in range(steps):
        A = [[sum(x[i][k] * x[j][k] for k in range(n)) for j in range(m)] for i in range(m)]
        AA = [[sum(A[i][k] * A[k][j] for k in range(m)) for j in range(m)] for i in range(m)]
        B = [[b * A[i][j] + c * AA[i][j] for j in range(m)] for i in range(m)]
        x = [[a * x[i][j] + sum(B[i][k] * x[k][j] for k in range(m)) for j in range(n)] for i in range(m)]
    return x


@pytest.mark.parametrize("rows", [
    [[3, 0, 4], [0, 0, 0]],                                  # 2 x 3, rank 1, ||Y|| = 5
    [[1, -1, -2], [3, -2, 0], [1, -2, -1]],                  # 3 x 3, full rank, ||Y|| = 5
    [[-1, -1, 1, 0, 3], [1, 3, 1, -1, -1]],                  # 2 x 5 (wide), ||Y|| = 5
    [[2, -2, 1], [3, 1, 1], [0, 3, -2], [-1, 1, 1]],         # 4 x 3 (tall), ||Y|| = 6
    [[3, -3, -1, -3], [3, 1, -1, 2], [-1, 0, -1, 2]],        # 3 x 4, ||Y|| = 7
])
def test_ns_against_exact_rational_iteration(rows):
    """The oracle's Newton-Schulz (fp64 NumPy) against the same iteration
    carried out exactly in rational arithmetic, on small integer matrices
    whose Frobenius norm is an integer (eps = 0, so X_0 = Y/||Y|| exactly).
    No floating point on the reference side: a dropped term, a wrong sign or
    a transposed operand in the oracle shows up at O(1), while its fp64
    rounding stays below 1e-13 relative.  The tall case is also run through
    the oracle's orientation flip (iterating on the transpose)."""
    y = np.array(rows, dtype=np.float64)
    for steps in (1, 2, 5):
        ref = _exact_ns(rows, steps, oracle.NS_COEFFS_QUINTIC)
        ref = np.array([[float(v) for v in row] for row in ref])
        got = oracle.newton_schulz(y, steps=steps, eps=0.0, orient=False)
        assert np.linalg.norm(got - ref) <= 1e-13 * max(1.0, np.linalg.norm(ref)), (steps, got, ref)
        got_o = oracle.newton_schulz(y, steps=steps, eps=0.0, orient=True)
        assert np.linalg.norm(got_o - ref) <= 1e-12 * max(1.0, np.linalg.norm(ref)), steps
    # the classical coefficients through the same exact route
    ref = np.array([[float(v) for v in row] for row in _exact_ns(rows, 3, oracle.NS_COEFFS_CLASSICAL)])
    got = oracle.newton_schulz(y, steps=3, coeffs=oracle.NS_COEFFS_CLASSICAL, eps=0.0, orient=False)
    assert np.linalg.norm(got - ref) <= 1e-13 * max(1.0, np.linalg.norm(ref))
