"""Learning-rate schedules of the pages, as plain formulas (test infrastructure).

The Hyperball weight LR is a fixed multiple of the base schedule,
eta^H = m * eta_base, with m = 10 in production [arXiv §3.3.1; App. C,
Tab. 8]; for MuonH-wrapped matrices eta^H is the effective LR itself.
"""

from __future__ import annotations

import math


def hyperball_lr(eta_base: float, multiplier: float = 10.0) -> float:
    """eta^H = m * eta_base [arXiv §3.3.1]."""
    return multiplier * eta_base


def lr_phase1_power(k: float, peak: float = 5e-3, floor: float = 5e-4,
                    warmup: float = 1000.0, tau: float = 1000.0, p: float = 0.5) -> float:
    """Phase-1 base schedule [arXiv App. C, Eq. (10)]: linear warmup to the
    peak over `warmup` steps, then floor + (peak - floor) (1 + (k - warmup)/tau)^(-p)."""
    if k <= warmup:
        return peak * k / warmup
    return floor + (peak - floor) * (1.0 + (k - warmup) / tau) ** (-p)


def lr_linear(eta0: float, eta_min: float, s: float, S: float) -> float:
    """Linear decay [arXiv App. C, Eq. (11)]: eta0 + (eta_min - eta0) s / S,
    for 0 <= s <= S (s is clamped to that range)."""
    s = min(max(s, 0.0), S)
    return eta0 + (eta_min - eta0) * s / S


def lr_wsd(k: float, peak: float, total: float, decay_ratio: float,
           warmup: float = 0.0, eta_min: float = 0.0) -> float:
    """Warmup-stable-decay with a linear decay over the last decay_ratio*total
    steps [arXiv §3.3.2; App. F.2].  The pages sweep peak and decay ratio but
    print no closed form; this is the plain reading: linear warmup, constant
    peak, linear decay to eta_min at k = total."""
    if warmup > 0.0 and k < warmup:
        return peak * k / warmup
    d0 = total * (1.0 - decay_ratio)
    if k <= d0:
        return peak
    return lr_linear(peak, eta_min, k - d0, total - d0)


def lr_constant_hold(k: float, k_hold: float, schedule) -> float:
    """Constant-LR continuation: the schedule is frozen at its value at step
    k_hold for every k >= k_hold [arXiv §3.4; notes §2.7]."""
    return schedule(min(k, k_hold))


def lr_cosine(k: float, total: float, eta_max: float, eta_min: float,
              warmup: float = 0.0) -> float:
    """Cosine decay from eta_max to eta_min over `total` steps (post-training
    schedule, [arXiv App. E])."""
    if warmup > 0.0 and k < warmup:
        return eta_max * k / warmup
    t = min(max((k - warmup) / max(total - warmup, 1.0), 0.0), 1.0)
    return eta_min + 0.5 * (eta_max - eta_min) * (1.0 + math.cos(math.pi * t))
