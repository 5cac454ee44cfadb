"""Shared driver of the GPU parity tests: run the library and the CPU oracle
on byte-identical inputs and collect per-matrix errors."""

from __future__ import annotations

import dataclasses
import math
from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

import inputs
import oracle
import pretraining_optimizer_amd as pm

# Tolerances (per-matrix relative Frobenius error of u_hat; norm invariant).
TOL_BF16 = 2e-2
TOL_F32 = 1e-4
TOL_NORM = 1e-5
TOL_MOM = 1e-6


def rel(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (nb if nb > 0 else 1.0)


def unit(a: np.ndarray) -> np.ndarray:
    n = float(np.linalg.norm(a))
    return a / n if n != 0 else a


@dataclasses.dataclass
class StepReport:
    step: int
    u_err: List[float]        # per checked matrix: ||u^_gpu - u^_oracle|| (both unit norm)
    w_err: List[float]        # ||W_gpu - W_oracle|| / ||W_oracle||
    m_err: List[float]
    norm_err: List[float]     # | ||W_gpu|| / R - 1 |, ALL matrices
    stats: List[dict]
    oracle_diag: list


def announce(msg: str):
    print(f"[parity] {msg}", flush=True)


def run_parity(shapes: Sequence, make_w: Callable[[int], torch.Tensor],
               make_g: Callable[[int, int], torch.Tensor], etas: Sequence[float],
               check: Sequence[int], ns: str = "bf16", oracle_opts: Optional[oracle.OracleOptions] = None,
               mode: int = pm.MUONH_MODE_HYPERBALL, weight_decay: float = 0.0,
               elr_scale: Optional[Sequence[float]] = None, radii=None, graph: bool = False,
               **lib_opts) -> List[StepReport]:
    """make_w(i) -> fp32 CUDA tensor, make_g(step, i) -> CUDA gradient.
    graph=True takes every step through the recorded-graph entry point."""
    dev = torch.device("cuda")
    oo = oracle_opts or oracle.OracleOptions()
    ws = [make_w(i).to(dev).contiguous() for i in range(len(shapes))]
    ms = [torch.zeros_like(w) for w in ws]
    gdt = make_g(0, 0).dtype
    w0 = {i: inputs.to_numpy64(ws[i]) for i in check}
    opt = pm.MuonH(ws, ms, grad_dtype=gdt, radii=radii,
                   ns_dtype=pm.MUONH_BF16 if ns == "bf16" else pm.MUONH_F32,
                   beta=oo.beta, ns_steps=oo.ns_steps, nesterov=int(oo.nesterov),
                   ns_a=oo.ns_coeffs[0], ns_b=oo.ns_coeffs[1], ns_c=oo.ns_coeffs[2],
                   ns_eps=oo.ns_eps, mode=mode, weight_decay=weight_decay, **lib_opts)
    R = opt.radii()
    states = {i: oracle.OracleMatrixState.from_arrays(w0[i], R=None if radii is None else radii[i])
              for i in check}
    if radii is None:
        for i in check:
            assert abs(R[i] / states[i].R - 1.0) < 1e-6, (i, R[i], states[i].R)
    reports = []
    for k, eta in enumerate(etas):
        gs = [make_g(k, i).to(dev).contiguous() for i in range(len(shapes))]
        opt.step(gs, eta, elr_scale=elr_scale, step=k, graph=graph)
        us = {i: inputs.to_numpy64(opt.copy_update(i)) for i in check}
        torch.cuda.synchronize()
        stats = opt.stats()
        rep = StepReport(k, [], [], [], [], stats, [])
        for i in check:
            st = states[i]
            g = inputs.to_numpy64(gs[i])
            st.m = oracle.momentum_update(st.m, g, oo.beta)
            y = oracle.ns_input(st.m, g, oo.beta, oo.nesterov)
            u = oracle.newton_schulz(y, oo.ns_steps, oo.ns_coeffs, oo.ns_eps, oo.orient)
            e = eta * (1.0 if elr_scale is None else elr_scale[i])
            if mode == pm.MUONH_MODE_HYPERBALL:
                st.w, d = oracle.hyperball_update(st.w, u, e, st.R)
            elif mode == pm.MUONH_MODE_MUON_WD:
                st.w, d = oracle.muon_wd_update(st.w, u, e, weight_decay), None
            else:
                st.w, d = oracle.elr_aligned_update(st.w, u, e)
            rep.oracle_diag.append((u, d))
            rep.u_err.append(rel(unit(us[i]), unit(u)))
            rep.w_err.append(rel(inputs.to_numpy64(ws[i]), st.w))
            rep.m_err.append(rel(inputs.to_numpy64(ms[i]), st.m))
        if mode == pm.MUONH_MODE_HYPERBALL:
            for i, w in enumerate(ws):
                wn = torch.linalg.vector_norm(w.double()).item()
                rep.norm_err.append(abs(wn / R[i] - 1.0))
        reports.append(rep)
        announce(f"step {k}: max u^ err {max(rep.u_err):.3e}, max W err {max(rep.w_err):.3e}, "
                 f"max M err {max(rep.m_err):.3e}, max |W|/R-1 "
                 f"{max(rep.norm_err) if rep.norm_err else float('nan'):.2e}")
    opt.close()
    return reports


def workload_fns(wl: inputs.Workload, device="cuda"):
    return (lambda i: inputs.make_weight(wl, i, device),
            lambda k, i: inputs.make_grad(wl, k, i, device))


def check_reports(reports: List[StepReport], tol_u: float, etas: Sequence[float],
                  tol_norm: float = TOL_NORM):
    acc = 0.0
    for rep, eta in zip(reports, etas):
        acc += abs(eta)
        assert max(rep.u_err) <= tol_u, (rep.step, rep.u_err)
        assert max(rep.m_err) <= TOL_MOM, (rep.step, rep.m_err)
        # W moves by eta*R*u^ per step, so its error is bounded by the
        # accumulated step sizes times the u^ tolerance (plus fp32 rounding).
        assert max(rep.w_err) <= 2.0 * acc * tol_u + 1e-5, (rep.step, rep.w_err)
        if rep.norm_err:
            assert max(rep.norm_err) <= tol_norm, (rep.step, max(rep.norm_err))
