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
# Localised-error gates on u_hat, as multiples of the Frobenius tolerance of
# the path: the largest row (column) error relative to the RMS row (column)
# norm, and the largest element error relative to the RMS element.  A whole
# wrong column of a 2048 x 6144 matrix moves the Frobenius ratio by only
# sqrt(1/6144) = 1.3e-2, but its own column error by about 1.
ROW_COL_FACTOR = 2.0
ELEM_FACTOR = 12.0


def rel(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (nb if nb > 0 else 1.0)


def unit(a: np.ndarray) -> np.ndarray:
    n = float(np.linalg.norm(a))
    return a / n if n != 0 else a


def local_errors(a: np.ndarray, b: np.ndarray):
    """(row, col, elem) errors of a against the reference b: the largest
    ||a_i - b_i|| over rows i divided by the RMS row norm of b, the same over
    columns, and the largest |a_ij - b_ij| divided by the RMS element of b."""
    d = a - b
    nb = float(np.linalg.norm(b))
    if nb == 0.0:
        return 0.0, 0.0, 0.0
    r, c = b.shape
    row = float(np.sqrt(np.max(np.einsum("ij,ij->i", d, d)))) / (nb / math.sqrt(r))
    col = float(np.sqrt(np.max(np.einsum("ij,ij->j", d, d)))) / (nb / math.sqrt(c))
    elem = float(np.max(np.abs(d))) / (nb / math.sqrt(r * c))
    return row, col, elem


def singular_vector_agreement(u_hat: np.ndarray, svd) -> float:
    """How far u_hat is from sharing the singular vectors of the NS input Y
    (svd = numpy's thin SVD (U, s, V^T) of Y): with C = U^T u_hat V, the
    energy of u_hat off the diagonal of C plus the energy outside the spans
    of U and V, over ||u_hat||:
        sqrt(||C - diag(C)||^2 + ||u_hat - U C V^T||^2) / ||u_hat||.
    The Newton-Schulz output is U p(S) V^T exactly, for which this is 0.
    Both terms are formed directly (not as ||u_hat||^2 - ||diag C||^2, whose
    cancellation floors the measure at about 1e-8)."""
    U, _, Vt = svd
    n = float(np.linalg.norm(u_hat))
    if n == 0.0:
        return 0.0
    C = U.T @ u_hat @ Vt.T
    off = C - np.diag(np.diag(C))
    rest = u_hat - U @ C @ Vt
    return math.sqrt(float(np.sum(off * off)) + float(np.sum(rest * rest))) / n


@dataclasses.dataclass
class StepReport:
    step: int
    u_err: List[float]        # per checked matrix: ||u^_gpu - u^_oracle|| (both unit norm)
    w_err: List[float]        # ||W_gpu - W_oracle|| / ||W_oracle||
    m_err: List[float]
    norm_err: List[float]     # | ||W_gpu|| / R - 1 |, ALL matrices
    stats: List[dict]
    oracle_diag: list
    u_row: List[float] = dataclasses.field(default_factory=list)   # local_errors of u^
    u_col: List[float] = dataclasses.field(default_factory=list)
    u_elem: List[float] = dataclasses.field(default_factory=list)
    checked: List[int] = dataclasses.field(default_factory=list)   # matrix index of each entry
    sv_err: dict = dataclasses.field(default_factory=dict)        # index -> singular-vector agreement


def announce(msg: str):
    print(f"[parity] {msg}", flush=True)


def run_parity(shapes: Sequence, make_w: Callable[[int], torch.Tensor],
               make_g: Callable[[int, int], torch.Tensor], etas: Sequence[float],
               check: Sequence[int], ns: str = "bf16", oracle_opts: Optional[oracle.OracleOptions] = None,
               mode: int = pm.MUONH_MODE_HYPERBALL, weight_decay: float = 0.0,
               elr_scale: Optional[Sequence[float]] = None, radii=None, graph: bool = False,
               check_first: Sequence[int] = (), svd_of: Optional[Callable] = None,
               **lib_opts) -> List[StepReport]:
    """make_w(i) -> fp32 CUDA tensor, make_g(step, i) -> CUDA gradient.
    graph=True takes every step through the recorded-graph entry point.
    The oracle follows the matrices in `check` through every step; those in
    `check_first` are checked at the first step only, one at a time (their
    W_0 is made again with make_w, so no host copy of the whole set is kept).
    svd_of(i, y) -> thin SVD of matrix i's first Newton-Schulz input y, or
    None: when given, the first step also records the singular-vector
    agreement of every checked u_hat (StepReport.sv_err)."""
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

        def compare(i, st, g, u_gpu, w_gpu, m_gpu):
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
            a, b = unit(u_gpu), unit(u)
            rep.u_err.append(rel(a, b))
            lr, lc, le = local_errors(a, b)
            rep.u_row.append(lr)
            rep.u_col.append(lc)
            rep.u_elem.append(le)
            rep.checked.append(i)
            rep.w_err.append(rel(w_gpu, st.w))
            rep.m_err.append(rel(m_gpu, st.m))
            if svd_of is not None and k == 0:
                sv = svd_of(i, y)
                if sv is not None:
                    rep.sv_err[i] = (singular_vector_agreement(a, sv), singular_vector_agreement(b, sv))

        for i in check:
            compare(i, states[i], inputs.to_numpy64(gs[i]), us[i], inputs.to_numpy64(ws[i]),
                    inputs.to_numpy64(ms[i]))
        if k == 0:
            for i in check_first:
                if i in states:
                    continue
                st = oracle.OracleMatrixState.from_arrays(
                    inputs.to_numpy64(make_w(i)), R=None if radii is None else radii[i])
                if radii is None:
                    assert abs(R[i] / st.R - 1.0) < 1e-6, (i, R[i], st.R)
                u_gpu = inputs.to_numpy64(opt.copy_update(i))
                compare(i, st, inputs.to_numpy64(gs[i]), u_gpu, inputs.to_numpy64(ws[i]),
                        inputs.to_numpy64(ms[i]))
                rep.oracle_diag[-1] = None   # drop the fp64 u of a matrix not followed further
                del st, u_gpu
        if mode == pm.MUONH_MODE_HYPERBALL:
            for i, w in enumerate(ws):
                wn = torch.linalg.vector_norm(w.double()).item()
                rep.norm_err.append(abs(wn / R[i] - 1.0))
        reports.append(rep)
        announce(f"step {k}: {len(rep.u_err)} matrices checked; max u^ err {max(rep.u_err):.3e} "
                 f"(row {max(rep.u_row):.3e}, col {max(rep.u_col):.3e}, elem {max(rep.u_elem):.3e}), "
                 f"max W err {max(rep.w_err):.3e}, max M err {max(rep.m_err):.3e}, max |W|/R-1 "
                 f"{max(rep.norm_err) if rep.norm_err else float('nan'):.2e}")
        if rep.sv_err:
            g_sv = max(v[0] for v in rep.sv_err.values())
            o_sv = max(v[1] for v in rep.sv_err.values())
            announce(f"step {k}: singular-vector agreement (off-diagonal energy of U^T u^ V): "
                     f"library max {g_sv:.3e}, oracle max {o_sv:.3e}")
    opt.close()
    return reports


def summarize(name: str, reports: List[StepReport]) -> dict:
    """Largest errors over all steps and checked matrices, announced and, when
    MUONH_PARITY_LOG names a file, appended to it as one JSON line (the
    margins under each gate)."""
    import json
    import os
    out = {"case": name, "steps": len(reports),
           "matrices_checked_first_step": len(reports[0].u_err) if reports else 0}
    for key in ("u_err", "u_row", "u_col", "u_elem", "w_err", "m_err", "norm_err"):
        vals = [v for r in reports for v in getattr(r, key)]
        out[key] = max(vals) if vals else None
    sv = [v for r in reports for v in r.sv_err.values()]
    if sv:
        out["sv_lib"] = max(v[0] for v in sv)
        out["sv_oracle"] = max(v[1] for v in sv)
    announce("summary " + json.dumps(out))
    path = os.environ.get("MUONH_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(out) + "\n")
    return out


def workload_fns(wl: inputs.Workload, device="cuda"):
    return (lambda i: inputs.make_weight(wl, i, device),
            lambda k, i: inputs.make_grad(wl, k, i, device))


def check_reports(reports: List[StepReport], tol_u: float, etas: Sequence[float],
                  tol_norm: float = TOL_NORM):
    acc = 0.0
    for rep, eta in zip(reports, etas):
        acc += abs(eta)
        assert max(rep.u_err) <= tol_u, (rep.step, rep.u_err)
        assert max(rep.u_row) <= ROW_COL_FACTOR * tol_u, (rep.step, "row", rep.u_row)
        assert max(rep.u_col) <= ROW_COL_FACTOR * tol_u, (rep.step, "col", rep.u_col)
        assert max(rep.u_elem) <= ELEM_FACTOR * tol_u, (rep.step, "elem", rep.u_elem)
        assert max(rep.m_err) <= TOL_MOM, (rep.step, rep.m_err)
        # W moves by eta*R*u^ per step, so its error is bounded by the
        # accumulated step sizes times the u^ tolerance (plus fp32 rounding).
        assert max(rep.w_err) <= 2.0 * acc * tol_u + 1e-5, (rep.step, rep.w_err)
        if rep.norm_err:
            assert max(rep.norm_err) <= tol_norm, (rep.step, max(rep.norm_err))
