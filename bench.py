#!/usr/bin/env python3
"""Benchmark of the MuonH optimizer step on one MI355X.

A "step" is one full MuonH step (momentum + pack, 5 quintic Newton-Schulz
iterations on the grouped MFMA GEMM engine, reductions, Hyperball update)
over every matrix of the workload, with weights, momenta and gradients
resident in HBM.  Default workload: the 196 Qwen3-1.7B-shaped matrices
(28 layers x q, k, v, o, gate, up, down), fp32 W and M, bf16 gradients,
bf16 Newton-Schulz operands with fp32 accumulation.  The AdamW step of the
parameters MuonH does not wrap (embedding, LM head, normalisation weights of
the untied Qwen3-1.7B model) is timed separately and reported beside it.

Prints ONE JSON line on stdout; a human-readable breakdown goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--graph]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MuonH optimizer steps/sec on Qwen3-1.7B weights; NS MFMA util; elementwise HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def per_kernel_work(shapes, ns_steps, tsize, gsize):
    """Algorithmic FLOP / bytes of each kernel family for one step.

    NS products per matrix and iteration (m = min side, n = max side):
      X X^T: 2 m^2 n,  A A: 2 m^3,  B X: 2 m^2 n  (dense counts).
    Elementwise bytes per matrix (p = rows*cols, padded NS area q = m_pad*n_pad):
      momentum: read G (gsize p) + read/write M (8 p) + write X_0 (tsize q; the fp32
                path also writes X_0^T, another tsize q)
      update:   read/write W (8 p) + read u (tsize p)
    (<W,u>, ||u||^2 and ||W||^2 are reduced in the last B X launch's epilogue,
    which reads W (4 p) beside its u stores: counted with that launch, not here.)
    """
    def pad(x):
        return (x + 255) // 256 * 256
    f = {"ns_gram": 0.0, "ns_poly": 0.0, "ns_apply": 0.0}
    b = {"momentum": 0.0, "update": 0.0}
    params = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        f["ns_gram"] += ns_steps * 2.0 * m * m * n
        f["ns_poly"] += ns_steps * 2.0 * m * m * m
        f["ns_apply"] += ns_steps * 2.0 * m * m * n
        p = r * c
        q = pad(m) * pad(n)
        params += p
        b["momentum"] += gsize * p + 8 * p + (1 if tsize == 2 else 2) * tsize * q
        b["update"] += 8 * p + tsize * p
    return f, b, params


def floor_flops(shapes, ns_steps):
    """The method's own Newton-Schulz work per step: the Gram products X X^T
    and A A are symmetric, so half of each suffices (m^2 n and m^3 per
    iteration), and B X is a full product (2 m^2 n): 3 m^2 n + m^3."""
    out = 0.0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        out += ns_steps * (3.0 * m * m * n + 1.0 * m * m * m)
    return out


def exec_flops(shapes, ns_steps, tsize, small: bool, symmetric: bool = True):
    """MFMA FLOP the grouped GEMM issues per step, per product, as the
    library plans it: on the 256 x 256 path every listed output tile runs the
    padded contraction (upper tiles only for X X^T and A A when symmetric);
    on the 64 x 64 path every valid tile runs the valid contraction rounded
    up to its 64-byte K stage."""
    def cdiv(a, b):
        return (a + b - 1) // b
    out = {"ns_gram": 0.0, "ns_poly": 0.0, "ns_apply": 0.0}
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        if small:
            kks = 64 // tsize
            mt, nt = cdiv(m, 64), cdiv(n, 64)
            t2 = 2.0 * 64 * 64
            out["ns_gram"] += ns_steps * t2 * mt * mt * cdiv(n, kks) * kks
            out["ns_poly"] += ns_steps * t2 * mt * mt * cdiv(m, kks) * kks
            out["ns_apply"] += ns_steps * t2 * mt * nt * cdiv(m, kks) * kks
        else:
            mp, np_ = cdiv(m, 256) * 256, cdiv(n, 256) * 256
            mt, nt = mp // 256, np_ // 256
            tri = mt * (mt + 1) // 2 if symmetric else mt * mt
            t2 = 2.0 * 256 * 256
            out["ns_gram"] += ns_steps * t2 * tri * np_
            out["ns_poly"] += ns_steps * t2 * tri * mp
            out["ns_apply"] += ns_steps * t2 * mt * nt * mp
    return out


def synthetic_data_label(wl) -> str:
    """The `data` field: how the workload's synthetic inputs are drawn."""
    grads = {"normal": "N(0,1) grads",
             "fan_in": "N(0,1)/sqrt(fan_in) grads",
             "lowrank": "rank-8 signal (singular values 10^U(-3,1)) plus N(0,1e-3) noise grads"}
    return f"synthetic (seeded {grads[wl.grad_kind]}, W_0 at Frobenius norm sqrt(rows))"


def plan_gemm_path(shapes, ns_steps, tsize, plan_total):
    """(exec_flops, small) on the GEMM path the library's plan took: the one
    whose total equals the plan's executed FLOP (small: the 64 x 64 path)."""
    for small in (False, True):
        ex = exec_flops(shapes, ns_steps, tsize, small)
        if abs(sum(ex.values()) - plan_total) <= 1e-9 * max(plan_total, 1.0):
            return ex, small
    raise RuntimeError("the executed-FLOP model matches neither GEMM path of the plan")


def plan_exec_flops(shapes, ns_steps, tsize, plan_total):
    """exec_flops on the GEMM path the library's plan took."""
    return plan_gemm_path(shapes, ns_steps, tsize, plan_total)[0]


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_apply_qwen3_1.7b_traffic.md")
KERNEL_SOURCES = ("gemm.hip", "device_util.h", "internal.h")


def kernel_source_sha() -> str:
    """SHA-256 of the GEMM sources with comments and blank lines removed, so
    the recorded traffic stays tied to the code it was measured on."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "pretraining_optimizer_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [l.rstrip() for l in text.splitlines() if l.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()


def traffic_for(kernel: str, workload: str, ns: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    profile (FETCH_SIZE and WRITE_SIZE runs, calibrated against a plain copy),
    or None when there is none for this kernel, workload and Newton-Schulz
    type, or the kernel sources changed since."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    kv = {}
    for line in lines:
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            kv[k.strip()] = v.strip().strip("`")
    if (kv.get("kernel-source-sha256") != kernel_source_sha() or kv.get("kernel") != kernel
            or kv.get("workload") != workload or kv.get("ns-dtype") != ns):
        return None
    return float(kv["hbm-bytes-per-launch"])


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline(wl, ws_cpu, grads_cpu, eta, indices):
    """The CPU oracle (fp64 NumPy, as it stands) timed on one step of the
    matrices in `indices` (every matrix of the workload by default), one
    matrix at a time so the host holds one matrix's fp64 state at once.
    Only the oracle step itself is inside the timed region; with a subset
    the time is scaled to the whole set by Newton-Schulz FLOP share."""
    import inputs
    import oracle
    from oracle.muonh import ns_dense_flops
    dt = 0.0
    for j, i in enumerate(indices):
        st = [oracle.OracleMatrixState.from_arrays(inputs.to_numpy64(ws_cpu[j]))]
        g = [inputs.to_numpy64(grads_cpu[j])]
        t0 = time.perf_counter()
        oracle.muonh_step(st, g, eta)
        dt += time.perf_counter() - t0
        del st, g
    share = sum(ns_dense_flops(*wl.shapes[i]) for i in indices) / sum(ns_dense_flops(*s) for s in wl.shapes)
    full = dt / share
    if len(indices) == len(wl.shapes):
        sample = (f"full step: one oracle step (fp64 NumPy) over all {len(indices)} matrices "
                  f"took {dt:.2f} s")
    else:
        sample = (f"one oracle step (fp64 NumPy) over {len(indices)} of {len(wl.shapes)} matrices "
                  f"({share:.4f} of the step's Newton-Schulz FLOP) took {dt:.2f} s; "
                  f"scaled by FLOP share to {full:.1f} s per full step")
    return {"value": 1.0 / full, "unit": "steps/s", "cores": blas_threads(), "kind": "oracle",
            "sample": sample, "seconds_sample": dt, "seconds_full_step": full,
            "host_cpus": os.cpu_count(), "blas_threads": blas_threads()}


def hbm_ceiling(n_elems: int, dev) -> dict:
    """Plain streaming rates of this GPU, measured with PyTorch's own kernels
    on three fp32 buffers of n_elems elements: read-only (sum), write-only (fill),
    copy, and a read-2/write-1 add.  Reads and writes do not stream at the
    same rate, so a kernel's fraction of the 8 TB/s peak is bounded by its
    read/write mix."""
    import torch
    a = torch.ones(n_elems, dtype=torch.float32, device=dev)
    b = torch.ones_like(a)
    c = torch.empty_like(a)
    ops = {"read_sum": (lambda: a.sum(), 4),
           "write_fill": (lambda: c.fill_(1.5), 4),
           "copy": (lambda: c.copy_(a), 8),
           "add_read2_write1": (lambda: torch.add(a, b, out=c), 12)}
    out = {}
    for name, (fn, bpe) in ops.items():
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / 5
        out[name + "_gbs"] = bpe * n_elems / (ms * 1e-3) / 1e9
    del a, b, c
    torch.cuda.empty_cache()
    return out


def time_adamw(steps: int, warmup: int, dev):
    """The AdamW step of the parameters MuonH does not wrap (untied Qwen3-1.7B
    embedding, LM head and normalisation weights), timed with HIP events on
    the stream it is launched on."""
    import torch
    import inputs
    import pretraining_optimizer_amd as pm
    grp = inputs.adamw_group("qwen3_1.7b")
    n = len(grp.tensors)
    ws = [inputs.make_adamw_param(grp, i, dev) for i in range(n)]
    ms = [torch.zeros_like(w) for w in ws]
    vs = [torch.zeros_like(w) for w in ws]
    gs = [inputs.make_adamw_grad(grp, 0, i, dev) for i in range(n)]
    opt = pm.AdamW(ws, ms, vs, grad_dtype=grp.g_dtype)
    for k in range(warmup):
        opt.step(gs, grp.lr(k), k + 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(steps):
        opt.step(gs, grp.lr(warmup + k), warmup + k + 1)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    opt.close()
    gsize = 2 if grp.g_dtype == torch.bfloat16 else 4
    nbytes = grp.params() * (gsize + 24)   # g in; W, m, v (fp32) in and out
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    log(f"adamw group: {grp.params() / 1e9:.3f} G params, {ms_step:.3f} ms/step, {gbs:.0f} GB/s")
    return {"params": grp.params(), "tensors": n, "ms": ms_step, "bytes_per_step": nbytes,
            "gbs": gbs, "frac_of_hbm": gbs / PEAK_HBM_GBS}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_1.7b")
    ap.add_argument("--ns-dtype", choices=("bf16", "f32"), default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-mats", type=int, default=0,
                    help="time the CPU oracle on the first N matrices only and scale by FLOP "
                         "share (default 0: a full step over every matrix)")
    ap.add_argument("--grad-sets", type=int, default=4)
    ap.add_argument("--no-adamw", action="store_true",
                    help="skip timing the AdamW step of the non-MuonH parameters")
    ap.add_argument("--no-hbm-ceiling", action="store_true",
                    help="skip measuring this GPU's plain streaming rates (torch read/write/copy/add)")
    ap.add_argument("--graph", action="store_true",
                    help="time steps replayed from a recorded HIP graph (muonh_step_graph); "
                         "the per-kernel breakdown then comes from a second, eager timed run")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run one plain device-to-device copy of BYTES (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the benchmark runs the step on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the step is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch
    import inputs
    import pretraining_optimizer_amd as pm

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = inputs.workload(args.workload)
    ns = args.ns_dtype or wl.ns_dtype
    log(f"workload {wl.name}: {len(wl.shapes)} matrices, {wl.params() / 1e9:.3f} G params, ns {ns}")

    ws = [inputs.make_weight(wl, i, dev) for i in range(len(wl.shapes))]
    ms = [torch.zeros_like(w) for w in ws]
    nsets = max(1, min(args.grad_sets, args.warmup + args.steps))
    pool = [[inputs.make_grad(wl, k, i, dev) for i in range(len(wl.shapes))] for k in range(nsets)]
    torch.cuda.synchronize()
    cpu_inputs = None
    if not args.no_cpu_baseline:
        # host copies of the step-0 inputs of the timed matrices for the oracle
        # (W_0 before any step; gradients of step 0)
        n_cpu = len(wl.shapes) if args.cpu_mats <= 0 else min(args.cpu_mats, len(wl.shapes))
        cpu_idx = list(range(n_cpu))
        cpu_inputs = ([ws[i].cpu() for i in cpu_idx], [pool[0][i].cpu() for i in cpu_idx])

    if args.copy_calibration > 0:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {4 * n} bytes done")
        del src, dst

    opt = pm.MuonH(ws, ms, grad_dtype=wl.g_dtype,
                   ns_dtype=pm.MUONH_BF16 if ns == "bf16" else pm.MUONH_F32)
    info = pm.plan_query(wl.shapes, pm.default_options(
        ns_dtype=pm.MUONH_BF16 if ns == "bf16" else pm.MUONH_F32), g_dtype=opt._gcode)
    S = opt.options.ns_steps
    for k in range(args.warmup):
        opt.step(pool[k % nsets], wl.eta(k % wl.steps), step=k)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    def timed_run(graph: bool) -> float:
        """Seconds for args.steps steps (eager runs record per-kernel events)."""
        if not graph:
            opt.set_timing(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            kk = args.warmup + k
            opt.step(pool[kk % nsets], wl.eta(kk % wl.steps), step=kk, graph=graph)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    eager_ms = None
    if args.graph:
        for k in range(args.warmup):
            opt.step(pool[k % nsets], wl.eta(k % wl.steps), step=k, graph=True)
        torch.cuda.synchronize()
        dt = timed_run(True)
        log(f"graph steps: {dt * 1e3 / args.steps:.3f} ms/step")
        eager_ms = timed_run(False) * 1e3 / args.steps
        log(f"eager steps (per-kernel events on): {eager_ms:.3f} ms/step")
    else:
        dt = timed_run(False)
    phases, nt = opt.timing()
    opt.set_timing(False)
    ms_per_step = dt * 1e3 / args.steps
    steps_per_s = args.steps / dt
    stats = opt.stats()
    R = opt.radii()
    norm_dev = max(abs(torch.linalg.vector_norm(w.double()).item() / R[i] - 1.0)
                   for i, w in enumerate(ws))
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {steps_per_s:.2f} steps/s; "
        f"max | |W|/R - 1 | = {norm_dev:.2e}; any nonfinite: {any(s['nonfinite'] for s in stats)}")

    tsize = 2 if ns == "bf16" else 4
    gsize = 2 if wl.g_dtype == torch.bfloat16 else 4
    flops, bytes_, params = per_kernel_work(wl.shapes, S, tsize, gsize)
    per_step = {k: v / nt for k, v in phases.items()}
    peak = PEAK_BF16_TFLOPS if ns == "bf16" else PEAK_F32_TFLOPS
    # Per NS kernel: launches per step and FLOP per step three ways --
    #   alg:   the method's own work (X X^T and A A symmetric: m^2 n and m^3
    #          per iteration; B X a full product, 2 m^2 n), the roofline's count;
    #   exec:  the MFMA FLOP the grouped GEMM issues (padding, upper tiles);
    #   dense: the dense-equivalent count (2 m^2 n, 2 m^3, 2 m^2 n).
    launches = {"ns_gram": S, "ns_poly": S, "ns_apply": S - 1, "ns_apply_last": 1}
    ex, small_path = plan_gemm_path(wl.shapes, S, tsize, info.ns_exec_flops)
    last = {"ns_gram": 1.0, "ns_poly": 1.0, "ns_apply": (S - 1) / S, "ns_apply_last": 1.0 / S}
    src = {"ns_gram": "ns_gram", "ns_poly": "ns_poly", "ns_apply": "ns_apply", "ns_apply_last": "ns_apply"}
    half = {"ns_gram": 0.5, "ns_poly": 0.5, "ns_apply": 1.0, "ns_apply_last": 1.0}
    fl_dense = {k: flops[src[k]] * last[k] for k in launches}
    fl_alg = {k: fl_dense[k] * half[k] for k in launches}
    fl_exec = {k: ex[src[k]] * last[k] for k in launches}
    kern = {}
    for k in ("ns_gram", "ns_poly", "ns_apply", "ns_apply_last"):
        if launches[k] == 0:
            continue
        t = per_step[k] * 1e-3   # seconds per step in this kernel
        rate = lambda f: f / t / 1e12
        kern[k] = {"ms_per_launch": per_step[k] / launches[k], "launches_per_step": launches[k],
                   "alg_tflops": rate(fl_alg[k]), "alg_frac_of_peak": rate(fl_alg[k]) / peak,
                   "exec_tflops": rate(fl_exec[k]), "exec_frac_of_peak": rate(fl_exec[k]) / peak,
                   "dense_equiv_tflops": rate(fl_dense[k])}
    for k in ("momentum", "update"):
        gbs = bytes_[k] / (per_step[k] * 1e-3) / 1e9
        kern[k] = {"ms": per_step[k], "gbs": gbs, "frac_of_hbm": gbs / PEAK_HBM_GBS}
    ns_ms = sum(per_step[k] for k in ("ns_gram", "ns_poly", "ns_apply", "ns_apply_last"))
    el_ms = sum(per_step[k] for k in ("momentum", "finalize", "update"))
    ns_s = ns_ms * 1e-3
    ns_floor = floor_flops(wl.shapes, S)
    ns_exec_tflops = info.ns_exec_flops / ns_s / 1e12
    ns_floor_tflops = ns_floor / ns_s / 1e12
    ns_dense_tflops = info.ns_dense_flops / ns_s / 1e12
    el_gbs = sum(bytes_.values()) / (el_ms * 1e-3) / 1e9
    alg_gbs = info.elem_bytes / (el_ms * 1e-3) / 1e9
    for k, v in per_step.items():
        log(f"  {k:13s} {v:8.3f} ms/step  {kern.get(k)}")
    log(f"  NS total {ns_ms:.3f} ms: {ns_exec_tflops:.1f} executed TFLOP/s ({ns_exec_tflops / peak:.1%} "
        f"of peak), {ns_floor_tflops:.1f} on the method's floor ({ns_floor_tflops / peak:.1%}), "
        f"{ns_dense_tflops:.1f} dense-equivalent; elementwise {el_ms:.3f} ms: {el_gbs:.0f} GB/s "
        f"kernel bytes, {alg_gbs:.0f} GB/s at 18 B/param")

    # The dominant kernel: the NS product with the largest share of the step,
    # priced on its algorithmic FLOP.
    names = {"ns_gram": "gemm_kernel<bf16, kGram> (A = X X^T)",
             "ns_poly": "gemm_kernel<bf16, kPoly> (B' = b A + c A A + a I)",
             "ns_apply": "gemm_kernel<bf16, kApply> (X' = B' X)",
             "ns_apply_last": "gemm_kernel<bf16, kApplyLast> (u = B' X)"}
    if ns != "bf16":
        names = {k: v.replace("<bf16", "<fp32") for k, v in names.items()}
    if small_path:
        names = {k: v.replace("gemm_kernel<", "gemm_small_kernel<") for k, v in names.items()}
    dom = max((k for k in kern if k in names), key=lambda k: per_step[k])
    roof = {"bound": "mfma", "achieved": kern[dom]["alg_tflops"], "peak": peak, "unit": "TFLOP/s",
            "frac": kern[dom]["alg_tflops"] / peak, "traffic": traffic_for(dom, wl.name, ns),
            "kernel": names[dom], "flop_per_launch": fl_alg[dom] / launches[dom],
            "ms_per_launch": kern[dom]["ms_per_launch"]}

    adamw = None if args.no_adamw else time_adamw(args.steps, args.warmup, dev)
    ceiling = None
    if not args.no_hbm_ceiling:
        ceiling = hbm_ceiling(max(params, 1 << 28), dev)
        log("plain streaming on this GPU (torch, fp32, one buffer of the workload's size): " +
            ", ".join(f"{k} {v:.0f} GB/s" for k, v in ceiling.items()))

    cpu = None
    if cpu_inputs is not None:
        log(f"cpu baseline: oracle on {len(cpu_idx)} matrices ...")
        cpu = cpu_baseline(wl, cpu_inputs[0], cpu_inputs[1], wl.eta(0), cpu_idx)
        log(f"  {cpu['sample']}; {cpu['value']:.5f} steps/s on {cpu['cores']} BLAS threads")

    out = {
        "metric": METRIC, "value": steps_per_s, "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ns, "data": synthetic_data_label(wl),
        "config": {"workload": f"{wl.name}: {len(wl.shapes)} matrices, {params} params, fp32 W/M, "
                               f"{'bf16' if gsize == 2 else 'fp32'} grads, {ns} Newton-Schulz x{S}",
                   "matrices": len(wl.shapes), "params": params, "parallelism": "single-gpu"},
        "roofline": roof,
        # NS phase rates: on the MFMA FLOP executed (the utilisation), on the
        # method's floor 3 m^2 n + m^3 per iteration, and dense-equivalent
        "ns_frac_of_peak": ns_exec_tflops / peak,
        "ns_exec_tflops": ns_exec_tflops, "ns_exec_frac_of_peak": ns_exec_tflops / peak,
        "ns_floor_tflops": ns_floor_tflops, "ns_floor_frac_of_peak": ns_floor_tflops / peak,
        "ns_dense_equiv_tflops": ns_dense_tflops, "ns_dense_equiv_frac": ns_dense_tflops / peak,
        "ns_exec_tflop_per_step": info.ns_exec_flops / 1e12,
        "ns_floor_tflop_per_step": ns_floor / 1e12,
        "ns_dense_tflop_per_step": info.ns_dense_flops / 1e12,
        "elementwise_gbs": el_gbs, "elementwise_frac_of_hbm": el_gbs / PEAK_HBM_GBS,
        "elementwise_alg18_gbs": alg_gbs,
        "step_path": "recorded HIP graph" if args.graph else "eager launches",
        "eager_ms_per_step": eager_ms,
        "kernels": kern, "phase_ms_per_step": per_step, "timed_steps_events": nt,
        "norm_invariant_max_dev": norm_dev,
        "adamw_group": adamw,
        "hbm_streaming_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    opt.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
