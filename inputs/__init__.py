"""Seeded synthetic workloads for the MuonH step.

This module only *makes inputs*: shapes, seeded random weights and
gradients, and the per-step effective-LR values of each workload.  It holds
none of the optimizer's arithmetic, so both the GPU library's tests and the
CPU oracle can consume the same bytes from it.

Weight shapes follow the PyTorch Linear convention (out x in) and the model
dimensions of [arXiv App. D, Tab. 10] (Qwen3-0.6B: d_model 1024, d_ff 3072;
Qwen3-1.7B: d_model 2048, d_ff 6144; 16 query / 8 KV heads of width 128).

Random streams: every (workload seed, step, matrix index, role) gets its own
torch.Generator seed, so any subset of matrices can be regenerated on its own
and a CPU and a GPU run draw identical values when both use the same device.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np
import torch

Shape = Tuple[int, int]

ROLE_W, ROLE_G = 1, 2
ROLE_AW, ROLE_AG = 3, 4     # parameters / gradients of the AdamW group


def stream_seed(seed: int, step: int, index: int, role: int) -> int:
    """Deterministic 63-bit seed for one (workload, step, matrix, role)."""
    h = (seed * 0x9E3779B97F4A7C15 + (step + 1) * 0xBF58476D1CE4E5B9
         + (index + 1) * 0x94D049BB133111EB + role * 0xD6E8FEB86659FD93)
    h &= (1 << 64) - 1
    h ^= h >> 31
    return h & ((1 << 63) - 1)


def _randn(shape: Shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


# ---------------------------------------------------------------------------
# shape sets


def qwen3_layer_shapes(d_model: int, d_ff: int, n_q: int = 16, n_kv: int = 8,
                       head: int = 128) -> List[Tuple[str, Shape]]:
    """The seven attention / MLP matrices of one Qwen3 decoder layer."""
    q = n_q * head
    kv = n_kv * head
    return [
        ("q", (q, d_model)), ("k", (kv, d_model)), ("v", (kv, d_model)),
        ("o", (d_model, q)), ("gate", (d_ff, d_model)), ("up", (d_ff, d_model)),
        ("down", (d_model, d_ff)),
    ]


def qwen3_fused_layer_shapes(d_model: int, d_ff: int, n_q: int = 16, n_kv: int = 8,
                             head: int = 128) -> List[Tuple[str, Shape]]:
    """The same layer with the projections that share an input fused into
    one matrix each: qkv = [q; k; v] and gate_up = [gate; up]."""
    q = n_q * head
    kv = n_kv * head
    return [("qkv", (q + 2 * kv, d_model)), ("o", (d_model, q)),
            ("gate_up", (2 * d_ff, d_model)), ("down", (d_model, d_ff))]


def diag170m_layer_shapes() -> List[Tuple[str, Shape]]:
    return [("q", (768, 768)), ("k", (768, 768)), ("v", (768, 768)), ("o", (768, 768)),
            ("gate", (2048, 768)), ("up", (2048, 768)), ("down", (768, 2048))]


def stress_shapes(seed: int = 0, count: int = 64) -> List[Tuple[str, Shape]]:
    """64 matrices with aspect ratios 1:1 to 1:8 and every side in [128, 4096].
    Even index: wide (short, long); odd index: tall (long, short)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        a = 2.0 ** rng.uniform(0.0, 3.0)
        s = int(round(2.0 ** rng.uniform(7.0, 12.0 - math.log2(a))))
        s = min(max(s, 128), 4096)
        l = min(4096, max(s, int(round(s * a))))
        shape = (s, l) if i % 2 == 0 else (l, s)
        out.append((f"s{i}", shape))
    return out


# ---------------------------------------------------------------------------
# workloads


@dataclasses.dataclass
class Workload:
    name: str
    matrices: List[Tuple[str, Shape]]
    g_dtype: torch.dtype              # dtype the gradients are stored in
    ns_dtype: str                     # "bf16" or "f32": Newton-Schulz operand type
    steps: int
    beta: float
    eta: Callable[[int], float]       # effective LR at step k (0-based)
    w_std: float = 1.0                # W_0 ~ N(0, w_std^2) before rescaling
    grad_kind: str = "normal"         # "normal", "fan_in", "lowrank"
    seed: int = 0

    @property
    def shapes(self) -> List[Shape]:
        return [s for _, s in self.matrices]

    def params(self) -> int:
        return sum(r * c for r, c in self.shapes)


def _linear_decay(peak: float, total: int) -> Callable[[int], float]:
    return lambda k: peak * (1.0 - k / total)


# Phase-2 start of the production schedule: the Phase-1 power law evaluated
# at the end of Phase 1 (438.84B tokens at 1536 x 4096 tokens per step),
# decayed linearly to 1e-5 by the last step of the run (222,569), times the
# Hyperball multiplier 10 [arXiv App. C, Eqs. (10)-(11); notes §2.7].
_TOKENS_PER_STEP = 1536 * 4096
_K1 = 438.84e9 / _TOKENS_PER_STEP
_ETA0 = 5e-4 + 4.5e-3 * (1.0 + (_K1 - 1000.0) / 1000.0) ** -0.5
_S2 = 222569 - 69752


def _phase2_start(k: int) -> float:
    return 10.0 * (_ETA0 + (1e-5 - _ETA0) * k / _S2)


def workload(name: str) -> Workload:
    """The synthetic workloads (shapes, dtypes, steps and LR)."""
    if name == "single":
        return Workload("single", [("w", (256, 128))], torch.float32, "f32", 3, 0.95,
                        lambda k: 0.01, w_std=0.02)
    if name == "diag170m":
        mats = [(f"l{l}.{n}", s) for l in range(12) for n, s in diag170m_layer_shapes()]
        return Workload("diag170m", mats, torch.bfloat16, "bf16", 20, 0.95,
                        _linear_decay(0.012, 20), grad_kind="fan_in")
    if name == "qwen3_0.6b":
        mats = [(f"l{l}.{n}", s) for l in range(28) for n, s in qwen3_layer_shapes(1024, 3072)]
        return Workload("qwen3_0.6b", mats, torch.bfloat16, "bf16", 10, 0.95,
                        _linear_decay(0.024, 10))
    if name == "qwen3_1.7b":
        mats = [(f"l{l}.{n}", s) for l in range(28) for n, s in qwen3_layer_shapes(2048, 6144)]
        return Workload("qwen3_1.7b", mats, torch.bfloat16, "bf16", 10, 0.95, _phase2_start)
    if name == "qwen3_1.7b_fused":
        mats = [(f"l{l}.{n}", s) for l in range(28) for n, s in qwen3_fused_layer_shapes(2048, 6144)]
        return Workload("qwen3_1.7b_fused", mats, torch.bfloat16, "bf16", 10, 0.95, _phase2_start)
    if name == "stress":
        return Workload("stress", stress_shapes(0), torch.float32, "f32", 3, 0.95,
                        lambda k: 0.02, grad_kind="lowrank")
    raise KeyError(name)


WORKLOADS = ("single", "diag170m", "qwen3_0.6b", "qwen3_1.7b", "qwen3_1.7b_fused", "stress")


# ---------------------------------------------------------------------------
# tensors


def make_weight(wl: Workload, index: int, device="cpu") -> torch.Tensor:
    """W_0 for matrix `index`: N(0, w_std^2), rescaled to Frobenius norm sqrt(rows)."""
    r, c = wl.shapes[index]
    w = _randn((r, c), stream_seed(wl.seed, 0, index, ROLE_W), device) * wl.w_std
    w = w * (math.sqrt(r) / torch.linalg.vector_norm(w.double()).item())
    return w.contiguous()


def _lowrank_grad(shape: Shape, seed: int, rank: int = 8) -> np.ndarray:
    """Rank-8 signal with singular values 10^U(-3,1) plus N(0, 1e-3) noise
    (variance 1e-3)."""
    rng = np.random.default_rng(seed)
    r, c = shape
    uq, _ = np.linalg.qr(rng.standard_normal((r, rank)))
    vq, _ = np.linalg.qr(rng.standard_normal((c, rank)))
    sv = 10.0 ** rng.uniform(-3.0, 1.0, size=rank)
    return (uq * sv) @ vq.T + math.sqrt(1e-3) * rng.standard_normal((r, c))


def make_grad(wl: Workload, step: int, index: int, device="cpu") -> torch.Tensor:
    """Gradient of matrix `index` at step `step`, stored in wl.g_dtype
    (bf16 values are the round-to-nearest-even image of fp32 draws)."""
    r, c = wl.shapes[index]
    seed = stream_seed(wl.seed, step, index, ROLE_G)
    if wl.grad_kind == "lowrank":
        g = torch.from_numpy(_lowrank_grad((r, c), seed % (2 ** 32))).to(torch.float32).to(device)
    else:
        g = _randn((r, c), seed, device)
        if wl.grad_kind == "fan_in":
            g = g * (1.0 / math.sqrt(c))
    return g.to(wl.g_dtype).contiguous()


def make_weights(wl: Workload, device="cpu", indices: Optional[Sequence[int]] = None):
    idx = range(len(wl.shapes)) if indices is None else indices
    return [make_weight(wl, i, device) for i in idx]


def make_grads(wl: Workload, step: int, device="cpu", indices: Optional[Sequence[int]] = None):
    idx = range(len(wl.shapes)) if indices is None else indices
    return [make_grad(wl, step, i, device) for i in idx]


def to_numpy64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a (possibly bf16) tensor, on the host."""
    return t.detach().to("cpu", torch.float64).numpy()


# ---------------------------------------------------------------------------
# the AdamW parameter group (embeddings, normalisation layers, LM head)

# Qwen3 tokenizer vocabulary.  The pages state only that the untied Qwen3-1.7B
# architecture has about 2B parameters [arXiv §2.1]; with this vocabulary the
# embedding and LM head add 2 x 151936 x 2048 = 0.62B to the 1.41B of the
# MuonH matrices (2.03B in total).
QWEN3_VOCAB = 151936


@dataclasses.dataclass
class AdamwGroup:
    name: str
    tensors: List[Tuple[str, int, str]]   # (name, numel, kind: "matrix" | "norm")
    g_dtype: torch.dtype
    steps: int
    lr: Callable[[int], float]            # base LR at step k (0-based)
    seed: int = 0

    def numels(self) -> List[int]:
        return [n for _, n, _ in self.tensors]

    def params(self) -> int:
        return sum(self.numels())


def qwen3_adamw_tensors(d_model: int, layers: int = 28, head: int = 128,
                        vocab: int = QWEN3_VOCAB) -> List[Tuple[str, int, str]]:
    """Flat sizes of the parameters AdamW trains in the untied Qwen3
    architecture: embedding and LM head [vocab x d_model]; per layer the two
    RMSNorm weights and the q / k head norms; the final norm."""
    out = [("embed", vocab * d_model, "matrix"), ("lm_head", vocab * d_model, "matrix")]
    for l in range(layers):
        out += [(f"l{l}.input_norm", d_model, "norm"), (f"l{l}.post_attn_norm", d_model, "norm"),
                (f"l{l}.q_norm", head, "norm"), (f"l{l}.k_norm", head, "norm")]
    out.append(("final_norm", d_model, "norm"))
    return out


def _phase2_base(k: int) -> float:
    return _ETA0 + (1e-5 - _ETA0) * k / _S2


RAGGED_ADAMW = [1, 3, 5, 1000, 4096, 16384, 16385, 70001, 6149]


def adamw_group(name: str) -> AdamwGroup:
    """'qwen3_1.7b': the AdamW group of the untied Qwen3-1.7B model at the
    Phase-2 start of the base schedule; 'ragged_bf16' / 'ragged_f32': small
    tensors with ragged sizes for element-by-element parity."""
    if name == "qwen3_1.7b":
        return AdamwGroup(name, qwen3_adamw_tensors(2048), torch.bfloat16, 10, _phase2_base)
    if name in ("ragged_bf16", "ragged_f32"):
        ts = [(f"t{i}", n, "norm" if i % 3 == 0 else "matrix") for i, n in enumerate(RAGGED_ADAMW)]
        g = torch.bfloat16 if name == "ragged_bf16" else torch.float32
        return AdamwGroup(name, ts, g, 4, lambda k: 3e-3 * (1.0 - k / 8.0), seed=7)
    raise KeyError(name)


def make_adamw_param(grp: AdamwGroup, index: int, device="cpu") -> torch.Tensor:
    """Parameter `index` at step 0: N(0, 0.02^2) for matrices, 1 + N(0, 0.02^2)
    for normalisation weights (fp32, flat)."""
    _, n, kind = grp.tensors[index]
    p = _randn((n,), stream_seed(grp.seed, 0, index, ROLE_AW), device) * 0.02
    if kind == "norm":
        p = p + 1.0
    return p.contiguous()


def make_adamw_grad(grp: AdamwGroup, step: int, index: int, device="cpu") -> torch.Tensor:
    """Gradient of tensor `index` at step `step`: N(0, 1), stored in grp.g_dtype."""
    _, n, _ = grp.tensors[index]
    return _randn((n,), stream_seed(grp.seed, step, index, ROLE_AG), device).to(grp.g_dtype).contiguous()
