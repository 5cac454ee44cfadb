"""ctypes binding of libmuonh.so (argument marshalling only).

The C entry points keep their names (muonh_init, muonh_step, ...); the
MuonH class below only turns torch tensors into device pointers and the
current torch stream into a hipStream_t.  Every step of the optimizer runs in
the library's HIP kernels; there is no Python or CPU fallback: loading fails
loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmuonh.so")

MUONH_OK = 0
MUONH_EINVAL = -1
MUONH_EMISMATCH = -2
MUONH_ENOMEM = -3
MUONH_EHIP = -4
MUONH_ESTATE = -5
MUONH_ENODEV = -6

MUONH_F32 = 0
MUONH_BF16 = 1

MUONH_MODE_HYPERBALL = 0
MUONH_MODE_MUON_WD = 1
MUONH_MODE_ELR_ALIGNED = 2

PHASES = ("momentum", "ns_gram", "ns_poly", "ns_apply", "ns_apply_last", "finalize", "update")


class muonh_matrix_desc(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("g_dtype", ctypes.c_int32), ("radius", ctypes.c_float)]


class muonh_options(ctypes.Structure):
    _fields_ = [("beta", ctypes.c_float), ("ns_steps", ctypes.c_int32),
                ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
                ("ns_eps", ctypes.c_float), ("ns_dtype", ctypes.c_int32),
                ("nesterov", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("weight_decay", ctypes.c_float), ("symmetric", ctypes.c_int32),
                ("deterministic", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class muonh_step_args(ctypes.Structure):
    _fields_ = [("elr", ctypes.c_float), ("elr_scale", ctypes.POINTER(ctypes.c_float)),
                ("step", ctypes.c_int64), ("want_stats", ctypes.c_int32)]


class muonh_adamw_tensor(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("numel", ctypes.c_int64), ("g_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class muonh_adamw_options(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float)]


class muonh_stats(ctypes.Structure):
    _fields_ = [("y_norm", ctypes.c_double), ("u_norm", ctypes.c_double),
                ("w_norm", ctypes.c_double), ("inner", ctypes.c_double), ("c", ctypes.c_double),
                ("wt_norm", ctypes.c_double), ("elr", ctypes.c_double),
                ("angle", ctypes.c_double), ("nonfinite", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


class muonh_plan_info(ctypes.Structure):
    _fields_ = [("n_matrices", ctypes.c_int32), ("n_buckets", ctypes.c_int32),
                ("gemm_tiles", ctypes.c_int64 * 3), ("mom_tiles", ctypes.c_int64),
                ("flat_chunks", ctypes.c_int64), ("ns_dense_flops", ctypes.c_double),
                ("ns_exec_flops", ctypes.c_double), ("elem_bytes", ctypes.c_double),
                ("workspace_bytes", ctypes.c_size_t)]


_libs = {}

# (name, restype, argtypes)
_SIGNATURES = [
    ("muonh_default_options", None, [ctypes.POINTER(muonh_options)]),
    ("muonh_workspace_size", ctypes.c_int, [ctypes.POINTER(muonh_matrix_desc), ctypes.c_int32,
                                            ctypes.POINTER(muonh_options), ctypes.POINTER(ctypes.c_size_t)]),
    ("muonh_plan_query", ctypes.c_int, [ctypes.POINTER(muonh_matrix_desc), ctypes.c_int32,
                                        ctypes.POINTER(muonh_options), ctypes.POINTER(muonh_plan_info)]),
    ("muonh_init", ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(muonh_matrix_desc),
                                  ctypes.c_int32, ctypes.POINTER(muonh_options), ctypes.c_void_p]),
    ("muonh_step", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(muonh_matrix_desc), ctypes.c_int32,
                                  ctypes.POINTER(muonh_step_args), ctypes.c_void_p]),
    ("muonh_step_graph", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(muonh_matrix_desc), ctypes.c_int32,
                                        ctypes.POINTER(muonh_step_args), ctypes.c_void_p]),
    ("muonh_step_noalloc", ctypes.c_int, [ctypes.POINTER(muonh_matrix_desc), ctypes.c_int32,
                                          ctypes.POINTER(muonh_options), ctypes.POINTER(muonh_step_args),
                                          ctypes.c_void_p]),
    ("muonh_get_radii", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int32]),
    ("muonh_get_stats", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(muonh_stats), ctypes.c_int32]),
    ("muonh_copy_update", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    ("muonh_set_timing", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("muonh_get_timing", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int32)]),
    ("muonh_destroy", ctypes.c_int, [ctypes.c_void_p]),
    ("muonh_status_str", ctypes.c_char_p, [ctypes.c_int]),
    ("muonh_last_error", ctypes.c_char_p, []),
    ("muonh_lr_linear", ctypes.c_double, [ctypes.c_double] * 4),
    ("muonh_lr_power", ctypes.c_double, [ctypes.c_double] * 6),
    ("muonh_lr_wsd", ctypes.c_double, [ctypes.c_double] * 6),
    ("muonh_lr_linear_hold", ctypes.c_double, [ctypes.c_double] * 5),
    ("muonh_lr_cosine", ctypes.c_double, [ctypes.c_double] * 5),
    ("muonh_elr_from_base", ctypes.c_double, [ctypes.c_double] * 2),
    ("muonh_adamw_default_options", None, [ctypes.POINTER(muonh_adamw_options)]),
    ("muonh_adamw_init", ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(muonh_adamw_tensor),
                                        ctypes.c_int32, ctypes.POINTER(muonh_adamw_options)]),
    ("muonh_adamw_step", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(muonh_adamw_tensor), ctypes.c_int32,
                                        ctypes.c_float, ctypes.c_int64, ctypes.c_void_p]),
    ("muonh_adamw_destroy", ctypes.c_int, [ctypes.c_void_p]),
]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmuonh.so (once per path); raises if it has not been built."""
    path = os.path.abspath(path)
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m pretraining_optimizer_amd.build`"
                           " (or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, res, args in _SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _libs[path] = lib
    return lib


class MuonHError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = load_library()
        super().__init__(f"{what}: {lib.muonh_status_str(status).decode()} ({status}): "
                         f"{lib.muonh_last_error().decode()}")
        self.status = status


def _check(status: int, what: str):
    if status != MUONH_OK:
        raise MuonHError(status, what)


def default_options(**kw) -> muonh_options:
    lib = load_library()
    o = muonh_options()
    lib.muonh_default_options(ctypes.byref(o))
    for k, v in kw.items():
        if not hasattr(o, k):
            raise KeyError(k)
        setattr(o, k, v)
    return o


def shape_descs(shapes: Sequence, g_dtype: int = MUONH_BF16, radius: float = 1.0):
    """Descriptors with shapes only (for the host-side queries)."""
    arr = (muonh_matrix_desc * len(shapes))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows, arr[i].cols, arr[i].g_dtype, arr[i].radius = r, c, g_dtype, radius
    return arr


def plan_query(shapes: Sequence, options: Optional[muonh_options] = None,
               g_dtype: int = MUONH_BF16) -> muonh_plan_info:
    lib = load_library()
    opt = options or default_options()
    info = muonh_plan_info()
    descs = shape_descs(shapes, g_dtype)
    _check(lib.muonh_plan_query(descs, len(shapes), ctypes.byref(opt), ctypes.byref(info)),
           "muonh_plan_query")
    return info


def workspace_size(shapes: Sequence, options: Optional[muonh_options] = None,
                   g_dtype: int = MUONH_BF16) -> int:
    lib = load_library()
    opt = options or default_options()
    n = ctypes.c_size_t()
    _check(lib.muonh_workspace_size(shape_descs(shapes, g_dtype), len(shapes), ctypes.byref(opt),
                                    ctypes.byref(n)), "muonh_workspace_size")
    return n.value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MUONH_BF16
    if t.dtype == torch.float32:
        return MUONH_F32
    raise TypeError(f"unsupported gradient dtype {t.dtype}")


def _stream_ptr(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _record(stream, tensors):
    """Work enqueued on a stream other than torch's current one reads and
    writes these tensors asynchronously: tell torch's caching allocator, so
    their memory is not handed out again before that stream has passed them."""
    import torch
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        t.record_stream(stream)


class MuonH:
    """One MuonH optimizer over a list of fp32 CUDA matrices (W, M in place).

    weights, moms : lists of contiguous fp32 CUDA tensors of equal shapes
    grad_dtype    : torch dtype of the gradients passed to step()
    radii         : optional per-matrix R (resume); default R = ||W_0||_F
    options       : keyword overrides of muonh_options (beta, ns_steps, ...)
    """

    def __init__(self, weights: List, moms: List, grad_dtype=None, radii=None, stream=None,
                 **options):
        import torch
        self._lib = load_library()
        if len(weights) != len(moms) or not weights:
            raise ValueError("weights and moms must be non-empty lists of equal length")
        grad_dtype = torch.bfloat16 if grad_dtype is None else grad_dtype
        for w, m in zip(weights, moms):
            if not (w.is_cuda and m.is_cuda):
                raise ValueError("weights and momenta must be CUDA tensors")
            if w.dtype != torch.float32 or m.dtype != torch.float32:
                raise TypeError("weights and momenta must be float32")
            if w.dim() != 2 or w.shape != m.shape or not w.is_contiguous() or not m.is_contiguous():
                raise ValueError("weights/momenta must be contiguous 2-D tensors of equal shape")
        self.n = len(weights)
        self.shapes = [tuple(w.shape) for w in weights]
        self.weights, self.moms = list(weights), list(moms)
        self._gcode = {torch.bfloat16: MUONH_BF16, torch.float32: MUONH_F32}[grad_dtype]
        self.options = default_options(**options)
        descs = (muonh_matrix_desc * self.n)()
        for i, (w, m) in enumerate(zip(weights, moms)):
            descs[i].w, descs[i].g, descs[i].m = w.data_ptr(), None, m.data_ptr()
            descs[i].rows, descs[i].cols = w.shape
            descs[i].g_dtype = self._gcode
            descs[i].radius = 0.0 if radii is None else float(radii[i])
        h = ctypes.c_void_p()
        _check(self._lib.muonh_init(ctypes.byref(h), descs, self.n, ctypes.byref(self.options),
                                    _stream_ptr(stream)), "muonh_init")
        self._h = h
        self._descs = descs

    def step(self, grads: Sequence, elr: float, elr_scale: Optional[Sequence[float]] = None,
             step: int = 0, stream=None, graph: bool = False):
        """One step; graph=True goes through muonh_step_graph (a recorded HIP graph)."""
        if len(grads) != self.n:
            raise ValueError("one gradient per matrix is required")
        d = self._descs
        for i, g in enumerate(grads):
            if not g.is_cuda or not g.is_contiguous() or tuple(g.shape) != self.shapes[i]:
                raise ValueError(f"gradient {i}: must be a contiguous CUDA tensor of shape {self.shapes[i]}")
            if _dtype_code(g) != self._gcode:
                raise TypeError(f"gradient {i}: dtype differs from the one given at init")
            d[i].w = self.weights[i].data_ptr()
            d[i].g = g.data_ptr()
            d[i].m = self.moms[i].data_ptr()
        _record(stream, list(grads) + self.weights + self.moms)
        args = muonh_step_args()
        args.elr = float(elr)
        scale_arr = None
        if elr_scale is not None:
            scale_arr = (ctypes.c_float * self.n)(*[float(x) for x in elr_scale])
            args.elr_scale = ctypes.cast(scale_arr, ctypes.POINTER(ctypes.c_float))
        args.step = int(step)
        fn, name = ((self._lib.muonh_step_graph, "muonh_step_graph") if graph
                    else (self._lib.muonh_step, "muonh_step"))
        _check(fn(self._h, d, self.n, ctypes.byref(args), _stream_ptr(stream)), name)

    def radii(self) -> List[float]:
        out = (ctypes.c_float * self.n)()
        _check(self._lib.muonh_get_radii(self._h, out, self.n), "muonh_get_radii")
        return list(out)

    def stats(self) -> List[dict]:
        out = (muonh_stats * self.n)()
        _check(self._lib.muonh_get_stats(self._h, out, self.n), "muonh_get_stats")
        return [s.as_dict() for s in out]

    def copy_update(self, idx: int, stream=None):
        """The Newton-Schulz output u of matrix idx from the last step (fp32 CUDA tensor)."""
        import torch
        r, c = self.shapes[idx]
        dst = torch.empty((r, c), dtype=torch.float32, device=self.weights[idx].device)
        _record(stream, [dst])
        _check(self._lib.muonh_copy_update(self._h, idx, dst.data_ptr(), _stream_ptr(stream)),
               "muonh_copy_update")
        return dst

    def set_timing(self, enable: bool = True):
        _check(self._lib.muonh_set_timing(self._h, 1 if enable else 0), "muonh_set_timing")

    def timing(self):
        """(per-phase total milliseconds, number of timed steps) since the last read."""
        out = (ctypes.c_float * len(PHASES))()
        n = ctypes.c_int32()
        _check(self._lib.muonh_get_timing(self._h, out, len(PHASES), ctypes.byref(n)),
               "muonh_get_timing")
        return dict(zip(PHASES, list(out))), n.value

    def close(self):
        if getattr(self, "_h", None):
            self._lib.muonh_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# Bytes of device workspace the allocation-free step can use per GPU (the
# header's MUONH_NOALLOC_MAX_WORKSPACE).
NOALLOC_MAX_WORKSPACE = 64 << 20


def step_noalloc(weights: Sequence, moms: Sequence, grads: Sequence, radii: Sequence[float],
                 elr: float, elr_scale: Optional[Sequence[float]] = None, step: int = 0,
                 stream=None, **options):
    """One MuonH step through muonh_step_noalloc: no handle, no device
    allocation (the library's static per-GPU buffer holds the workspace).
    weights, moms: contiguous fp32 CUDA matrices (updated in place); grads:
    contiguous CUDA gradients (bf16 or fp32, one dtype); radii: R per matrix
    (> 0); options: muonh_options overrides (beta, ns_dtype, ...)."""
    lib = load_library()
    n = len(weights)
    if not (n and len(moms) == n and len(grads) == n and len(radii) == n):
        raise ValueError("weights, moms, grads and radii must be non-empty lists of equal length")
    d = (muonh_matrix_desc * n)()
    for i, (w, m, g) in enumerate(zip(weights, moms, grads)):
        if not (w.is_cuda and m.is_cuda and g.is_cuda) or w.dim() != 2:
            raise ValueError(f"matrix {i}: CUDA tensors of two dims are required")
        if w.shape != m.shape or w.shape != g.shape:
            raise ValueError(f"matrix {i}: weight, momentum and gradient shapes differ")
        if not (w.is_contiguous() and m.is_contiguous() and g.is_contiguous()):
            raise ValueError(f"matrix {i}: tensors must be contiguous")
        d[i].w, d[i].g, d[i].m = w.data_ptr(), g.data_ptr(), m.data_ptr()
        d[i].rows, d[i].cols = w.shape
        d[i].g_dtype = _dtype_code(g)
        d[i].radius = float(radii[i])
    _record(stream, list(grads) + list(weights) + list(moms))
    opt = default_options(**options)
    args = muonh_step_args()
    args.elr = float(elr)
    scale_arr = None
    if elr_scale is not None:
        scale_arr = (ctypes.c_float * n)(*[float(x) for x in elr_scale])
        args.elr_scale = ctypes.cast(scale_arr, ctypes.POINTER(ctypes.c_float))
    args.step = int(step)
    _check(lib.muonh_step_noalloc(d, n, ctypes.byref(opt), ctypes.byref(args), _stream_ptr(stream)),
           "muonh_step_noalloc")


def adamw_default_options(**overrides) -> muonh_adamw_options:
    opt = muonh_adamw_options()
    load_library().muonh_adamw_default_options(ctypes.byref(opt))
    for k, v in overrides.items():
        if not hasattr(opt, k):
            raise KeyError(f"unknown AdamW option {k}")
        setattr(opt, k, v)
    return opt


class AdamW:
    """AdamW over a list of fp32 CUDA tensors (parameters, first and second
    moments updated in place), one multi-tensor launch per step.

    params, exp_avgs, exp_avg_sqs : lists of contiguous fp32 CUDA tensors
    grad_dtype                    : torch dtype of the gradients passed to step()
    options                       : beta1, beta2, eps, weight_decay overrides
    """

    def __init__(self, params: List, exp_avgs: List, exp_avg_sqs: List, grad_dtype=None,
                 **options):
        import torch
        self._lib = load_library()
        if not params or not (len(params) == len(exp_avgs) == len(exp_avg_sqs)):
            raise ValueError("params, exp_avgs and exp_avg_sqs must be non-empty lists of equal length")
        grad_dtype = torch.bfloat16 if grad_dtype is None else grad_dtype
        for p, m, v in zip(params, exp_avgs, exp_avg_sqs):
            for t in (p, m, v):
                if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
                    raise ValueError("params and moments must be contiguous fp32 CUDA tensors")
            if p.numel() != m.numel() or p.numel() != v.numel():
                raise ValueError("a parameter and its moments must have the same size")
        self.n = len(params)
        self.params, self.exp_avgs, self.exp_avg_sqs = list(params), list(exp_avgs), list(exp_avg_sqs)
        self.numels = [p.numel() for p in params]
        self._gcode = {torch.bfloat16: MUONH_BF16, torch.float32: MUONH_F32}[grad_dtype]
        self.options = adamw_default_options(**options)
        d = (muonh_adamw_tensor * self.n)()
        for i in range(self.n):
            d[i].numel = self.numels[i]
            d[i].g_dtype = self._gcode
        h = ctypes.c_void_p()
        _check(self._lib.muonh_adamw_init(ctypes.byref(h), d, self.n, ctypes.byref(self.options)),
               "muonh_adamw_init")
        self._h = h
        self._d = d

    def step(self, grads: Sequence, lr: float, step: int, stream=None):
        """One step at step count `step` (1-based) with learning rate `lr`."""
        if len(grads) != self.n:
            raise ValueError("one gradient per tensor is required")
        d = self._d
        for i, g in enumerate(grads):
            if not g.is_cuda or not g.is_contiguous() or g.numel() != self.numels[i]:
                raise ValueError(f"gradient {i}: must be a contiguous CUDA tensor of {self.numels[i]} elements")
            if _dtype_code(g) != self._gcode:
                raise TypeError(f"gradient {i}: dtype differs from the one given at init")
            d[i].w = self.params[i].data_ptr()
            d[i].g = g.data_ptr()
            d[i].m = self.exp_avgs[i].data_ptr()
            d[i].v = self.exp_avg_sqs[i].data_ptr()
        _record(stream, list(grads) + self.params + self.exp_avgs + self.exp_avg_sqs)
        _check(self._lib.muonh_adamw_step(self._h, d, self.n, float(lr), int(step), _stream_ptr(stream)),
               "muonh_adamw_step")

    def close(self):
        if getattr(self, "_h", None):
            self._lib.muonh_adamw_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
