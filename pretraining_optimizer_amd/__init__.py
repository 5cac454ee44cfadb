"""MI355X (gfx950) MuonH optimizer step: HIP kernels behind a C ABI.

The library (libmuonh.so, built from csrc/ by ``build.py``) runs momentum,
quintic Newton-Schulz on a grouped bf16/fp32 MFMA GEMM engine and the
Hyperball update of Eq. (1) of "Puro-2B: Poor Lab's Qwen2-1.5B Trained on
RTX 5090 within $5090" (arXiv HTML §3.3), plus the AdamW step of the
parameters MuonH does not wrap.  ``muonh`` is its ctypes binding.
"""

from .muonh import (  # noqa: F401
    AdamW,
    MuonH,
    MuonHError,
    NOALLOC_MAX_WORKSPACE,
    adamw_default_options,
    default_options,
    load_library,
    plan_query,
    step_noalloc,
    workspace_size,
    MUONH_BF16,
    MUONH_F32,
    MUONH_MODE_HYPERBALL,
    MUONH_MODE_MUON_WD,
    MUONH_MODE_ELR_ALIGNED,
)
