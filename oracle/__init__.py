"""CPU fp64 oracle for the MuonH optimizer step and the AdamW step of the
parameters MuonH does not wrap.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
statement of what the GPU library computes.  Only the tests, the smoke check
and the CPU-baseline leg of the benchmark may import it; the product path
(``pretraining_optimizer_amd``) never does, and the two share no code.

Sources (the pages are cited by title and section / equation only):

* "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090"
  (arXiv HTML), cited below as [arXiv].
* "Puro-2B：低成本从零预训练的系统、优化与数据配方" (reading notes on the
  same paper), cited below as [notes].

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (SVD closed forms, textbook special cases, invariants,
values printed on the pages).  The one choice no page fixes is the
Newton-Schulz coefficient values (a reading, configurable): the functions
that use them are pinned by their mathematics for any coefficients, but which
values the authors ran cannot be checked from the pages.
"""

from .muonh import (  # noqa: F401
    NS_COEFFS_QUINTIC,
    NS_COEFFS_CLASSICAL,
    OracleOptions,
    OracleMatrixState,
    fro,
    radius,
    momentum_update,
    ns_input,
    newton_schulz,
    hyperball_update,
    muon_wd_update,
    elr_aligned_update,
    muonh_step,
    muonh_trajectory,
    chord_angle,
    closed_form_angle,
)
from .schedules import (  # noqa: F401
    lr_phase1_power,
    lr_linear,
    lr_wsd,
    lr_constant_hold,
    lr_cosine,
    hyperball_lr,
)
from .adamw import (  # noqa: F401
    AdamWOptions,
    adamw_step,
    adamw_trajectory,
    adamw_bytes_per_element,
    first_step_direction,
    constant_gradient_closed_form,
)
