"""fp64 CPU oracle for the EMA-Gram quarter-power preconditioner step.

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline may import this package. It shares no code with the HIP library.
"""

from .step import (  # noqa: F401
    FLAG_NONFINITE,
    FLAG_NOT_PD,
    FLAG_ZERO_TRACE,
    NORM_NONE,
    NORM_TRACE,
    gram_ema_update,
    hyperball_update,
    inv_quarter_root,
    inv_sqrt_root,
    left_gram,
    momentum_ema,
    polar_cans,
    precondition_apply,
    preconditioner_step,
    relative_frobenius,
    rescale,
    right_gram,
    run_sequence,
)
