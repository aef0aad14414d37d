"""Test-only fp64 CPU oracle of the whole-tensor Muon step.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The product path never does.
"""

from .muon_ref import (  # noqa: F401
    DEFAULT_EPS,
    DEFAULT_NS_STEPS,
    QUINTIC_COEFFS,
    frobenius_norm,
    frobenius_normalize,
    momentum_update,
    muon_step,
    newton_schulz,
    orthogonalize,
    step_flops,
    update_scale,
)
