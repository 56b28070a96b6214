"""Plain fp64 CPU oracle for the batched Muon step -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python
binding) never imports, calls or links it, and it shares no code with that
path: no kernels, helpers, tables or constants.

See `oracle.muon` for what is computed and where each step comes from.
"""
from .muon import (  # noqa: F401
    QUINTIC_COEFFS,
    momentum_update,
    frobenius_normalize,
    newton_schulz,
    update_scale,
    apply_update,
    muon_matrix_step,
    muon_step,
    nominal_ns_flops,
)
