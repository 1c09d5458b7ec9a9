"""Float64 CPU oracle for the Muon Newton-Schulz update (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python binding)
never does; see ``oracle/muon_oracle.py`` for the arithmetic and its sources.
"""
from .muon_oracle import (  # noqa: F401
    bf16_round,
    fp32_round,
    two_sum,
    round_exact_sum,
    momentum_update,
    frobenius_normalize,
    newton_schulz,
    ns_polynomial_step,
    orthogonalize,
    muon_update,
    apply_weight,
    adam_update,
    falg_flops,
)
