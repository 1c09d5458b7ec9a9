"""Seeded synthetic workloads (matrix sets and their gradients).

This package holds input recipes only: shapes, seeds and random draws. It
contains none of the update's arithmetic, so both the float64 oracle and the
HIP path can take their inputs from it without sharing any computation.
"""
from .configs import CONFIGS, WorkloadConfig, config_names  # noqa: F401
from .generators import (  # noqa: F401
    gaussian_matrix,
    spiked_matrix,
    powerlaw_matrix,
    make_gradients,
    make_workload,
    to_f64,
)
from .sharding import matrix_flops, owner_split  # noqa: F401
from .adam import (  # noqa: F401
    gpt2_124m_adam_shapes,
    gpt2_124m_adam_multipliers,
    make_adam_state,
    new_grads,
)
