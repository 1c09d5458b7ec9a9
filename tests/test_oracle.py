"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_tiny_fp32_draw_and_polar_error():
    """The tiny check: N(0,1) 64 x 128 from seed 0 stored in fp32, 10 cubic
    steps; its first entries and its distance to U V^T."""
    from workloads import make_workload, to_f64
    cfg, grads, bufs = make_workload("tiny_fp32_64x128_cubic")
    g = to_f64(grads[0])
    assert np.allclose(g[0, :3], [0.12573022, -0.13210486, 0.64042264], atol=1e-8)
    out = oracle.orthogonalize(g, *cfg.coeffs, cfg.steps, cfg.eps)
    U, _, Vt = np.linalg.svd(g, full_matrices=False)
    err = np.linalg.norm(out - U @ Vt) / np.linalg.norm(U @ Vt)
    assert abs(err - 4.742e-4) < 5e-6


def test_falg_flops_matches_workload_totals():
    from workloads import CONFIGS
    c3 = CONFIGS["gpt2_124m_matrix_set"]
    tot = sum(oracle.falg_flops(r, c, c3.steps) for r, c in c3.shapes)
    assert tot == c3.falg_flops() == 1142158786560
