"""The five matrix-set workloads of the Muon Newton-Schulz update.

Shapes follow GPT-2 hidden weight matrices (a block has four d x d attention
projections q, k, v, o, one d x 4d and one 4d x d MLP matrix). The pages run
Muon on the hidden matrices of a 124M GPT-2 in the speedrun (blog.hotdry.top,
"How to train a GPT model in 3 minutes", section 2, Muon item) and name a
350M GPT-2 medium track (yongjin360.com Modded-NanoGPT article). Real
gradients and weights are not available; the generators in ``generators.py``
stand in for them with spectra of the stated kinds.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


def _gpt2_set(layers: int, d: int, mlp: int) -> List[Tuple[int, int]]:
    shapes: List[Tuple[int, int]] = []
    # grouped by shape: all square attention matrices, then the wide MLP
    # matrices, then the tall ones
    shapes += [(d, d)] * (4 * layers)
    shapes += [(d, mlp)] * layers
    shapes += [(mlp, d)] * layers
    return shapes


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    cfg_id: int                       # seed component
    shapes: Tuple[Tuple[int, int], ...]
    dtype: str                        # "fp32" or "bf16" (grads, buffers, out)
    generator: str                    # "gaussian" | "spiked" | "powerlaw"
    coeffs: Tuple[float, float, float]
    steps: int
    momentum: float
    nesterov: bool
    spike_rank: int = 0
    noise: float = 0.0
    eps: float = 1e-7
    tol: float = field(default=2e-2)  # relative Frobenius error bound per matrix

    @property
    def n_matrices(self) -> int:
        return len(self.shapes)

    def falg_flops(self) -> int:
        tot = 0
        for r, c in self.shapes:
            m, n = min(r, c), max(r, c)
            tot += self.steps * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n)
        return tot

    def elements(self) -> int:
        return sum(r * c for r, c in self.shapes)


CONFIGS = {
    # one fp32 64 x 128 matrix, N(0,1) from seed 0, cubic coefficients, 10 steps
    "tiny_fp32_64x128_cubic": WorkloadConfig(
        name="tiny_fp32_64x128_cubic", cfg_id=1, shapes=((64, 128),), dtype="fp32",
        generator="gaussian", coeffs=CUBIC, steps=10, momentum=0.0, nesterov=False,
        tol=1e-4),
    # one GPT-2-small block (d = 768)
    "gpt2_small_block": WorkloadConfig(
        name="gpt2_small_block", cfg_id=2, shapes=tuple(_gpt2_set(1, 768, 3072)),
        dtype="bf16", generator="spiked", coeffs=QUINTIC, steps=5, momentum=0.95,
        nesterov=True, spike_rank=8, noise=0.1),
    # all 72 hidden matrices of GPT-2 124M (12 layers)
    "gpt2_124m_matrix_set": WorkloadConfig(
        name="gpt2_124m_matrix_set", cfg_id=3, shapes=tuple(_gpt2_set(12, 768, 3072)),
        dtype="bf16", generator="spiked", coeffs=QUINTIC, steps=5, momentum=0.95,
        nesterov=True, spike_rank=8, noise=0.1),
    # GPT-2 medium (350M) shapes: 24 layers, d = 1024
    "gpt2_350m_matrix_set": WorkloadConfig(
        name="gpt2_350m_matrix_set", cfg_id=4, shapes=tuple(_gpt2_set(24, 1024, 4096)),
        dtype="bf16", generator="spiked", coeffs=QUINTIC, steps=5, momentum=0.95,
        nesterov=True, spike_rank=16, noise=0.1),
    # large-width stress: 32 wide + 32 tall 2048 x 8192, power-law spectrum
    "wide_2048x8192_powerlaw": WorkloadConfig(
        name="wide_2048x8192_powerlaw", cfg_id=5,
        shapes=tuple([(2048, 8192)] * 32 + [(8192, 2048)] * 32),
        dtype="bf16", generator="powerlaw", coeffs=QUINTIC, steps=5, momentum=0.95,
        nesterov=True),
}


def config_names():
    return list(CONFIGS)
