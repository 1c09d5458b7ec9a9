"""Seeded synthetic inputs for the Adam branch: the GPT-2 124M parameters
that stay off the Muon path (token and position embeddings, LayerNorm scales
and shifts, linear-layer biases), and random parameter/gradient/moment
tensors of any shapes. Input recipes only; no optimizer arithmetic."""
from __future__ import annotations

from typing import List, Tuple

import torch

D_MODEL, N_LAYER, VOCAB, CTX = 768, 12, 50257, 1024


def gpt2_124m_adam_shapes() -> List[Tuple[int, ...]]:
    """Shapes of GPT-2 124M's non-projection parameters, in model order:
    wte (vocab x d), wpe (ctx x d), then per block ln_1 (scale, shift), the
    attention's qkv and output biases, ln_2 (scale, shift), the MLP's two
    biases, and the final LayerNorm (39.5 M elements in all)."""
    d = D_MODEL
    shapes: List[Tuple[int, ...]] = [(VOCAB, d), (CTX, d)]
    for _ in range(N_LAYER):
        shapes += [(d,), (d,), (3 * d,), (d,), (d,), (d,), (4 * d,), (d,)]
    shapes += [(d,), (d,)]
    return shapes


def gpt2_124m_adam_multipliers(shapes) -> Tuple[List[float], List[float]]:
    """(lr_mul, wd_mul) per tensor: 1.0 learning-rate multipliers, and no
    weight decay on the one-dimensional biases and scales."""
    return [1.0] * len(shapes), [0.0 if len(s) == 1 else 1.0 for s in shapes]


def make_adam_state(shapes, dtype: torch.dtype, seed: int, device="cpu", moments="random"):
    """params ~ 0.02 N(0,1), grads ~ 1e-3 N(0,1) in ``dtype``; float32
    moments, zero or a plausible mid-training state (m ~ 1e-4 N, v ~ 1e-6 U)."""
    gen = torch.Generator().manual_seed(seed)
    params, grads, ms, vs = [], [], [], []
    for s in shapes:
        params.append((0.02 * torch.randn(s, generator=gen)).to(dtype).to(device))
        grads.append((1e-3 * torch.randn(s, generator=gen)).to(dtype).to(device))
        if moments == "zero":
            ms.append(torch.zeros(s, dtype=torch.float32, device=device))
            vs.append(torch.zeros(s, dtype=torch.float32, device=device))
        else:
            ms.append((1e-4 * torch.randn(s, generator=gen)).to(device))
            vs.append((1e-6 * torch.rand(s, generator=gen)).to(device))
    return params, grads, ms, vs


def new_grads(grads, seed: int):
    """Overwrites the gradient tensors in place with a fresh seeded draw."""
    gen = torch.Generator().manual_seed(seed)
    for g in grads:
        g.copy_((1e-3 * torch.randn(g.shape, generator=gen)).to(g.dtype))
