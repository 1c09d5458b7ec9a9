"""Seeded random matrices for the workloads.

Recipes (all draws from numpy ``default_rng(SeedSequence([cfg_id, step, idx]))``):
  gaussian  G = N(0,1) entries (the tiny check uses ``default_rng(0)``).
  spiked    G = U diag(linspace(10, 1, r)) V^T + noise * N(0,1), where U
            (rows x r) and V (cols x r) are Gaussian matrices orthonormalised
            by QR with the sign of diag(R) folded in.
  powerlaw  G = U diag(1/i) V^T, i = 1..min(rows, cols), U and V with
            orthonormal columns from QR of Gaussian matrices (no noise).
Matrices are formed in float64 (float32 for the power-law recipe on a GPU)
and stored at the workload dtype with round-to-nearest-even (torch's cast).
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import CONFIGS, WorkloadConfig

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _rng(cfg_id: int, step: int, idx: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, step, idx]))


def _orthonormal(rng: np.random.Generator, n: int, r: int) -> np.ndarray:
    q, rr = np.linalg.qr(rng.standard_normal((n, r)))
    return q * np.sign(np.diag(rr))[None, :]


def gaussian_matrix(rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal((rows, cols))


def spiked_matrix(rows: int, cols: int, rank: int, noise: float,
                  rng: np.random.Generator) -> np.ndarray:
    rank = min(rank, rows, cols)          # tiny test shapes
    u = _orthonormal(rng, rows, rank)
    v = _orthonormal(rng, cols, rank)
    s = np.linspace(10.0, 1.0, rank)
    g = (u * s[None, :]) @ v.T
    if noise:
        g += noise * rng.standard_normal((rows, cols))
    return g


def powerlaw_matrix(rows: int, cols: int, rng: np.random.Generator,
                    device: str = "cpu") -> torch.Tensor:
    """U diag(1/i) V^T; on a GPU device the QR factorisations run there in
    float32 (the Gaussian draws are the same numpy draws either way)."""
    m = min(rows, cols)
    gu = rng.standard_normal((rows, m), dtype=np.float32)
    gv = rng.standard_normal((cols, m), dtype=np.float32)
    s = 1.0 / np.arange(1, m + 1, dtype=np.float64)
    if device == "cpu":
        qu, ru = np.linalg.qr(gu.astype(np.float64))
        qv, rv = np.linalg.qr(gv.astype(np.float64))
        qu *= np.sign(np.diag(ru))[None, :]
        qv *= np.sign(np.diag(rv))[None, :]
        return torch.from_numpy((qu * s[None, :]) @ qv.T)
    tu = torch.from_numpy(gu).to(device)
    tv = torch.from_numpy(gv).to(device)
    qu, ru = torch.linalg.qr(tu)
    qv, rv = torch.linalg.qr(tv)
    qu = qu * torch.sign(torch.diagonal(ru))[None, :]
    qv = qv * torch.sign(torch.diagonal(rv))[None, :]
    st = torch.from_numpy(s.astype(np.float32)).to(device)
    return (qu * st[None, :]) @ qv.t().contiguous()


def make_gradients(cfg: WorkloadConfig, step: int = 0, device: str = "cpu",
                   shapes=None):
    """One gradient per matrix of ``cfg`` (or of ``shapes``), as torch tensors
    of the workload dtype on ``device``."""
    shapes = cfg.shapes if shapes is None else shapes
    tdt = _TORCH_DTYPE[cfg.dtype]
    out = []
    for idx, (r, c) in enumerate(shapes):
        if cfg.generator == "gaussian":
            rng = np.random.default_rng(0) if (cfg.cfg_id == 1 and step == 0 and idx == 0) \
                else _rng(cfg.cfg_id, step, idx)
            t = torch.from_numpy(gaussian_matrix(r, c, rng))
        elif cfg.generator == "spiked":
            t = torch.from_numpy(spiked_matrix(r, c, cfg.spike_rank, cfg.noise,
                                               _rng(cfg.cfg_id, step, idx)))
        elif cfg.generator == "powerlaw":
            t = powerlaw_matrix(r, c, _rng(cfg.cfg_id, step, idx), device)
        else:
            raise ValueError(cfg.generator)
        out.append(t.to(device=device, dtype=tdt).contiguous())
    return out


def make_workload(name: str, step: int = 0, device: str = "cpu", shapes=None):
    """Gradients plus zero-initialised momentum buffers for workload ``name``."""
    cfg = CONFIGS[name]
    grads = make_gradients(cfg, step, device, shapes)
    bufs = [torch.zeros_like(g) for g in grads] if cfg.momentum else None
    return cfg, grads, bufs


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a tensor (bf16 and fp32 upcast exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()
