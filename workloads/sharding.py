"""Matrix ownership for a data-parallel Muon step over several GPUs.

The update is independent per matrix, so a sharded step gives each rank a
subset of the matrices: a reduce-scatter delivers the summed gradients of the
matrices a rank owns, the rank runs the update on them, and an all-gather
returns the results. This module only decides the subsets (host logic); the
step on one GPU is the library, unchanged, on a rank's subset.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def matrix_flops(rows: int, cols: int) -> int:
    """Algorithmic flops of one Newton-Schulz step on one matrix: the Gram
    and A A on their symmetric halves plus B X, with m = min, n = max."""
    m, n = min(rows, cols), max(rows, cols)
    return m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n


def owner_split(shapes: Sequence[Tuple[int, int]], world: int) -> List[List[int]]:
    """Indices of the matrices each of `world` ranks owns: longest first
    (stable order among equals), each onto the rank with the least work so
    far (the lower rank on ties). Every matrix goes to exactly one rank."""
    if world < 1:
        raise ValueError("world must be >= 1")
    cost = [matrix_flops(r, c) for r, c in shapes]
    order = sorted(range(len(shapes)), key=lambda i: -cost[i])
    load = [0] * world
    owned: List[List[int]] = [[] for _ in range(world)]
    for i in order:
        k = min(range(world), key=lambda r: (load[r], r))
        owned[k].append(i)
        load[k] += cost[i]
    return [sorted(o) for o in owned]
