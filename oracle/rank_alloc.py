"""fp64 CPU oracle of entropy-driven rank allocation.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

MILO (summary at paperlayer.ai/abs/2609.29913v1, "4.3 Dynamic Rank
Allocation") gives every block a rank under a fixed total budget, using
entropy so that slowly decaying spectra receive more: each block starts at a
minimum rank, then the remaining rank units go one at a time to the block
whose next unit has the largest marginal information gain.  Keys and values
may get different ranks ("4.4 MILO Workflow"); each has its own budget.

The pages define neither the entropy nor the gain.  The readings here:
  - a block's spectrum distribution is its normalised energy
        p_i = sigma_i^2 / sum_j sigma_j^2
    per KV head, averaged over the heads (the rank is shared by the
    block's heads), then renormalised to sum 1 (heads without energy
    contribute nothing; a block without energy has p = 0);
  - its entropy is H = -sum_i p_i ln p_i (0 ln 0 = 0): flat spectra have
    high entropy, fast-decaying ones low;
  - the marginal gain of the unit that raises the rank from r to r + u is
    H * (p_r + ... + p_{r+u-1}) (components 0-based, descending): the
    energy fraction the unit adds, weighted by the block's entropy.
Ties go to the lowest block index.  Ranks never exceed head_dim.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def block_distribution(sigma_b: np.ndarray) -> Tuple[float, np.ndarray]:
    """(H, p) of one block from its per-head spectra sigma_b [Hkv][d]."""
    s = np.asarray(sigma_b, dtype=np.float64)
    h, d = s.shape
    p = np.zeros(d)
    for g in range(h):
        e = s[g] ** 2
        tot = e.sum()
        if tot > 0:
            p += e / tot
    p /= h
    tot = p.sum()
    if tot > 0:
        p /= tot
    nz = p[p > 0]
    H = float(-(nz * np.log(nz)).sum())
    return H, p


def unit_gain(H: float, p: np.ndarray, r: int, unit: int) -> float:
    """Gain of raising a block from rank r to r + unit."""
    return H * float(p[r:r + unit].sum())


def allocate(sigma: np.ndarray, budget: int, r_min: int, unit: int = 1) -> np.ndarray:
    """Ranks [n_blocks] for spectra sigma [n_blocks][Hkv][d] (descending per
    head) under a total budget, greedy as the pages describe it."""
    sigma = np.asarray(sigma, dtype=np.float64)
    nb, _, d = sigma.shape
    if unit < 1 or r_min < 0 or r_min > d:
        raise ValueError("unit >= 1 and 0 <= r_min <= head_dim")
    per_block = (d - r_min) // unit
    extra = budget - nb * r_min
    if extra < 0 or extra % unit or extra // unit > nb * per_block:
        raise ValueError("budget must be n_blocks*r_min plus a whole number of units that fit")
    # gains[b][j]: the gain of block b's unit raising rank r_min + j*unit
    gains = []
    for b in range(nb):
        H, p = block_distribution(sigma[b])
        gains.append([unit_gain(H, p, r_min + j * unit, unit) for j in range(per_block)])
    taken = [0] * nb
    for _ in range(extra // unit):
        best, best_g = -1, -1.0
        for b in range(nb):
            if taken[b] == per_block:
                continue
            g = gains[b][taken[b]]
            if g > best_g:
                best, best_g = b, g
        taken[best] += 1
    return np.array([r_min + unit * t for t in taken], dtype=np.int64)


def objective(sigma: np.ndarray, ranks, r_min: int, unit: int = 1) -> float:
    """Total gain of an allocation: the sum of its units' gains above r_min."""
    total = 0.0
    for b, rb in enumerate(ranks):
        H, p = block_distribution(sigma[b])
        for r in range(r_min, int(rb), unit):
            total += unit_gain(H, p, r, unit)
    return total
