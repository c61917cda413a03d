"""fp64 CPU oracle of the encode step: per-block low-rank factors of dense
keys and values.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library and reads the dense context drawn by
``synth`` (stored values, converted exactly to float64).

MILO (summary at paperlayer.ai/abs/2609.29913v1) approximates the keys and
the values of each block *separately* by low-rank factors ("4.2 Block-wise
Low-Rank Compression"), at block-specific ranks ("4.3 Dynamic Rank
Allocation"; keys and values may differ, "4.4 MILO Workflow").  The pages do
not name the factorisation; the reading here is the truncated SVD, which is
the best rank-r approximation in Frobenius norm (Eckart-Young), and the
spectrum it produces is what the entropy-driven rank allocation consumes.

For a block X (T x d) with SVD X = U_x diag(s) V_x^T the rank-r factors are
    W = V_x[:, :r]^T          (r x d, orthonormal rows)
    U = X W^T                 (T x r, equal to U_x[:, :r] diag(s[:r]))
so that U W = X V_r V_r^T, the projection of X's rows onto its top-r right
singular subspace.  The library routine ``numpy.linalg.svd`` is the one
step taken from a library; everything else is written out below.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np


def block_spectrum(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Singular values s (length d, descending, zeros past min(T, d)) and a
    full orthonormal basis vt (d x d) whose row i is the right singular
    vector of s[i]."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    if T == 0:
        return np.zeros(d), np.eye(d)
    _, s, vt = np.linalg.svd(x, full_matrices=True)
    sf = np.zeros(d)
    sf[:len(s)] = s
    return sf, vt


def encode_block(x: np.ndarray, r: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rank-r factors (U: T x r, W: r x d) of one dense block, and its spectrum."""
    x = np.asarray(x, dtype=np.float64)
    s, vt = block_spectrum(x)
    w = vt[:r]
    u = x @ w.T
    return u, w, s


def approx(x: np.ndarray, r: int) -> np.ndarray:
    """The rank-r approximation U W of a dense block."""
    u, w, _ = encode_block(x, r)
    return u @ w


def context_spectra(ctx) -> np.ndarray:
    """Singular values of every (block, KV head, K/V) of a ``synth``
    DenseContext: float64 [n_blocks][Hkv][2][d]."""
    nb, h, d = len(ctx.n_tok), ctx.cfg.n_kv_heads, ctx.cfg.head_dim
    out = np.zeros((nb, h, 2, d))
    for b in range(nb):
        for g in range(h):
            for kv in range(2):
                out[b, g, kv] = block_spectrum(ctx.dense_f64(kv, b, g))[0]
    return out


def context_approx(ctx, ranks: np.ndarray, blocks: Optional[List[int]] = None):
    """Rank-(r_b, r'_b) approximations of the given blocks (default all):
    {b: float64 [Hkv][2][T_b][d]}."""
    h = ctx.cfg.n_kv_heads
    res = {}
    for b in (range(len(ctx.n_tok)) if blocks is None else blocks):
        T, d = int(ctx.n_tok[b]), ctx.cfg.head_dim
        a = np.zeros((h, 2, T, d))
        for g in range(h):
            for kv in range(2):
                a[g, kv] = approx(ctx.dense_f64(kv, b, g), int(ranks[b][kv]))
        res[b] = a
    return res
