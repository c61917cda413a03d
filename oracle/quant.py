"""CPU oracle of 8-bit factor quantisation (the quantised-factor variant).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

MILO (summary at paperlayer.ai/abs/2609.29913v1, "5.3 Performance Analysis")
combines its low-rank cache with asymmetric INT8 quantisation.  The pages
give neither the grouping nor the rounding; the reading here quantises the
token factors U^T and U'^T of every block and KV head row by row (one rank
component over the block's tokens: a per-channel group), asymmetrically:
    lo = min_t x_t,  hi = max_t x_t,  scale = (hi - lo) / 255,
    code_t = clamp(round_half_even((x_t - lo) / scale), 0, 255)   (0 if scale is 0),
    x_t ~= scale * code_t + lo.
The codes are integers decided by floating point, so this oracle takes that
decision in the precision the kernel uses: every step above in IEEE fp32
(numpy float32 operations, correctly rounded division).  W and W' are not
quantised.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def quantize_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Codes uint8 [rows][n], scale float32 [rows], bias float32 [rows] of a
    float32 array x [rows][n] (n may be 0)."""
    x = np.asarray(x, dtype=np.float32)
    rows, n = x.shape
    if n == 0:
        return np.zeros((rows, 0), np.uint8), np.zeros(rows, np.float32), np.zeros(rows, np.float32)
    lo = x.min(axis=1)
    hi = x.max(axis=1)
    scale = (hi - lo) / np.float32(255.0)
    codes = np.zeros((rows, n), np.uint8)
    for k in range(rows):
        if scale[k] > 0:
            q = np.rint((x[k] - lo[k]) / scale[k])           # float32 ops, round half to even
            codes[k] = np.clip(q, 0, 255).astype(np.uint8)
    return codes, scale.astype(np.float32), lo.astype(np.float32)


def dequantize_rows(codes: np.ndarray, scale: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Exact value of the quantised rows, float64 [rows][n]: scale * code + bias."""
    return (np.asarray(scale, np.float64)[:, None] * np.asarray(codes, np.float64)
            + np.asarray(bias, np.float64)[:, None])


def quantize_logical_blocks(blocks):
    """The logical blocks of ``oracle.attend_logical`` (per sequence a list of
    U [Hkv][T][r], W, Up [Hkv][T][r'], Wp, float64 holding bf16 values) with
    U and Up replaced by the exact values of their 8-bit quantisation, each
    row of U^T / U'^T (one rank component over the block's tokens) a group."""
    out = []
    for seq in blocks:
        qs = []
        for (U, W, Up, Wp) in seq:
            Uq = np.empty_like(U)
            Upq = np.empty_like(Up)
            for g in range(U.shape[0]):
                Uq[g] = dequantize_rows(*quantize_rows(U[g].T.astype(np.float32))).T
                Upq[g] = dequantize_rows(*quantize_rows(Up[g].T.astype(np.float32))).T
            qs.append((Uq, W, Upq, Wp))
        out.append(qs)
    return out


def attend_q8(wl, seq_index=None, sel=None):
    """Oracle output of a bf16 ``synth`` workload whose token factors are
    stored as 8-bit codes: attention over the dequantized factors, fp64."""
    import oracle
    q, blocks, kt, vt, tl = oracle.logical_from_workload(wl, seq_index)
    return oracle.attend_logical(q, quantize_logical_blocks(blocks), kt, vt, tl, wl.scale, sel)
