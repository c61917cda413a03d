"""CPU oracle of KIVI-style low-bit quantisation of the token factors.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

MILO (summary at paperlayer.ai/abs/2609.29913v1, "5.3 Performance Analysis")
combines its low-rank cache with KIVI quantisation.  KIVI quantises keys per
channel (a group is one channel over a run of consecutive tokens) and values
per token (a group is a run of consecutive channels of one token), both
asymmetric, with 2- or 4-bit codes and a scale and a bias per group kept in
fp16.  The pages give no more; the reading here applies that grouping to the
token factors of every block and KV head (W and W' are not quantised):

  keys   U  (T x r):   group = rank component k over tokens 64j .. 64j+63
                       (the last group of a block may be shorter);
  values U' (T x r'):  group = token t over rank components 32j .. 32j+31
                       (the last group may be narrower).

Per group, with L = 2^bits - 1 levels:
    lo = min x,  hi = max x                           (fp32)
    a = fp16((hi - lo) / L),  b = fp16(lo)            (stored scale and bias)
    code = clamp(round_half_even((x - b) / a), 0, L)  (fp32; 0 where a is 0)
    x ~= a * code + b                                 (exact dequantised value)
The codes are integers decided by floating point: every step above is a
correctly rounded fp32 operation on the stored fp16 a and b, the precision
the kernel uses, so both sides reach the same codes.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

KEY_GROUP_TOKENS = 64
VALUE_GROUP_RANKS = 32


def levels(bits: int) -> int:
    if bits not in (2, 4):
        raise ValueError("KIVI-style codes have 2 or 4 bits")
    return (1 << bits) - 1


def quantize_groups(x: np.ndarray, bits: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantise each row of x [groups][n] (float32) as one group.  Returns
    codes uint8 [groups][n], scale float16 [groups], bias float16 [groups]."""
    L = np.float32(levels(bits))
    x = np.asarray(x, dtype=np.float32)
    g, n = x.shape
    codes = np.zeros((g, n), np.uint8)
    if n == 0:
        return codes, np.zeros(g, np.float16), np.zeros(g, np.float16)
    lo = x.min(axis=1)
    hi = x.max(axis=1)
    a16 = ((hi - lo) / L).astype(np.float16)
    b16 = lo.astype(np.float16)
    a = a16.astype(np.float32)
    b = b16.astype(np.float32)
    ok = a > 0
    # float32 ops, round half to even; groups with a = 0 keep code 0
    q = np.rint((x - b[:, None]) / np.where(ok, a, np.float32(1))[:, None])
    codes = np.where(ok[:, None], np.clip(q, 0, L), 0).astype(np.uint8)
    return codes, a16, b16


def dequantize_groups(codes: np.ndarray, scale: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Exact value of quantised groups, float64 [groups][n]: scale * code + bias."""
    return (np.asarray(scale, np.float64)[:, None] * np.asarray(codes, np.float64)
            + np.asarray(bias, np.float64)[:, None])


def quantize_keys(U: np.ndarray, bits: int):
    """Key token factor U [T][r]: per rank component, groups of 64 tokens.
    Returns codes uint8 [T][r], scale and bias float16 [ceil(T/64)][r]."""
    U = np.asarray(U, np.float32)
    T, r = U.shape
    ng = -(-T // KEY_GROUP_TOKENS)
    codes = np.zeros((T, r), np.uint8)
    sc = np.zeros((ng, r), np.float16)
    bi = np.zeros((ng, r), np.float16)
    for j in range(ng):
        t0, t1 = j * KEY_GROUP_TOKENS, min(T, (j + 1) * KEY_GROUP_TOKENS)
        c, a, b = quantize_groups(U[t0:t1].T, bits)      # one group per rank component
        codes[t0:t1] = c.T
        sc[j], bi[j] = a, b
    return codes, sc, bi


def dequantize_keys(codes, sc, bi) -> np.ndarray:
    T, r = codes.shape
    out = np.zeros((T, r), np.float64)
    for j in range(sc.shape[0]):
        t0, t1 = j * KEY_GROUP_TOKENS, min(T, (j + 1) * KEY_GROUP_TOKENS)
        out[t0:t1] = dequantize_groups(codes[t0:t1].T, sc[j], bi[j]).T
    return out


def quantize_values(Up: np.ndarray, bits: int):
    """Value token factor U' [T][r']: per token, groups of 32 rank
    components.  Returns codes uint8 [T][r'], scale and bias float16
    [T][ceil(r'/32)]."""
    Up = np.asarray(Up, np.float32)
    T, rv = Up.shape
    ng = -(-rv // VALUE_GROUP_RANKS)
    codes = np.zeros((T, rv), np.uint8)
    sc = np.zeros((T, ng), np.float16)
    bi = np.zeros((T, ng), np.float16)
    for j in range(ng):
        k0, k1 = j * VALUE_GROUP_RANKS, min(rv, (j + 1) * VALUE_GROUP_RANKS)
        c, a, b = quantize_groups(Up[:, k0:k1], bits)    # one group per token
        codes[:, k0:k1] = c
        sc[:, j], bi[:, j] = a, b
    return codes, sc, bi


def dequantize_values(codes, sc, bi) -> np.ndarray:
    T, rv = codes.shape
    out = np.zeros((T, rv), np.float64)
    for j in range(sc.shape[1]):
        k0, k1 = j * VALUE_GROUP_RANKS, min(rv, (j + 1) * VALUE_GROUP_RANKS)
        out[:, k0:k1] = dequantize_groups(codes[:, k0:k1], sc[:, j], bi[:, j])
    return out


def quantize_logical_blocks(blocks, bits: int):
    """The logical blocks of ``oracle.attend_logical`` (per sequence a list of
    U [Hkv][T][r], W, Up [Hkv][T][r'], Wp, float64 holding bf16 values) with
    U and Up replaced by the exact values of their KIVI-style quantisation."""
    out = []
    for seq in blocks:
        qs = []
        for (U, W, Up, Wp) in seq:
            Uq = np.empty_like(U)
            Upq = np.empty_like(Up)
            for g in range(U.shape[0]):
                Uq[g] = dequantize_keys(*quantize_keys(U[g], bits))
                Upq[g] = dequantize_values(*quantize_values(Up[g], bits))
            qs.append((Uq, W, Upq, Wp))
        out.append(qs)
    return out


def attend_kivi(wl, bits: int, seq_index=None, sel=None):
    """Oracle output of a bf16 ``synth`` workload whose token factors are
    stored as KIVI-style codes: attention over the dequantized factors, fp64."""
    import oracle
    q, blocks, kt, vt, tl = oracle.logical_from_workload(wl, seq_index)
    return oracle.attend_logical(q, quantize_logical_blocks(blocks, bits), kt, vt, tl, wl.scale, sel)
