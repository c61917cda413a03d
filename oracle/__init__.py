"""fp64 CPU oracle for attention over a block-wise low-rank KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library: it consumes the logical per-block arrays
drawn by ``synth`` (token-major U, row-major W), never the packed pool.

The arithmetic lives in ``milo_oracle.c`` (reconstruct K = U W, V = U' W',
then plain two-pass softmax attention in double precision); this module only
builds that file and marshals arrays into it.  ``oracle.encode`` is the
encode step's oracle (per-block truncated SVD in numpy float64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "milo_oracle.c")
_LIB = os.path.join(_HERE, "libmilo_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Args(ctypes.Structure):
    _fields_ = [
        ("n_seq", ctypes.c_int32), ("q_len", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("q", ctypes.c_void_p), ("seq_blk", ctypes.c_void_p), ("blk_tok", ctypes.c_void_p),
        ("blk_rk", ctypes.c_void_p), ("blk_rv", ctypes.c_void_p), ("blk_base", ctypes.c_void_p),
        ("fac", ctypes.c_void_p),
        ("tail_cap", ctypes.c_int32),
        ("k_tail", ctypes.c_void_p), ("v_tail", ctypes.c_void_p), ("tail_len", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("sel", ctypes.c_void_p), ("n_sel", ctypes.c_int32),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = ctypes.CDLL(_LIB)
        _lib.milo_oracle_attend.argtypes = [ctypes.POINTER(_Args)]
        _lib.milo_oracle_attend.restype = ctypes.c_int
        _lib.milo_oracle_threads.restype = ctypes.c_int
    return _lib


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().milo_oracle_threads())


def _f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float64)


def attend_logical(q: np.ndarray, blocks, k_tail: np.ndarray, v_tail: np.ndarray,
                   tail_len: np.ndarray, scale: float,
                   sel: Optional[Sequence[Tuple[int, int, int]]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over logical fp64 inputs.

    q        [B][Q][Hq][d] float64
    blocks   per sequence a list of (U [Hkv][T][r], W [Hkv][r][d],
             Up [Hkv][T][r'], Wp [Hkv][r'][d]) float64 arrays
    k_tail, v_tail [B][Hkv][cap][d] float64; tail_len int [B]
    sel      optional (seq, q_pos, q_head) rows to compute; other rows are NaN
    Returns (out [B][Q][Hq][d], lse [B][Q][Hq]) float64.
    """
    lib = _load()
    q = np.ascontiguousarray(q, np.float64)
    B, Q, Hq, d = q.shape
    Hkv = k_tail.shape[1]
    seq_blk = np.zeros(B + 1, np.int64)
    tok, rk, rv, base, parts = [], [], [], [], []
    off = 0
    for i, bl in enumerate(blocks):
        seq_blk[i + 1] = seq_blk[i] + len(bl)
        for (U, W, Up, Wp) in bl:
            T, r, r2 = U.shape[1], U.shape[2], Up.shape[2]
            tok.append(T); rk.append(r); rv.append(r2); base.append(off)
            for g in range(Hkv):
                for x in (U[g], W[g], Up[g], Wp[g]):
                    parts.append(np.ascontiguousarray(x, np.float64).ravel())
                    off += x.size
    fac = np.concatenate(parts) if parts else np.zeros(1, np.float64)
    tok = np.array(tok or [0], np.int32)
    rk = np.array(rk or [0], np.int32)
    rv = np.array(rv or [0], np.int32)
    base = np.array(base or [0], np.int64)
    kt = np.ascontiguousarray(k_tail, np.float64)
    vt = np.ascontiguousarray(v_tail, np.float64)
    tl = np.ascontiguousarray(tail_len, np.int32)
    out = np.full((B, Q, Hq, d), np.nan)
    lse = np.full((B, Q, Hq), np.nan)
    sel_arr = None
    if sel is not None:
        sel_arr = np.ascontiguousarray(np.array(sel, np.int32).reshape(-1, 3))
    a = _Args(B, Q, Hq, Hkv, d, float(scale),
              q.ctypes.data, seq_blk.ctypes.data, tok.ctypes.data, rk.ctypes.data,
              rv.ctypes.data, base.ctypes.data, fac.ctypes.data,
              int(kt.shape[2]), kt.ctypes.data, vt.ctypes.data, tl.ctypes.data,
              out.ctypes.data, lse.ctypes.data,
              sel_arr.ctypes.data if sel_arr is not None else None,
              0 if sel_arr is None else int(sel_arr.shape[0]))
    rc = lib.milo_oracle_attend(ctypes.byref(a))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return out, lse


def logical_from_workload(wl, seq_index: Optional[Sequence[int]] = None):
    """fp64 logical arrays (token-major U) of a ``synth`` workload."""
    dt = wl.dtype
    idx = list(range(wl.batch)) if seq_index is None else list(seq_index)
    blocks = []
    for i in idx:
        bl = []
        for b in wl.blocks[i]:
            U = np.ascontiguousarray(np.swapaxes(_f64(b.ut, dt), 1, 2))
            Up = np.ascontiguousarray(np.swapaxes(_f64(b.upt, dt), 1, 2))
            bl.append((U, _f64(b.w, dt), Up, _f64(b.wp, dt)))
        blocks.append(bl)
    q = _f64(wl.q[idx], dt)
    kt = _f64(wl.k_tail[idx], dt)
    vt = _f64(wl.v_tail[idx], dt)
    return q, blocks, kt, vt, np.asarray(wl.tail_len)[idx]


def attend(wl, seq_index: Optional[Sequence[int]] = None,
           sel: Optional[Sequence[Tuple[int, int, int]]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Oracle output for a ``synth`` workload (optionally a subset of its
    sequences, given as indices into the workload's batch; ``sel`` indexes
    that subset)."""
    q, blocks, kt, vt, tl = logical_from_workload(wl, seq_index)
    return attend_logical(q, blocks, kt, vt, tl, wl.scale, sel)
