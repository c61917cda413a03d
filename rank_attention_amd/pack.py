"""Pack logical per-block factors into the device pool layout of milo_attn.h.

Pool layout (elements of the storage dtype):  for every block, its KV heads
back to back;  per head
    U^T [rank_k][ld_tok] | W [rank_k][d] | U'^T [rank_v][ld_tok] | W' [rank_v][d]
with ld_tok = n_tok rounded up to a multiple of 8 (plus ``ld_extra``).  Row
padding and the gaps between blocks hold NaN, so a kernel that reads them
produces NaN.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

BLOCK_DTYPE = np.dtype([("off", "<i8"), ("n_tok", "<i4"), ("ld_tok", "<i4"),
                        ("rank_k", "<i4"), ("rank_v", "<i4")])
assert BLOCK_DTYPE.itemsize == 24

NAN_BF16 = np.uint16(0x7FC0)


@dataclass
class PackedCache:
    dtype: str                 # "bf16" (uint16 bits) or "f32"
    head_dim: int
    n_kv_heads: int
    pool: np.ndarray           # 1-D, storage dtype
    blocks: np.ndarray         # BLOCK_DTYPE descriptors, CSR order
    seq_blocks: np.ndarray     # int32 [B+1]
    max_blocks: int
    q: np.ndarray              # [B][Q][Hq][d]
    k_tail: np.ndarray         # [B][Hkv][cap][d]
    v_tail: np.ndarray
    tail_len: np.ndarray       # int32 [B]
    unit_order: Optional[np.ndarray] = None   # int32 decode schedule (largest first)


def _nan(dtype: str):
    return NAN_BF16 if dtype == "bf16" else np.float32(np.nan)


def pack(wl, gap: int = 8, shuffle_pool: Optional[int] = None,
         max_blocks: Optional[int] = None, poison_tail: bool = True,
         plan: bool = True, ld_extra: int = 0) -> PackedCache:
    """Pack a ``synth`` workload.

    gap           NaN elements left between consecutive blocks (multiple of 8)
    shuffle_pool  seed: place blocks in the pool in a random order (the CSR
                  order is unchanged), to exercise arbitrary offsets
    max_blocks    host bound for the grid (default: the largest count)
    plan          compute the largest-first decode schedule (unit_order)
    ld_extra      extra NaN padding per U^T / U'^T row beyond n_tok rounded up
                  to 8 (multiple of 8): whole padding chunks past the block end
    """
    assert gap % 8 == 0 and ld_extra % 8 == 0 and ld_extra >= 0
    d, hkv = wl.cfg.head_dim, wl.cfg.n_kv_heads
    st = np.uint16 if wl.dtype == "bf16" else np.float32
    flat = [b for s in wl.blocks for b in s]
    sizes = []
    for b in flat:
        ld = (b.n_tok + 7) // 8 * 8 + ld_extra
        sizes.append(hkv * (b.rank_k + b.rank_v) * (ld + d))
    order = np.arange(len(flat))
    if shuffle_pool is not None:
        order = np.random.default_rng(shuffle_pool).permutation(len(flat))
    offs = np.zeros(len(flat), np.int64)
    pos = gap
    for k in order:
        offs[k] = pos
        pos += sizes[k] + gap
    pool = np.full(max(pos, 8), _nan(wl.dtype), dtype=st)
    desc = np.zeros(len(flat), BLOCK_DTYPE)
    for k, b in enumerate(flat):
        ld = (b.n_tok + 7) // 8 * 8 + ld_extra
        desc[k] = (offs[k], b.n_tok, ld, b.rank_k, b.rank_v)
        head = (b.rank_k + b.rank_v) * (ld + d)
        for g in range(hkv):
            base = offs[k] + g * head
            o = base
            if b.rank_k:
                pool[o:o + b.rank_k * ld].reshape(b.rank_k, ld)[:, :b.n_tok] = b.ut[g]
            o += b.rank_k * ld
            pool[o:o + b.rank_k * d] = b.w[g].ravel()
            o += b.rank_k * d
            if b.rank_v:
                pool[o:o + b.rank_v * ld].reshape(b.rank_v, ld)[:, :b.n_tok] = b.upt[g]
            o += b.rank_v * ld
            pool[o:o + b.rank_v * d] = b.wp[g].ravel()
    counts = [len(s) for s in wl.blocks]
    seq_blocks = np.zeros(len(counts) + 1, np.int32)
    seq_blocks[1:] = np.cumsum(counts)
    kt = np.array(wl.k_tail, copy=True)
    vt = np.array(wl.v_tail, copy=True)
    if poison_tail:
        for i, L in enumerate(wl.tail_len):
            kt[i, :, L:] = _nan(wl.dtype)
            vt[i, :, L:] = _nan(wl.dtype)
    mb = max(counts) if counts else 0
    if max_blocks is not None:
        assert max_blocks >= mb
        mb = max_blocks
    tl = np.asarray(wl.tail_len, np.int32)
    order = plan_decode(desc, seq_blocks, tl if kt.shape[2] > 0 else None, hkv, mb, d) if plan else None
    return PackedCache(dtype=wl.dtype, head_dim=d, n_kv_heads=hkv, pool=pool, blocks=desc,
                       seq_blocks=seq_blocks, max_blocks=mb, q=np.ascontiguousarray(wl.q),
                       k_tail=kt, v_tail=vt, tail_len=tl, unit_order=order)


def plan_decode(blocks: np.ndarray, seq_blocks: np.ndarray, tail_len, n_kv_heads: int,
                max_blocks: int, head_dim: int) -> np.ndarray:
    """Largest-first decode schedule from the library's host-side planner."""
    import ctypes
    from . import _lib
    lib = _lib.load()
    B = len(seq_blocks) - 1
    out = np.empty(B * n_kv_heads * (max_blocks + 1), np.int32)
    blocks = np.ascontiguousarray(blocks)
    sb = np.ascontiguousarray(seq_blocks, np.int32)
    tl = None if tail_len is None else np.ascontiguousarray(tail_len, np.int32)
    rc = lib.milo_attn_plan_decode(blocks.ctypes.data if len(blocks) else None, len(blocks), sb.ctypes.data,
                                   None if tl is None else tl.ctypes.data, B, n_kv_heads,
                                   max_blocks, head_dim, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"milo_attn_plan_decode failed ({rc})")
    return out
