"""Attention over a block-wise low-rank compressed KV cache on MI355X.

Thin Python binding of the C ABI in include/milo_attn.h.  Every step of the
attention runs in the HIP kernels of ``libmilo_attn.so``; this module only
marshals torch tensors (device memory and the current stream) into the C
call.  If the library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import numpy as np

from . import _lib
from ._lib import (MILO_BF16, MILO_BF16_KV2, MILO_BF16_KV4, MILO_BF16_Q8, MILO_F32, MILO_PATH_CHUNK, MILO_PATH_DECODE, MILO_PATH_SHARED, MiloAttnArgs,
                   MILO_OK, MILO_ERR_DEVICE)
from .pack import BLOCK_DTYPE, PackedCache, pack  # noqa: F401

__all__ = ["decode", "decode_noalloc", "chunk", "decode_shared", "validate_tables", "workspace_bytes", "abi_version", "status_str", "DeviceCache",
           "pack", "PackedCache", "MiloError", "library_path"]

library_path = _lib.LIB_PATH


class MiloError(ValueError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"milo_attn status {code}: {msg}")
        self.code = code


def abi_version() -> int:
    return int(_lib.load().milo_abi_version())


def status_str(code: int) -> str:
    return _lib.load().milo_status_str(int(code)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype in (torch.int16, torch.bfloat16) or str(t.dtype) == "torch.uint16":
        return MILO_BF16
    if t.dtype == torch.float32:
        return MILO_F32
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def _uint8():
    import torch
    return torch.uint8


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def make_args(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, *, n_kv_heads: int,
              scale: float, max_blocks: int, out=None, lse=None, workspace=None,
              workspace_bytes: Optional[int] = None, prof_events=(None, None),
              unit_order=None, storage: Optional[int] = None) -> MiloAttnArgs:
    """Fill the C argument struct from device tensors (no checks: the library
    checks).  ``storage`` sets the dtype code of the pool (a byte pool is
    8-bit storage unless it says otherwise)."""
    B, Q, Hq, d = (int(x) for x in q.shape)
    cap = 0 if k_tail is None else int(k_tail.shape[2])
    a = MiloAttnArgs()
    a.struct_size = ctypes.sizeof(MiloAttnArgs)
    a.dtype = _dtype_code(q)
    if pool is not None and a.dtype == MILO_BF16 and pool.dtype == _uint8():
        a.dtype = MILO_BF16_Q8   # 8-bit token factors (milo_quantize_factors)
    if storage is not None:
        a.dtype = int(storage)
    a.batch, a.q_len, a.n_q_heads, a.n_kv_heads, a.head_dim = B, Q, Hq, int(n_kv_heads), d
    a.scale = float(scale)
    a.q, a.pool, a.blocks, a.seq_blocks = _ptr(q), _ptr(pool), _ptr(blocks), _ptr(seq_blocks)
    a.max_blocks_per_seq = int(max_blocks)
    a.tail_cap = cap
    a.k_tail, a.v_tail, a.tail_len = _ptr(k_tail), _ptr(v_tail), _ptr(tail_len)
    a.out, a.lse, a.workspace = _ptr(out), _ptr(lse), _ptr(workspace)
    a.workspace_bytes = int(workspace_bytes if workspace_bytes is not None else
                            (0 if workspace is None else workspace.numel() * workspace.element_size()))
    a.prof_events[0] = prof_events[0]
    a.prof_events[1] = prof_events[1]
    a.unit_order = _ptr(unit_order)
    return a


def workspace_bytes(args: MiloAttnArgs, path: int) -> int:
    return int(_lib.load().milo_attn_workspace_bytes(ctypes.byref(args), int(path)))


def _run(path: int, q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, *, n_kv_heads, scale,
         max_blocks, out=None, lse=None, workspace=None, stream=None, prof_events=(None, None),
         unit_order=None, want_lse=True, storage=None) -> Tuple[object, object]:
    import torch
    lib = _lib.load()
    B, Q, Hq, d = (int(x) for x in q.shape)
    dev = q.device
    if out is None:
        out = torch.empty((B, Q, Hq, d), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Q, Hq), dtype=torch.float32, device=dev)
    a = make_args(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, n_kv_heads=n_kv_heads,
                  scale=scale, max_blocks=max_blocks, out=out, lse=lse, workspace=workspace,
                  prof_events=prof_events, unit_order=unit_order, storage=storage)
    fn = {MILO_PATH_DECODE: lib.milo_attn_decode, MILO_PATH_CHUNK: lib.milo_attn_chunk,
          MILO_PATH_SHARED: lib.milo_attn_decode_shared}[path]
    if workspace is None:
        need = lib.milo_attn_workspace_bytes(ctypes.byref(a), path)
        if need == 0:
            rc = fn(ctypes.byref(a), None)
            raise MiloError(rc, status_str(rc))
        workspace = torch.empty(int(need), dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), int(need)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = fn(ctypes.byref(a), ctypes.c_void_p(int(stream)))
    if rc != MILO_OK:
        if rc == MILO_ERR_DEVICE:
            raise RuntimeError(f"milo_attn: {status_str(rc)}")
        raise MiloError(rc, status_str(rc))
    return out, lse


def decode(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, *, n_kv_heads: int, scale: float,
           max_blocks: int, **kw):
    """Decode attention (q_len = 1).  Returns (out fp32 [B][1][Hq][d], lse [B][1][Hq])."""
    return _run(MILO_PATH_DECODE, q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len,
                n_kv_heads=n_kv_heads, scale=scale, max_blocks=max_blocks, **kw)


def decode_noalloc(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, *, n_kv_heads: int, scale: float,
                   max_blocks: int, out=None, lse=None, stream=None, unit_order=None, storage=None):
    """Decode (q_len = 1) through milo_attn_decode_noalloc: the library keeps
    the partials in its own static device buffer, so no workspace is passed.
    out and lse may be preallocated (then nothing is allocated here either)."""
    import torch
    lib = _lib.load()
    B, Q, Hq, d = (int(x) for x in q.shape)
    if out is None:
        out = torch.empty((B, Q, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Q, Hq), dtype=torch.float32, device=q.device)
    a = make_args(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, n_kv_heads=n_kv_heads,
                  scale=scale, max_blocks=max_blocks, out=out, lse=lse, unit_order=unit_order, storage=storage)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.milo_attn_decode_noalloc(ctypes.byref(a), ctypes.c_void_p(int(stream)))
    if rc != MILO_OK:
        if rc == MILO_ERR_DEVICE:
            raise RuntimeError(f"milo_attn: {status_str(rc)}")
        raise MiloError(rc, status_str(rc))
    return out, lse


def chunk(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, *, n_kv_heads: int, scale: float,
          max_blocks: int, **kw):
    """Chunked-query attention (q_len = Q, bottom-right causal over the tail)."""
    return _run(MILO_PATH_CHUNK, q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len,
                n_kv_heads=n_kv_heads, scale=scale, max_blocks=max_blocks, **kw)


def decode_shared(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, *, n_kv_heads: int,
                  scale: float, max_blocks: int, **kw):
    """Decode (q_len = 1) with the blocks of sequence 0 shared by every
    sequence; each sequence keeps its own tail.  Same result layout as decode."""
    kw.pop("unit_order", None)
    return _run(MILO_PATH_SHARED, q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len,
                n_kv_heads=n_kv_heads, scale=scale, max_blocks=max_blocks, **kw)


def validate_tables(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, *, n_kv_heads: int,
                    max_blocks: int, path: int = MILO_PATH_DECODE, scale: float = 1.0, unit_order=None,
                    storage=None):
    """Check the device tables against the contract (milo_attn_validate) and
    wait for the result: None if every rule holds, else (rule name, index).
    With a decode schedule (unit_order) it is checked too, using a scratch
    workspace of 4 bytes per unit."""
    import torch
    lib = _lib.load()
    status = torch.empty(1, dtype=torch.int64, device=q.device)
    workspace = None
    if unit_order is not None:
        workspace = torch.empty(max(4 * int(unit_order.numel()), 256), dtype=torch.uint8, device=q.device)
    a = make_args(q, pool, blocks, seq_blocks, k_tail, v_tail, tail_len, n_kv_heads=n_kv_heads, scale=scale,
                  max_blocks=max_blocks, workspace=workspace, unit_order=unit_order, storage=storage)
    n_desc = int(blocks.numel() * blocks.element_size()) // BLOCK_DTYPE.itemsize
    pool_elems = int(pool.numel()) if pool is not None else 0
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.milo_attn_validate(ctypes.byref(a), int(path), n_desc, pool_elems, status.data_ptr(),
                                ctypes.c_void_p(int(stream)))
    if rc != MILO_OK:
        raise MiloError(rc, status_str(rc))
    torch.cuda.synchronize(q.device)
    v = int(status.cpu().numpy().view(np.uint64)[0])
    if v == 0xFFFFFFFFFFFFFFFF:
        return None
    return _lib.TABLE_RULES.get(v >> 32, str(v >> 32)), int(v & 0xFFFFFFFF)


class DeviceCache:
    """A packed cache and its query moved to device memory (torch tensors)."""

    def __init__(self, packed: PackedCache, device="cuda", scale: Optional[float] = None):
        import torch

        def dev(a, raw16=False):
            a = np.ascontiguousarray(a)
            if raw16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)

        bf = packed.dtype == "bf16"
        self.packed = packed
        self.n_kv_heads = packed.n_kv_heads
        self.max_blocks = packed.max_blocks
        self.scale = scale if scale is not None else 1.0 / float(packed.head_dim) ** 0.5
        self.pool = dev(packed.pool, bf)
        self.blocks = dev(packed.blocks.view(np.uint8))
        self.seq_blocks = dev(packed.seq_blocks)
        self.q = dev(packed.q, bf)
        cap = packed.k_tail.shape[2]
        self.k_tail = dev(packed.k_tail, bf) if cap > 0 else None
        self.v_tail = dev(packed.v_tail, bf) if cap > 0 else None
        self.tail_len = dev(packed.tail_len) if cap > 0 else None
        self.unit_order = dev(packed.unit_order) if packed.unit_order is not None else None
        self.storage = None     # pool dtype code when not inferred from the tensors

    def tensors(self):
        return (self.q, self.pool, self.blocks, self.seq_blocks, self.k_tail, self.v_tail,
                self.tail_len)

    def decode(self, **kw):
        kw.setdefault("scale", self.scale)
        kw.setdefault("unit_order", self.unit_order)
        kw.setdefault("storage", self.storage)
        return decode(*self.tensors(), n_kv_heads=self.n_kv_heads, max_blocks=self.max_blocks, **kw)

    def decode_noalloc(self, **kw):
        kw.setdefault("scale", self.scale)
        kw.setdefault("unit_order", self.unit_order)
        kw.setdefault("storage", self.storage)
        return decode_noalloc(*self.tensors(), n_kv_heads=self.n_kv_heads, max_blocks=self.max_blocks, **kw)

    def chunk(self, **kw):
        kw.setdefault("scale", self.scale)
        return chunk(*self.tensors(), n_kv_heads=self.n_kv_heads, max_blocks=self.max_blocks, **kw)

    def validate(self, path: int = MILO_PATH_DECODE):
        order = self.unit_order if path == MILO_PATH_DECODE else None
        return validate_tables(*self.tensors(), n_kv_heads=self.n_kv_heads, max_blocks=self.max_blocks, path=path,
                               unit_order=order, storage=self.storage)

    def decode_shared(self, **kw):
        kw.setdefault("scale", self.scale)
        return decode_shared(*self.tensors(), n_kv_heads=self.n_kv_heads, max_blocks=self.max_blocks, **kw)

    def quantized(self, stream=None) -> "DeviceCache":
        """The same cache with 8-bit token factors (milo_quantize_factors on
        this cache's bf16 pool): decode reads it as MILO_BF16_Q8 storage.
        q, the tails and the decode schedule are shared with this cache."""
        import copy
        import torch
        from .encode import quantize
        if self.packed.dtype != "bf16" or self.pool.dtype == torch.uint8:
            raise ValueError("8-bit factors are made from bf16 storage")
        qc = copy.copy(self)
        qc.pool, qc.blocks, qc.blocks_host = quantize(self.pool, self.blocks, self.packed.blocks,
                                                      self.n_kv_heads, self.packed.head_dim, stream=stream)
        return qc

    def kivi(self, bits: int = 4, stream=None) -> "DeviceCache":
        """The same cache with KIVI-style token factors of the given width
        (milo_quantize_kivi on this cache's bf16 pool): decode reads it as
        MILO_BF16_KV4 or MILO_BF16_KV2 storage.  q, the tails and the decode
        schedule are shared with this cache."""
        import copy
        import torch
        from .encode import quantize_kivi
        if self.packed.dtype != "bf16" or self.pool.dtype == torch.uint8:
            raise ValueError("KIVI-style factors are made from bf16 storage")
        qc = copy.copy(self)
        qc.pool, qc.blocks, qc.blocks_host = quantize_kivi(self.pool, self.blocks, self.packed.blocks,
                                                           self.n_kv_heads, self.packed.head_dim, bits,
                                                           stream=stream)
        qc.storage = MILO_BF16_KV4 if bits == 4 else MILO_BF16_KV2
        return qc
