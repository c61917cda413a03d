"""Binding of the encode step (include/milo_encode.h): dense keys and values
of a context to per-block low-rank factors in a pool that the attention
entry points read.  Argument marshalling only: the spectra and the factors
are computed by the HIP kernels of ``libmilo_attn.so``."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import MILO_BF16, MILO_F32, MILO_OK, MILO_ERR_DEVICE, MiloEncodeArgs, MiloQuantArgs, MiloRankArgs
from .pack import BLOCK_DTYPE


def layout(n_tok: Sequence[int], rank_k: Sequence[int], rank_v: Sequence[int], n_kv_heads: int,
           head_dim: int) -> Tuple[np.ndarray, int]:
    """Descriptors (BLOCK_DTYPE) and pool size in elements for blocks of the
    given sizes and ranks, placed back to back (milo_encode_layout)."""
    from . import MiloError, status_str
    nt = np.ascontiguousarray(n_tok, np.int32)
    rk = np.ascontiguousarray(rank_k, np.int32)
    rv = np.ascontiguousarray(rank_v, np.int32)
    nb = len(nt)
    if len(rk) != nb or len(rv) != nb:
        raise ValueError("n_tok, rank_k and rank_v must have one entry per block")
    blocks = np.zeros(nb, BLOCK_DTYPE)
    elems = ctypes.c_int64(0)
    rc = _lib.load().milo_encode_layout(nt.ctypes.data, rk.ctypes.data, rv.ctypes.data, nb, int(n_kv_heads),
                                        int(head_dim), blocks.ctypes.data, ctypes.byref(elems))
    if rc != MILO_OK:
        raise MiloError(rc, status_str(rc))
    return blocks, int(elems.value)


def quant_layout(src_blocks: np.ndarray, n_kv_heads: int, head_dim: int) -> Tuple[np.ndarray, int]:
    """Descriptors (BLOCK_DTYPE) and size in bytes of the 8-bit pool for the
    blocks of a bf16 pool (milo_quant_layout)."""
    from . import MiloError, status_str
    src = np.ascontiguousarray(src_blocks, BLOCK_DTYPE)
    out = np.zeros(len(src), BLOCK_DTYPE)
    nbytes = ctypes.c_int64(0)
    rc = _lib.load().milo_quant_layout(src.ctypes.data if len(src) else None, len(src), int(n_kv_heads),
                                       int(head_dim), out.ctypes.data if len(src) else None, ctypes.byref(nbytes))
    if rc != MILO_OK:
        raise MiloError(rc, status_str(rc))
    return out, int(nbytes.value)


def quantize(pool, blocks_dev, blocks_host: np.ndarray, n_kv_heads: int, head_dim: int, stream=None):
    """8-bit token factors of a bf16 pool (milo_quantize_factors).  Returns
    (pool uint8 tensor, descriptors on the device, descriptors on the host);
    milo_attn_decode reads the result as MILO_BF16_Q8 storage."""
    import torch
    from . import MiloError, status_str
    lib = _lib.load()
    blocks, nbytes = quant_layout(blocks_host, n_kv_heads, head_dim)
    dev = pool.device
    qpool = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    qdev = torch.from_numpy(blocks.view(np.uint8).copy()).to(dev)
    a = MiloQuantArgs()
    a.struct_size = ctypes.sizeof(MiloQuantArgs)
    a.n_blocks, a.n_kv_heads, a.head_dim = len(blocks), int(n_kv_heads), int(head_dim)
    a.src_pool, a.src_blocks = pool.data_ptr(), blocks_dev.data_ptr()
    a.dst_pool, a.dst_blocks = qpool.data_ptr(), qdev.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.milo_quantize_factors(ctypes.byref(a), ctypes.c_void_p(int(stream)))
    if rc != MILO_OK:
        if rc == MILO_ERR_DEVICE:
            raise RuntimeError(f"milo_quantize_factors: {status_str(rc)}")
        raise MiloError(rc, status_str(rc))
    return qpool, qdev, blocks


def kivi_layout(src_blocks: np.ndarray, n_kv_heads: int, head_dim: int, bits: int) -> Tuple[np.ndarray, int]:
    """Descriptors (BLOCK_DTYPE) and size in bytes of the KIVI-style pool
    (bits 4 or 2) for the blocks of a bf16 pool (milo_kivi_layout)."""
    from . import MiloError, status_str
    src = np.ascontiguousarray(src_blocks, BLOCK_DTYPE)
    out = np.zeros(len(src), BLOCK_DTYPE)
    nbytes = ctypes.c_int64(0)
    rc = _lib.load().milo_kivi_layout(src.ctypes.data if len(src) else None, len(src), int(n_kv_heads),
                                      int(head_dim), int(bits), out.ctypes.data if len(src) else None,
                                      ctypes.byref(nbytes))
    if rc != MILO_OK:
        raise MiloError(rc, status_str(rc))
    return out, int(nbytes.value)


def quantize_kivi(pool, blocks_dev, blocks_host: np.ndarray, n_kv_heads: int, head_dim: int, bits: int,
                  stream=None):
    """KIVI-style token factors of a bf16 pool (milo_quantize_kivi).  Returns
    (pool uint8 tensor, descriptors on the device, descriptors on the host);
    milo_attn_decode reads the result as MILO_BF16_KV4 / MILO_BF16_KV2 storage."""
    import torch
    from . import MiloError, status_str
    lib = _lib.load()
    blocks, nbytes = kivi_layout(blocks_host, n_kv_heads, head_dim, bits)
    dev = pool.device
    qpool = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    qdev = torch.from_numpy(blocks.view(np.uint8).copy()).to(dev)
    a = MiloQuantArgs()
    a.struct_size = ctypes.sizeof(MiloQuantArgs)
    a.n_blocks, a.n_kv_heads, a.head_dim = len(blocks), int(n_kv_heads), int(head_dim)
    a.src_pool, a.src_blocks = pool.data_ptr(), blocks_dev.data_ptr()
    a.dst_pool, a.dst_blocks = qpool.data_ptr(), qdev.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.milo_quantize_kivi(ctypes.byref(a), int(bits), ctypes.c_void_p(int(stream)))
    if rc != MILO_OK:
        if rc == MILO_ERR_DEVICE:
            raise RuntimeError(f"milo_quantize_kivi: {status_str(rc)}")
        raise MiloError(rc, status_str(rc))
    return qpool, qdev, blocks


def allocate_ranks(sigma, budget_k: int, budget_v: int, r_min: int, unit: int = 1, stream=None):
    """Entropy-driven ranks (milo_rank_allocate) from device spectra sigma
    [n_blocks][Hkv][2][d] (fp32, descending per head).  Returns (ranks int32
    [n_blocks][2], entropy fp32 [n_blocks][2]) on the device."""
    import torch
    from . import MiloError, status_str
    nb, h, two, d = (int(x) for x in sigma.shape)
    if two != 2 or sigma.dtype != torch.float32:
        raise ValueError("sigma must be float32 [n_blocks][n_kv_heads][2][head_dim]")
    lib = _lib.load()
    ranks = torch.empty((nb, 2), dtype=torch.int32, device=sigma.device)
    ent = torch.empty((nb, 2), dtype=torch.float32, device=sigma.device)
    a = MiloRankArgs()
    a.struct_size = ctypes.sizeof(MiloRankArgs)
    a.n_blocks, a.n_kv_heads, a.head_dim = nb, h, d
    a.budget_k, a.budget_v, a.r_min, a.unit = int(budget_k), int(budget_v), int(r_min), int(unit)
    a.sigma, a.ranks, a.entropy = sigma.data_ptr(), ranks.data_ptr(), ent.data_ptr()
    need = lib.milo_rank_workspace_bytes(ctypes.byref(a))
    if need == 0:
        rc = lib.milo_rank_allocate(ctypes.byref(a), None)
        raise MiloError(rc, status_str(rc))
    ws = torch.empty(int(need), dtype=torch.uint8, device=sigma.device)
    a.workspace, a.workspace_bytes = ws.data_ptr(), int(need)
    if stream is None:
        stream = torch.cuda.current_stream(sigma.device).cuda_stream
    rc = lib.milo_rank_allocate(ctypes.byref(a), ctypes.c_void_p(int(stream)))
    if rc != MILO_OK:
        if rc == MILO_ERR_DEVICE:
            raise RuntimeError(f"milo_rank_allocate: {status_str(rc)}")
        raise MiloError(rc, status_str(rc))
    return ranks, ent


class DeviceContext:
    """Dense keys and values of one context ([Hkv][N][d], stored dtype: bf16
    bit patterns as uint16, or float32) in device memory, split into blocks
    at tok_start / n_tok, with the two encode calls on them."""

    def __init__(self, k: np.ndarray, v: np.ndarray, tok_start, n_tok, dtype: str = "bf16",
                 device="cuda"):
        import torch

        def dev(a, raw16=False):
            a = np.ascontiguousarray(a)
            if raw16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)

        if k.shape != v.shape or k.ndim != 3:
            raise ValueError("k and v must both be [n_kv_heads][n_tokens][head_dim]")
        self.dtype = dtype
        self.code = MILO_BF16 if dtype == "bf16" else MILO_F32
        self.n_kv_heads, self.n_tokens, self.head_dim = (int(x) for x in k.shape)
        self.k = dev(k, dtype == "bf16")
        self.v = dev(v, dtype == "bf16")
        self.n_tok = np.ascontiguousarray(n_tok, np.int32)
        self.tok_start = dev(np.ascontiguousarray(tok_start, np.int64))
        self.n_blocks = len(self.n_tok)
        self.device = device
        self.workspace = None
        self._spectrum_blocks = None

    def _args(self, blocks_dev, pool=None, sigma=None, iters=None) -> MiloEncodeArgs:
        a = MiloEncodeArgs()
        a.struct_size = ctypes.sizeof(MiloEncodeArgs)
        a.dtype = self.code
        a.n_blocks, a.n_kv_heads, a.head_dim, a.n_tokens = (self.n_blocks, self.n_kv_heads, self.head_dim,
                                                            self.n_tokens)
        a.k, a.v = self.k.data_ptr(), self.v.data_ptr()
        a.tok_start = self.tok_start.data_ptr()
        a.blocks = blocks_dev.data_ptr()
        a.sigma = None if sigma is None else sigma.data_ptr()
        a.iters = None if iters is None else iters.data_ptr()
        a.pool = None if pool is None else pool.data_ptr()
        if self.workspace is not None:
            a.workspace, a.workspace_bytes = self.workspace.data_ptr(), self.workspace.numel()
        return a

    def _call(self, fn, a, stream):
        import torch
        from . import MiloError, status_str
        if stream is None:
            stream = torch.cuda.current_stream(self.k.device).cuda_stream
        rc = fn(ctypes.byref(a), ctypes.c_void_p(int(stream)))
        if rc != MILO_OK:
            if rc == MILO_ERR_DEVICE:
                raise RuntimeError(f"milo_encode: {status_str(rc)}")
            raise MiloError(rc, status_str(rc))

    def spectrum(self, stream=None):
        """Singular values [n_blocks][Hkv][2][d] (fp32, descending; K then V)
        and QL iteration counts [n_blocks][Hkv][2]; keeps the singular
        vectors in this context's workspace for factors()."""
        import torch
        lib = _lib.load()
        blocks, _ = layout(self.n_tok, np.zeros(self.n_blocks, np.int32), np.zeros(self.n_blocks, np.int32),
                           self.n_kv_heads, self.head_dim)
        self._spectrum_blocks = torch.from_numpy(blocks.view(np.uint8)).to(self.device)
        sigma = torch.empty((self.n_blocks, self.n_kv_heads, 2, self.head_dim), dtype=torch.float32,
                            device=self.device)
        iters = torch.empty((self.n_blocks, self.n_kv_heads, 2), dtype=torch.int32, device=self.device)
        a = self._args(self._spectrum_blocks, sigma=sigma, iters=iters)
        need = lib.milo_encode_workspace_bytes(ctypes.byref(a))
        if need and (self.workspace is None or self.workspace.numel() < need):
            self.workspace = torch.empty(int(need), dtype=torch.uint8, device=self.device)
        a = self._args(self._spectrum_blocks, sigma=sigma, iters=iters)
        self._call(lib.milo_encode_spectrum, a, stream)
        return sigma, iters

    def factors(self, rank_k, rank_v, stream=None):
        """Factors at the given per-block ranks (after spectrum()): returns
        (pool, blocks_dev, blocks_host) where pool is in the stored dtype
        (int16 views of bf16) and the descriptors follow include/milo_attn.h."""
        import torch
        if self.workspace is None and self.n_blocks:
            raise RuntimeError("factors() needs the singular vectors of a spectrum() call")
        lib = _lib.load()
        blocks, elems = layout(self.n_tok, rank_k, rank_v, self.n_kv_heads, self.head_dim)
        bdev = torch.from_numpy(blocks.view(np.uint8).copy()).to(self.device)
        tdt = torch.int16 if self.dtype == "bf16" else torch.float32
        pool = torch.empty(max(elems, 8), dtype=tdt, device=self.device)
        self._call(lib.milo_encode_factors, self._args(bdev, pool=pool), stream)
        return pool, bdev, blocks
