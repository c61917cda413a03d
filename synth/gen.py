"""Seeded synthetic factors, queries and dense tails.

Every array is drawn from its own counter-free stream:
``PCG64(SeedSequence([seed, variant_id, stream, ...]))``, so the values of one
sequence or one block do not depend on which other sequences are generated or
on thread scheduling.  Floating values are drawn in float32 and stored either
as float32 or rounded to bfloat16 (round-to-nearest-even); bfloat16 arrays are
kept as their uint16 bit patterns.

Distributions (MILO compresses each block's keys and values separately with
a low-rank approximation, MILO summary "4.2 Block-wise Low-Rank Compression";
the synthetic stand-in for a truncated SVD is):
  U_b, U'_b ~ N(0, 1)                       (T_b x r_b, T_b x r'_b)
  W_b = diag(0.8^i) * Q^T                    (r_b x d), Q = orthonormal d x r_b
  q ~ N(0, 1)
  dense tail K_t = U_t W_t, V_t = U'_t W'_t with full rank r = d.
U is drawn rank-major (as U^T, r_b x T_b); any order of iid draws is valid.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .configs import Config, EncodeConfig

VARIANTS = {"base": 0, "sharp": 1}

# stream ids
_S_RANK, _S_Q, _S_BLOCK, _S_TAIL, _S_DENSE = 0, 1, 2, 3, 4


def _one_blas_thread():
    """Keep BLAS single-threaded while the generator runs its own threads."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        import contextlib
        return contextlib.nullcontext()


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    raise ValueError(dtype)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of a stored array as float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _orth_rows(rng: np.random.Generator, r: int, d: int, heads: int = 1) -> np.ndarray:
    """[heads][r][d]: diag(0.8^i) * Q^T with Q from the QR of a d x r Gaussian,
    column signs fixed so that diag(R) > 0."""
    if r == 0:
        return np.zeros((heads, 0, d), np.float64)
    g = rng.standard_normal((heads, d, r))
    qm, rm = np.linalg.qr(g)
    sgn = np.sign(np.diagonal(rm, axis1=1, axis2=2))
    sgn[sgn == 0] = 1.0
    qm = qm * sgn[:, None, :]
    return (0.8 ** np.arange(r))[None, :, None] * np.swapaxes(qm, 1, 2)


@dataclass
class LogicalBlock:
    """One compressed block, all KV heads, in the stored dtype.

    ut  [Hkv][rank_k][n_tok]  U_b^T   (keys:  K_b ~= U_b W_b)
    w   [Hkv][rank_k][d]      W_b
    upt [Hkv][rank_v][n_tok]  U'_b^T  (values: V_b ~= U'_b W'_b)
    wp  [Hkv][rank_v][d]      W'_b
    """
    n_tok: int
    rank_k: int
    rank_v: int
    ut: np.ndarray
    w: np.ndarray
    upt: np.ndarray
    wp: np.ndarray


@dataclass
class Workload:
    cfg: Config
    variant: str
    seqs: List[int]                 # which sequences of the config these are
    q: np.ndarray                   # [B][Q][Hq][d] stored dtype
    blocks: List[List[LogicalBlock]]  # per sequence, the blocks its CSR lists
    k_tail: np.ndarray              # [B][Hkv][L_cap][d]
    v_tail: np.ndarray
    tail_len: np.ndarray            # int32 [B]
    scale: float
    extra: dict = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.cfg.dtype

    @property
    def batch(self) -> int:
        return len(self.seqs)

    @property
    def tail_cap(self) -> int:
        return int(self.k_tail.shape[2])

    def context_tokens(self) -> int:
        """Tokens attended per call: all block tokens plus the tails."""
        return int(sum(b.n_tok for s in self.blocks for b in s) + int(self.tail_len.sum()))

    def factor_bytes(self) -> int:
        """Bytes of U, W, U', W' at their actual ranks, unpadded."""
        es = 2 if self.dtype == "bf16" else 4
        d = self.cfg.head_dim
        h = self.cfg.n_kv_heads
        return int(sum(h * es * (b.rank_k + b.rank_v) * (b.n_tok + d)
                       for s in self.blocks for b in s))

    def tail_bytes(self) -> int:
        es = 2 if self.dtype == "bf16" else 4
        return int(2 * es * self.cfg.n_kv_heads * self.cfg.head_dim * int(self.tail_len.sum()))


def draw_ranks(cfg: Config, variant: str, n_blocks: Sequence[int]) -> List[np.ndarray]:
    """Per sequence an int array [n_blocks][2] of (r_b, r'_b)."""
    rd = cfg.ranks
    rng = _rng(cfg.seed, VARIANTS[variant], _S_RANK)
    out = []
    for nb in n_blocks:
        if rd.kind == "list":
            rk = np.array([rd.values[b % len(rd.values)] for b in range(nb)], np.int64)
            rv = rk.copy()
        else:
            def draw(n):
                if rd.kind == "uniform":
                    return rng.integers(rd.lo, rd.hi + 1, size=n)
                if rd.kind == "lognormal":
                    x = np.rint(rd.median * np.exp(rd.sigma * rng.standard_normal(n)))
                    return np.clip(x, rd.lo, rd.hi).astype(np.int64)
                if rd.kind == "bimodal":
                    hi = rng.random(n) < rd.p_hi
                    a = rng.integers(rd.hi_lo, rd.hi_hi + 1, size=n)
                    b = rng.integers(rd.lo, rd.hi + 1, size=n)
                    return np.where(hi, a, b)
                raise ValueError(rd.kind)
            rk = draw(nb)
            rv = rk.copy() if cfg.v_rank_equals_k else draw(nb)
        out.append(np.stack([rk, rv], axis=1).astype(np.int64))
    return out


def _gen_block(cfg: Config, variant: str, seq: int, b: int, n_tok: int, rk: int, rv: int,
               u_scale: float) -> LogicalBlock:
    rng = _rng(cfg.seed, VARIANTS[variant], _S_BLOCK, seq, b)
    d, h = cfg.head_dim, cfg.n_kv_heads
    ut = rng.standard_normal((h, rk, n_tok), dtype=np.float32)
    w = _orth_rows(rng, rk, d, h)
    upt = rng.standard_normal((h, rv, n_tok), dtype=np.float32)
    wp = _orth_rows(rng, rv, d, h)
    if u_scale != 1.0:
        ut *= np.float32(u_scale)
    if variant == "sharp":
        upt += np.float32(1.0)
    return LogicalBlock(n_tok, rk, rv, _store(ut, cfg.dtype), _store(w, cfg.dtype),
                        _store(upt, cfg.dtype), _store(wp, cfg.dtype))


def make_workload(cfg: Config, variant: str = "base", seqs: Optional[Sequence[int]] = None,
                  n_blocks: Optional[Sequence[int]] = None,
                  tokens: Optional[Sequence[Sequence[int]]] = None,
                  tail_len: Optional[Sequence[int]] = None,
                  threads: Optional[int] = None) -> Workload:
    """Draw the inputs of one call.

    seqs      which sequences of the workload to draw (default: all); a subset
              has exactly the values the full draw has for those sequences.
    n_blocks  per-sequence block counts (default cfg.n_blocks for every one).
    tokens    per-sequence list of T_b (default cfg.block_tokens).
    tail_len  per-sequence visible tail lengths (default cfg.tail_len).
    """
    B = cfg.batch
    nbs = list(n_blocks) if n_blocks is not None else [cfg.n_blocks] * B
    if len(nbs) != B:
        raise ValueError("n_blocks must list every sequence of the workload")
    seqs = list(range(B)) if seqs is None else [int(s) for s in seqs]
    ranks = draw_ranks(cfg, variant, nbs)
    d, hq, hkv, Q = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.q_len

    tl = np.array(tail_len if tail_len is not None else [cfg.tail_len] * B, np.int32)
    cap = int(max(cfg.tail_len, int(tl.max()) if len(tl) else 0))

    # sharp variant: q scaled so that the score std is about 3 (the synthetic
    # score std is scale * sqrt(sum_i 0.64^i) ~= 1.667 * scale), and key
    # factors of later blocks scaled up so the running max rises block by block.
    q_mult = 1.0
    if variant == "sharp":
        q_mult = 3.0 / (cfg.scale * np.sqrt(1.0 / (1.0 - 0.64)))

    tasks = []
    for si, s in enumerate(seqs):
        nb = nbs[s]
        for b in range(nb):
            T = int(tokens[s][b]) if tokens is not None else cfg.block_tokens
            u_scale = 1.0
            if variant == "sharp":
                u_scale = 0.5 + (b / max(1, nb - 1))
            tasks.append((si, s, b, T, int(ranks[s][b, 0]), int(ranks[s][b, 1]), u_scale))

    nthr = threads or min(16, os.cpu_count() or 1)
    with _one_blas_thread(), ThreadPoolExecutor(max_workers=nthr) as ex:
        res = list(ex.map(lambda t: _gen_block(cfg, variant, t[1], t[2], t[3], t[4], t[5], t[6]), tasks))
    blocks: List[List[LogicalBlock]] = [[] for _ in seqs]
    for t, blk in zip(tasks, res):
        blocks[t[0]].append(blk)

    q = np.empty((len(seqs), Q, hq, d), np.float32)
    kt = np.zeros((len(seqs), hkv, cap, d), np.float32)
    vt = np.zeros((len(seqs), hkv, cap, d), np.float32)
    for si, s in enumerate(seqs):
        rq = _rng(cfg.seed, VARIANTS[variant], _S_Q, s)
        q[si] = rq.standard_normal((Q, hq, d), dtype=np.float32) * np.float32(q_mult)
        if cap > 0:
            rt = _rng(cfg.seed, VARIANTS[variant], _S_TAIL, s)
            uk = rt.standard_normal((hkv, cap, d))
            wk = _orth_rows(rt, d, d, hkv)
            uv = rt.standard_normal((hkv, cap, d))
            wv = _orth_rows(rt, d, d, hkv)
            kt[si] = (uk @ wk).astype(np.float32)
            vt[si] = (uv @ wv).astype(np.float32)
            if variant == "sharp":
                vt[si] += np.float32(1.0)
    return Workload(cfg=cfg, variant=variant, seqs=seqs, q=_store(q, cfg.dtype), blocks=blocks,
                    k_tail=_store(kt, cfg.dtype), v_tail=_store(vt, cfg.dtype),
                    tail_len=tl[seqs].astype(np.int32), scale=cfg.scale)


# ---------------------------------------------------------------------------
# Dense contexts for the encode step
# ---------------------------------------------------------------------------
ENCODE_VARIANTS = {"base": 0, "planted": 1}


@dataclass
class DenseContext:
    """Dense keys and values of one context, split into blocks.

    k, v       [Hkv][N][d] in the stored dtype, N = sum of the block sizes
    tok_start  int64 [n_blocks]: block b covers tokens tok_start[b] .. + n_tok[b] - 1
    n_tok      int32 [n_blocks]
    ranks      int64 [n_blocks][2]: target (r_b, r'_b) drawn from the config
    decay      float64 [n_blocks][Hkv][2]: the rho each (block, head, K/V) was drawn with
    """
    cfg: EncodeConfig
    variant: str
    k: np.ndarray
    v: np.ndarray
    tok_start: np.ndarray
    n_tok: np.ndarray
    ranks: np.ndarray
    decay: np.ndarray

    def dense_f64(self, kv: int, b: int, g: int) -> np.ndarray:
        """Exact stored values of block b, KV head g, keys (kv 0) or values (kv 1)."""
        a = self.k if kv == 0 else self.v
        s, n = int(self.tok_start[b]), int(self.n_tok[b])
        return stored_to_f64(a[g, s:s + n], self.cfg.dtype)


def _dense_block(cfg: EncodeConfig, variant: str, b: int, T: int):
    """[Hkv][2][T][d] float32 and the drawn decays [Hkv][2]."""
    rng = _rng(cfg.seed, ENCODE_VARIANTS[variant], _S_DENSE, b)
    d, h = cfg.head_dim, cfg.n_kv_heads
    out = np.empty((h, 2, T, d), np.float32)
    rho = rng.uniform(cfg.decay_lo, cfg.decay_hi, size=(h, 2))
    for g in range(h):
        for kv in range(2):
            a = rng.standard_normal((T, d))
            qm, rm = np.linalg.qr(rng.standard_normal((d, d)))
            scale = rho[g, kv] ** np.arange(d)
            if variant == "planted":   # exactly rank planted_rank (before rounding), flat spectrum
                scale = (np.arange(d) < cfg.planted_rank).astype(np.float64)
            out[g, kv] = ((a * scale[None, :]) @ qm.T).astype(np.float32)
    return out, rho


def make_dense_context(cfg: EncodeConfig, variant: str = "base",
                       tokens: Optional[Sequence[int]] = None) -> DenseContext:
    """Draw one context's dense K and V (tokens: per-block sizes, default
    cfg.block_tokens each)."""
    toks = [int(t) for t in tokens] if tokens is not None else [cfg.block_tokens] * cfg.n_blocks
    nb = len(toks)
    starts = np.concatenate([[0], np.cumsum(toks)[:-1]]).astype(np.int64) if nb else np.zeros(0, np.int64)
    N = int(sum(toks))
    d, h = cfg.head_dim, cfg.n_kv_heads
    k = np.empty((h, N, d), np.float32)
    v = np.empty((h, N, d), np.float32)
    decay = np.empty((nb, h, 2))
    with _one_blas_thread(), ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        res = list(ex.map(lambda b: _dense_block(cfg, variant, b, toks[b]), range(nb)))
    for b, (x, rho) in enumerate(res):
        s = starts[b]
        k[:, s:s + toks[b]] = x[:, 0]
        v[:, s:s + toks[b]] = x[:, 1]
        decay[b] = rho
    # target ranks: the decode workloads' rank model on a one-sequence draw
    rcfg = Config(name=cfg.name, batch=1, q_len=1, n_q_heads=h, n_kv_heads=h, head_dim=d,
                  n_blocks=nb, block_tokens=cfg.block_tokens, ranks=cfg.ranks, tail_len=0,
                  dtype=cfg.dtype, path="decode", seed=cfg.seed)
    ranks = draw_ranks(rcfg, "base", [nb])[0]
    return DenseContext(cfg=cfg, variant=variant, k=_store(k, cfg.dtype), v=_store(v, cfg.dtype),
                        tok_start=starts, n_tok=np.array(toks, np.int32), ranks=ranks, decay=decay)


_S_SPECTRA = 5


def make_spectra(n_blocks: int, n_kv_heads: int, head_dim: int, seed: int,
                 decay_lo: float = 0.6, decay_hi: float = 0.98) -> np.ndarray:
    """Seeded singular-value spectra float32 [n_blocks][Hkv][2][head_dim],
    descending: sigma_i = a * rho^i with rho ~ U[decay_lo, decay_hi] per
    (block, head, K/V) and a ~ lognormal.  Block 1 (if present) has a
    planted rank of head_dim // 4, block 2 is all zero, block 3 is flat."""
    rng = _rng(seed, _S_SPECTRA)
    rho = rng.uniform(decay_lo, decay_hi, size=(n_blocks, n_kv_heads, 2))
    amp = np.exp(rng.standard_normal((n_blocks, n_kv_heads, 2)))
    s = amp[..., None] * rho[..., None] ** np.arange(head_dim)
    if n_blocks > 1:
        s[1, ..., head_dim // 4:] = 0.0
    if n_blocks > 2:
        s[2] = 0.0
    if n_blocks > 3:
        s[3] = amp[3][..., None]
    return s.astype(np.float32)
