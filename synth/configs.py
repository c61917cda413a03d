"""Workload shapes for attention over a block-wise low-rank KV cache.

The five workloads mirror the head shapes of Qwen2.5 models used by MILO
(MILO summary, "5.1 Experimental Setup": Qwen2.5-3B/7B) and its block
granularity of about 32 demonstrations per block ("5.3 Performance
Analysis": gains up to ~32 examples per block, i.e. 512-2048 tokens here).
Where the workload text leaves a parameter open, the reading is recorded in
the field's comment.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class RankDist:
    """How the per-block ranks r_b (keys) and r'_b (values) are drawn.

    kind:
      "list"      explicit ranks, block b gets values[b % len(values)]
      "uniform"   integer uniform on [lo, hi]
      "lognormal" clip(round(median * exp(sigma * N(0,1))), lo, hi)
      "bimodal"   with prob p_hi: uniform [hi_lo, hi_hi], else uniform [lo, hi]
    """
    kind: str
    values: Tuple[int, ...] = ()
    lo: int = 0
    hi: int = 0
    median: float = 0.0
    sigma: float = 0.5
    p_hi: float = 0.0
    hi_lo: int = 0
    hi_hi: int = 0


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    q_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_blocks: int            # blocks per sequence
    block_tokens: int        # T_b (all blocks of a workload share it)
    ranks: RankDist
    tail_len: int            # dense uncompressed recent tokens per sequence
    dtype: str               # "f32" or "bf16": storage type of q, factors, tail
    path: str                # "decode" or "chunk"
    seed: int
    v_rank_equals_k: bool = False   # the tiny workload ties r'_b to r_b
    desc: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # 1 head, d=64, 4 blocks x 256 tokens with ranks 8/16/24/32, fp32, no tail.
    "tiny": Config(
        name="tiny", batch=1, q_len=1, n_q_heads=1, n_kv_heads=1, head_dim=64,
        n_blocks=4, block_tokens=256, ranks=RankDist("list", values=(8, 16, 24, 32)),
        tail_len=0, dtype="f32", path="decode", seed=0, v_rank_equals_k=True,
        desc="tiny: 1/1 heads, d64, 4x256 tokens, ranks {8,16,24,32}, fp32, B=1"),
    # Qwen2.5-0.5B-like layer: 14/2 heads, d=64, 16k context in 512-token blocks.
    "qwen05b_16k": Config(
        name="qwen05b_16k", batch=8, q_len=1, n_q_heads=14, n_kv_heads=2, head_dim=64,
        n_blocks=32, block_tokens=512, ranks=RankDist("uniform", lo=8, hi=48),
        tail_len=128, dtype="bf16", path="decode", seed=1,
        desc="Qwen2.5-0.5B-like: 14/2 heads, d64, 32x512 tokens, r~U{8..48}, tail 128, B=8"),
    # Qwen2.5-7B-like layer at 64k: the headline decode workload.
    # The lognormal sigma is not stated; read sigma = 0.5.
    "qwen7b_64k": Config(
        name="qwen7b_64k", batch=16, q_len=1, n_q_heads=28, n_kv_heads=4, head_dim=128,
        n_blocks=64, block_tokens=1024,
        ranks=RankDist("lognormal", median=48.0, sigma=0.5, lo=16, hi=96),
        tail_len=256, dtype="bf16", path="decode", seed=2,
        desc="Qwen2.5-7B-like: 28/4 heads, d128, 64x1024 tokens, r~clip(lognormal(48)), tail 256, B=16"),
    # Qwen2.5-7B-like layer at 128k with a bimodal rank mix.
    "qwen7b_128k": Config(
        name="qwen7b_128k", batch=32, q_len=1, n_q_heads=28, n_kv_heads=4, head_dim=128,
        n_blocks=64, block_tokens=2048,
        ranks=RankDist("bimodal", p_hi=0.3, hi_lo=96, hi_hi=128, lo=8, hi=32),
        tail_len=512, dtype="bf16", path="decode", seed=3,
        desc="Qwen2.5-7B-like: 28/4 heads, d128, 64x2048 tokens, 30% r~U{96..128} / 70% r~U{8..32}, tail 512, B=32"),
    # Qwen2.5-32B-like layer, chunked query path.  The tail length is not
    # stated; read L = Q = 256 (the tail is the chunk itself).  The lognormal
    # range is not stated; read clip to [16, 128], sigma 0.5.
    "qwen32b_chunk": Config(
        name="qwen32b_chunk", batch=4, q_len=256, n_q_heads=40, n_kv_heads=8, head_dim=128,
        n_blocks=96, block_tokens=1024,
        ranks=RankDist("lognormal", median=64.0, sigma=0.5, lo=16, hi=128),
        tail_len=256, dtype="bf16", path="chunk", seed=4,
        desc="Qwen2.5-32B-like chunk: 40/8 heads, d128, 96x1024 tokens, Q=256 causal over a 256-token tail, B=4"),
}

CONFIG_ORDER = ["tiny", "qwen05b_16k", "qwen7b_64k", "qwen7b_128k", "qwen32b_chunk"]


def get_config(name: str) -> Config:
    return CONFIGS[name]


# ---------------------------------------------------------------------------
# Encode workloads: dense keys and values of a demonstration context, split
# into blocks, to be factorised per block (MILO summary, "4.2 Block-wise
# Low-Rank Compression" and "4.4 MILO Workflow").  Per block, KV head and K/V
# the dense matrix is A diag(rho^i) Q^T (A ~ N(0,1), Q orthonormal), the same
# model as the decode workloads' factors, with a decay rho drawn per matrix
# so that blocks differ in how fast their spectra fall (what rank allocation,
# "4.3 Dynamic Rank Allocation", responds to).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class EncodeConfig:
    name: str
    n_blocks: int
    block_tokens: int
    n_kv_heads: int
    head_dim: int
    decay_lo: float          # rho ~ U[decay_lo, decay_hi] per (block, head, K/V)
    decay_hi: float
    ranks: RankDist          # target (r_b, r'_b) when ranks are given
    dtype: str
    seed: int
    planted_rank: int = 0    # variant "planted": scale 1 for i < planted_rank, 0 after
    desc: str = ""

    def with_(self, **kw) -> "EncodeConfig":
        return replace(self, **kw)


ENCODE_CONFIGS = {
    "enc_small": EncodeConfig(
        name="enc_small", n_blocks=5, block_tokens=256, n_kv_heads=2, head_dim=128,
        decay_lo=0.6, decay_hi=0.97, ranks=RankDist("uniform", lo=0, hi=128), dtype="bf16",
        seed=40, planted_rank=24,
        desc="5 blocks x 256 tokens, 2 KV heads, d128, rho~U[0.6,0.97], r~U{0..128}"),
    # One pre-encoded demonstration context at the headline decode shape:
    # 64 blocks of 1024 tokens, Qwen2.5-7B-like KV heads.
    "enc_qwen7b_64k": EncodeConfig(
        name="enc_qwen7b_64k", n_blocks=64, block_tokens=1024, n_kv_heads=4, head_dim=128,
        decay_lo=0.7, decay_hi=0.97,
        ranks=RankDist("lognormal", median=48.0, sigma=0.5, lo=16, hi=96), dtype="bf16",
        seed=41, planted_rank=48,
        desc="one 64k context: 64 blocks x 1024 tokens, 4 KV heads, d128, rho~U[0.7,0.97], "
             "r~clip(lognormal(48))"),
    "enc_d64_f32": EncodeConfig(
        name="enc_d64_f32", n_blocks=3, block_tokens=512, n_kv_heads=2, head_dim=64,
        decay_lo=0.6, decay_hi=0.95, ranks=RankDist("uniform", lo=0, hi=64), dtype="f32",
        seed=42, planted_rank=12,
        desc="3 blocks x 512 tokens, 2 KV heads, d64, fp32, r~U{0..64}"),
}


def get_encode_config(name: str) -> EncodeConfig:
    return ENCODE_CONFIGS[name]
