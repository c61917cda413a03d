"""The seeded input generator: determinism, subsets, rounding, distributions,
and the byte accounting against the figures the pages print."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from synth.gen import draw_ranks, f32_to_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_is_rne_like_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0, 1e-30], np.float32)])
    mine = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_is_deterministic_and_subsets_match():
    cfg = synth.get_config("qwen05b_16k").with_(batch=3, n_blocks=3)
    a = synth.make_workload(cfg)
    b = synth.make_workload(cfg, threads=1)
    c = synth.make_workload(cfg, seqs=[2])
    for x, y in [(a.q, b.q), (a.k_tail, b.k_tail)]:
        np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(a.q[2], c.q[0])
    np.testing.assert_array_equal(a.v_tail[2], c.v_tail[0])
    for blk_a, blk_c in zip(a.blocks[2], c.blocks[0]):
        assert (blk_a.rank_k, blk_a.rank_v) == (blk_c.rank_k, blk_c.rank_v)
        for f in ("ut", "w", "upt", "wp"):
            np.testing.assert_array_equal(getattr(blk_a, f), getattr(blk_c, f))


def test_factor_rows_are_scaled_orthonormal():
    cfg = synth.get_config("tiny")
    wl = synth.make_workload(cfg)
    for b in wl.blocks[0]:
        W = b.w[0].astype(np.float64)
        G = W @ W.T
        np.testing.assert_allclose(G, np.diag(0.64 ** np.arange(b.rank_k)), atol=1e-6)
    assert [b.rank_k for b in wl.blocks[0]] == [8, 16, 24, 32]
    assert [b.rank_v for b in wl.blocks[0]] == [8, 16, 24, 32]


@pytest.mark.parametrize("name,lo,hi,mean_lo,mean_hi", [
    ("qwen05b_16k", 8, 48, 25, 31),
    ("qwen7b_64k", 16, 96, 46, 56),
    ("qwen32b_chunk", 16, 128, 62, 76),
])
def test_rank_draws(name, lo, hi, mean_lo, mean_hi):
    cfg = synth.get_config(name)
    r = np.concatenate(draw_ranks(cfg, "base", [cfg.n_blocks] * cfg.batch))
    assert r.min() >= lo and r.max() <= hi
    assert mean_lo <= r.mean() <= mean_hi


def test_bimodal_rank_mix():
    cfg = synth.get_config("qwen7b_128k")
    r = np.concatenate(draw_ranks(cfg, "base", [cfg.n_blocks] * cfg.batch)).ravel()
    hi = (r >= 96).mean()
    assert 0.25 < hi < 0.35
    assert set(np.unique(r[r >= 96])) <= set(range(96, 129))
    assert set(np.unique(r[r < 96])) <= set(range(8, 33))


def test_pages_memory_figures():
    """Byte accounting against the figures the MILO summary prints."""
    figs = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    # (a) half the rank budget gives half the KV bytes once blocks are long
    half = figs["kv_memory_at_half_rank"]
    d = 128
    for T in (1024, 8192, 1 << 20):
        r = d // 2
        ratio = (r + r) * (T + d) / (2 * T * d)
        assert ratio >= half["fraction"]
    assert abs((64 + 64) * ((1 << 20) + d) / (2 * (1 << 20) * d) - half["fraction"]) < 1e-3
    # (b) dense KV bytes of a many-shot context on an 8B dense model
    kv = figs["extra_kv_for_90k"]
    m = kv["model_reading"]
    dense = kv["tokens"] * m["layers"] * m["kv_heads"] * m["head_dim"] * 2 * m["bytes_per_value"]
    assert abs(dense / 2 ** 30 - kv["gigabytes"]) / kv["gigabytes"] < kv["rel_tol"]


def test_workload_byte_counts():
    cfg = synth.get_config("qwen05b_16k").with_(batch=2, n_blocks=4)
    wl = synth.make_workload(cfg)
    exp = sum(2 * 2 * (b.rank_k + b.rank_v) * (b.n_tok + 64) for s in wl.blocks for b in s)
    assert wl.factor_bytes() == exp
    assert wl.context_tokens() == 2 * 4 * 512 + 2 * 128
