"""GPU parity of the decode path (HIP kernels through the C ABI) against the
fp64 oracle, on the seeded workloads and on edge cases."""
import numpy as np
import pytest

import oracle
import synth
from synth.gen import LogicalBlock
from tests.gpu_util import compare, custom_workload, note, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# --------------------------------------------------------------------------
# seeded workloads
# --------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_tiny_fp32(variant):
    wl = synth.make_workload(synth.get_config("tiny"), variant=variant)
    out, lse = run_hip(wl)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=f"tiny/{variant}")
    # fp32 storage: the only rounding is fp32 accumulation
    np.testing.assert_allclose(out, ref_o, rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_qwen05b_16k_full(variant):
    wl = synth.make_workload(synth.get_config("qwen05b_16k"), variant=variant)
    out, lse = run_hip(wl)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=(variant == "sharp"), name=f"qwen05b_16k/{variant}")


@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_qwen7b_64k_sampled(variant):
    """Full 64k workload on the GPU; oracle on two whole sequences."""
    cfg = synth.get_config("qwen7b_64k")
    wl = synth.make_workload(cfg, variant=variant)
    out, lse = run_hip(wl)
    seqs = [0, cfg.batch - 1]
    ref_o, ref_l = oracle.attend(wl, seq_index=seqs)
    compare(out[seqs], lse[seqs], ref_o, ref_l, sharp_gates=(variant == "sharp"),
            name=f"qwen7b_64k/{variant}")


def test_qwen7b_64k_group8_sampled():
    """The 64k workload with 32 query heads (group size 8, the largest group
    the vector-ALU decode unit takes) on the sharp variant; oracle on two
    whole sequences."""
    cfg = synth.get_config("qwen7b_64k").with_(name="qwen7b_64k_g8", n_q_heads=32)
    wl = synth.make_workload(cfg, variant="sharp")
    out, lse = run_hip(wl)
    seqs = [0, cfg.batch - 1]
    ref_o, ref_l = oracle.attend(wl, seq_index=seqs)
    compare(out[seqs], lse[seqs], ref_o, ref_l, sharp_gates=True, name="qwen7b_64k_g8/sharp")


def test_qwen7b_128k_sampled():
    cfg = synth.get_config("qwen7b_128k")
    wl = synth.make_workload(cfg, variant="sharp")
    out, lse = run_hip(wl)
    seqs = [0, 17]
    ref_o, ref_l = oracle.attend(wl, seq_index=seqs)
    compare(out[seqs], lse[seqs], ref_o, ref_l, sharp_gates=True, name="qwen7b_128k/sharp")


# --------------------------------------------------------------------------
# ragged shapes: every group size, both head dims and dtypes, ragged tokens,
# odd/zero/full ranks, empty sequences, partial tails, multi-tile blocks
# --------------------------------------------------------------------------
RAGGED = [
    # (dtype, d, Hq, Hkv)
    ("bf16", 128, 7, 1), ("bf16", 128, 8, 1), ("bf16", 128, 10, 2), ("bf16", 64, 12, 4),
    ("bf16", 64, 3, 3), ("bf16", 128, 12, 2), ("bf16", 128, 6, 2), ("bf16", 64, 14, 2),
    ("bf16", 128, 4, 2), ("bf16", 64, 8, 2), ("bf16", 128, 16, 4), ("bf16", 64, 4, 1),
    ("f32", 64, 4, 2), ("f32", 128, 7, 1), ("f32", 128, 5, 5),
]


@pytest.mark.parametrize("dtype,d,hq,hkv", RAGGED)
def test_ragged_shapes(dtype, d, hq, hkv):
    base = synth.get_config("qwen05b_16k")
    cfg = base.with_(name=f"ragged_{dtype}_{d}_{hq}_{hkv}", batch=4, n_q_heads=hq, n_kv_heads=hkv,
                     head_dim=d, dtype=dtype, tail_len=70,
                     ranks=synth.configs.RankDist("uniform", lo=0, hi=d), seed=11)
    toks = [[1, 37, 1024, 2049, 8], [], [511, 7], [3000]]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[len(t) for t in toks], tokens=toks,
                             tail_len=[70, 0, 1, 33])
    out, lse = run_hip(wl, shuffle_pool=3, max_blocks=6)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)
    # sequence 1 has nothing to attend to
    assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))


def test_full_and_extreme_ranks():
    cfg = synth.get_config("qwen7b_64k").with_(name="rank_extremes", batch=2, n_blocks=4,
                                               ranks=synth.configs.RankDist("list", values=(128, 1, 0, 127)),
                                               v_rank_equals_k=False, seed=12)
    wl = synth.make_workload(cfg, variant="sharp", tail_len=[256, 13])
    out, lse = run_hip(wl)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name="rank_extremes")


def test_schedule_does_not_change_results():
    """The largest-first unit order only changes when units run."""
    cfg = synth.get_config("qwen7b_64k").with_(batch=3, n_blocks=6)
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[6, 1, 4], tail_len=[256, 3, 0])
    o1, l1 = run_hip(wl, plan=True)
    o2, l2 = run_hip(wl, plan=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_deterministic_and_bounded_writes():
    import torch
    import rank_attention_amd as ra
    cfg = synth.get_config("qwen05b_16k").with_(batch=3, n_blocks=5)
    wl = synth.make_workload(cfg, variant="sharp")
    (o1, l1), (o2, l2) = run_hip(wl, repeat=2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # guard bands around out and lse stay untouched
    dc = ra.DeviceCache(ra.pack(wl), scale=wl.scale)
    B, Q, Hq, d = wl.q.shape
    note("guard-band decode")
    big = torch.full((B * Q * Hq * d + 2 * 64,), 12345.0, device="cuda")
    lbig = torch.full((B * Q * Hq + 2 * 64,), 777.0, device="cuda")
    out = big[64:64 + B * Q * Hq * d].view(B, Q, Hq, d)
    lse = lbig[64:64 + B * Q * Hq].view(B, Q, Hq)
    dc.decode(out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(big[:64] == 12345.0) and torch.all(big[-64:] == 12345.0)
    assert torch.all(lbig[:64] == 777.0) and torch.all(lbig[-64:] == 777.0)
    assert np.array_equal(out.cpu().numpy(), o1.astype(np.float32))


# --------------------------------------------------------------------------
# bit-exact indexing probe
# --------------------------------------------------------------------------
def code_row(i, g, b, k, d):
    j = np.arange(d)
    return (((i * 31 + g * 17 + b * 7 + k * 5 + j) % 251) - 125).astype(np.float32)


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 28, 4), ("bf16", 64, 14, 2),
                                            ("f32", 64, 8, 1), ("bf16", 128, 40, 8)])
def test_one_hot_indexing_is_bit_exact(dtype, d, hq, hkv):
    """Each query head has one winning token (score gap 200) whose value is a
    row of W' holding integers that encode (sequence, KV head, block, rank
    row); the output must equal that row exactly."""
    from tests.gpu_util import bf16_bits
    G = hq // hkv
    cfg = synth.get_config("qwen7b_64k").with_(name=f"onehot_{dtype}_{d}", batch=3, n_q_heads=hq,
                                               n_kv_heads=hkv, head_dim=d, dtype=dtype)
    rng = np.random.default_rng(7)
    store = (lambda x: bf16_bits(x)) if dtype == "bf16" else (lambda x: np.asarray(x, np.float32))
    A = 200.0 / cfg.scale
    toks = [[37, 1024, 2049, 8, 600], [1000, 9, 3], [2500]]
    cap = 48
    q = np.zeros((3, 1, hq, d), np.float32)
    kt = np.zeros((3, hkv, cap, d), np.float32)
    vt = rng.standard_normal((3, hkv, cap, d)).astype(np.float32)
    tail_len = [40, 0, 48]
    expected = np.zeros((3, 1, hq, d), np.float32)
    blocks = []
    for i, tl in enumerate(toks):
        nb = len(tl)
        rks = [int(rng.integers(G, d + 1)) for _ in range(nb)]
        rvs = [int(rng.integers(1, d + 1)) for _ in range(nb)]
        ut = [np.zeros((hkv, rks[b], tl[b]), np.float32) for b in range(nb)]
        w = [np.zeros((hkv, rks[b], d), np.float32) for b in range(nb)]
        upt = [rng.standard_normal((hkv, rvs[b], tl[b])).astype(np.float32) for b in range(nb)]
        wp = [np.stack([np.stack([code_row(i, g, b, k, d) for k in range(rvs[b])]) for g in range(hkv)])
              for b in range(nb)]
        for b in range(nb):
            for k in range(rks[b]):
                w[b][:, k, k] = 1.0            # W rows are unit vectors e_k
        for g in range(hkv):
            used = set()
            for hl in range(G):
                h = g * G + hl
                q[i, 0, h, hl] = A
                if (hl % 3 == 2 and tail_len[i] > 0) or nb == 0:
                    t = (7 * hl + i) % tail_len[i]
                    kt[i, g, t, hl] = 1.0
                    vt[i, g, t] = code_row(i, g, 99, t, d)
                    expected[i, 0, h] = vt[i, g, t]
                    continue
                while True:
                    b = int(rng.integers(nb))
                    t = int(rng.integers(tl[b]))
                    if (b, t) not in used:
                        break
                used.add((b, t))
                k = int(rng.integers(rvs[b])) if hl % 2 else rvs[b] - 1
                ut[b][g, hl, t] = 1.0
                upt[b][g, :, t] = 0.0
                upt[b][g, k, t] = 1.0
                expected[i, 0, h] = wp[b][g, k]
        blocks.append([LogicalBlock(tl[b], rks[b], rvs[b], store(ut[b]), store(w[b]), store(upt[b]),
                                    store(wp[b])) for b in range(nb)])
    wl = custom_workload(cfg, blocks, store(q), store(kt), store(vt), tail_len)
    exp = expected.astype(np.float64)
    if dtype == "bf16":
        exp = synth.gen.bf16_bits_to_f32(bf16_bits(expected)).astype(np.float64)
    out, lse = run_hip(wl, shuffle_pool=1)
    assert np.array_equal(out, exp), f"max diff {np.abs(out - exp).max()}"
    ref_o, _ = oracle.attend(wl)
    np.testing.assert_allclose(ref_o, exp, rtol=0, atol=1e-9)


# --------------------------------------------------------------------------
# group sizes 9-16: decode on the matrix-core kernel of the chunked path
# --------------------------------------------------------------------------
@pytest.mark.parametrize("hq,hkv", [(12, 1), (32, 2), (48, 4)])
def test_large_group_decode(hq, hkv):
    cfg = synth.get_config("qwen7b_64k").with_(name=f"large_group_{hq}_{hkv}", batch=3, n_q_heads=hq,
                                               n_kv_heads=hkv, n_blocks=6, seed=61,
                                               ranks=synth.configs.RankDist("uniform", lo=0, hi=128))
    toks = [[1024, 37, 0, 64, 700, 2], [65], []]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[len(t) for t in toks], tokens=toks,
                             tail_len=[256, 0, 9])
    out, lse = run_hip(wl, shuffle_pool=4, ld_extra=8)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)
