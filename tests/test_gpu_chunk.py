"""GPU parity of the chunked-query path (MFMA kernel through the C ABI)
against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import chunk_ranges, compare, note, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def small_chunk_cfg(**kw):
    base = synth.get_config("qwen32b_chunk").with_(name="chunk_small", batch=2, n_q_heads=10,
                                                   n_kv_heads=2, n_blocks=5, q_len=48, tail_len=80)
    return base.with_(**kw)


@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_chunk_small_full(variant):
    cfg = small_chunk_cfg()
    wl = synth.make_workload(cfg, variant=variant)
    out, lse = run_hip(wl, path="chunk")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=(variant == "sharp"), name=f"chunk_small/{variant}")


@pytest.mark.parametrize("hq,hkv,q_len", [(8, 1, 33), (6, 2, 16), (3, 3, 70), (16, 2, 40)])
def test_chunk_ragged(hq, hkv, q_len):
    cfg = small_chunk_cfg(name=f"chunk_ragged_{hq}_{hkv}_{q_len}", batch=3, n_q_heads=hq,
                          n_kv_heads=hkv, q_len=q_len, tail_len=q_len + 9,
                          ranks=synth.configs.RankDist("uniform", lo=0, hi=128), seed=21)
    toks = [[37, 1000, 64, 65], [], [1, 130, 2049]]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[len(t) for t in toks], tokens=toks,
                             tail_len=[q_len + 9, q_len, q_len + 100])
    out, lse = run_hip(wl, path="chunk", shuffle_pool=5, max_blocks=5)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)



def test_chunk_long_tails():
    """Tails of up to 11 tiles of 64 tokens: the tail loop's LDS stages wrap
    and refill while loads are in flight; lengths off the tile grid."""
    cfg = small_chunk_cfg(name="chunk_long_tails", batch=3, q_len=20, tail_len=700, n_blocks=2, seed=23)
    wl = synth.make_workload(cfg, variant="sharp", tail_len=[700, 20, 321])
    out, lse = run_hip(wl, path="chunk")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)

def test_chunk_causal_planted_token():
    """A tail token whose key matches every query strongly may only reach the
    queries at or after its position."""
    cfg = small_chunk_cfg(name="chunk_causal", batch=1, n_q_heads=4, n_kv_heads=1, q_len=32,
                          tail_len=40, n_blocks=2)
    wl = synth.make_workload(cfg)
    from synth.gen import bf16_bits_to_f32, f32_to_bf16_bits
    q = bf16_bits_to_f32(wl.q).copy()
    q[...] = 0.0
    q[..., 0] = 1.0
    kt = bf16_bits_to_f32(wl.k_tail).copy()
    vt = bf16_bits_to_f32(wl.v_tail).copy()
    L, Q = 40, 32
    lstar = 20                      # visible to query j iff 20 <= L - Q + j, i.e. j >= 12
    kt[0, 0, lstar] = 0.0
    kt[0, 0, lstar, 0] = 2048.0     # score 2048/sqrt(128) = 181 above everything else
    vt[0, 0, lstar] = 7.0
    wl.q = f32_to_bf16_bits(q)
    wl.k_tail = f32_to_bf16_bits(kt)
    wl.v_tail = f32_to_bf16_bits(vt)
    out, lse = run_hip(wl, path="chunk")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, name="chunk_causal")
    for j in range(Q):
        if j >= L - Q + 0 and lstar <= L - Q + j:
            np.testing.assert_allclose(out[0, j], 7.0, atol=1e-6)
        else:
            assert np.all(np.abs(out[0, j] - 7.0) > 0.5), j


def test_chunk_with_one_query_matches_decode():
    cfg = synth.get_config("qwen7b_64k").with_(name="chunk_vs_decode", batch=2, n_blocks=4)
    wl = synth.make_workload(cfg, variant="sharp")
    od, ld = run_hip(wl, path="decode")
    oc, lc = run_hip(wl, path="chunk")
    compare(oc, lc, od, ld, sharp_gates=True, name="chunk_vs_decode")


def _gate_fails(*args, **kw) -> bool:
    try:
        compare(*args, **kw)
    except AssertionError:
        return True
    return False


def test_chunk_qwen32b_sampled():
    """Full 32B-like chunk workload (24 blocks per range, the launch the
    benchmark times) on the sharp variant, oracle on sampled query rows with
    the per-row relative L2 and lse gates.  The same gates reject an all-zero
    output and the exact output of the context with one block dropped."""
    cfg = synth.get_config("qwen32b_chunk")
    wl = synth.make_workload(cfg, variant="sharp")
    import rank_attention_amd as ra
    dc = ra.DeviceCache(ra.pack(wl), scale=wl.scale)
    nr = chunk_ranges(dc)
    assert cfg.n_blocks / nr >= 2, f"{nr} ranges: fewer than two blocks per range"
    note(f"qwen32b_chunk sharp: {nr} block ranges of {-(-cfg.n_blocks // nr)} blocks")
    out, lse = dc.chunk()
    import torch
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    seqs = [0, cfg.batch - 1]
    js = [0, 1, 77, 128, cfg.q_len - 2, cfg.q_len - 1]
    sel = [(si, j, h) for si in range(len(seqs)) for j in js for h in range(cfg.n_q_heads)]
    note(f"oracle on {len(sel)} sampled rows")
    ref_o, ref_l = oracle.attend(wl, seq_index=seqs, sel=sel)
    idx_g = tuple(np.array([(seqs[si], j, h) for (si, j, h) in sel]).T)
    idx_r = tuple(np.array(sel).T)
    compare(out[idx_g], lse[idx_g], ref_o[idx_r], ref_l[idx_r], sharp_gates=True, name="qwen32b_chunk/sharp")
    # the gates discriminate at this shape: an all-zero output and the output
    # with one block (the middle block of a range) missing both fail them
    zero = np.zeros_like(ref_o[idx_r])
    assert _gate_fails(zero, ref_l[idx_r], ref_o[idx_r], ref_l[idx_r], sharp_gates=True)
    drop = synth.gen.Workload(cfg=wl.cfg, variant=wl.variant, seqs=wl.seqs, q=wl.q,
                              blocks=[list(bl) for bl in wl.blocks], k_tail=wl.k_tail, v_tail=wl.v_tail,
                              tail_len=wl.tail_len, scale=wl.scale)
    for si in seqs:
        del drop.blocks[si][cfg.n_blocks // 2]
    d_o, d_l = oracle.attend(drop, seq_index=seqs, sel=sel)
    assert _gate_fails(d_o[idx_r], d_l[idx_r], ref_o[idx_r], ref_l[idx_r], sharp_gates=True)


# Blocks per sequence in ranges of three (the chunk split of the shapes below
# gives 8 ranges of 3 blocks): each range has a short (one 64-token tile) or
# empty middle block, so the W of block b + 1 and the tiles of block b + 2
# are both in flight during block b.
RANGE_TOKENS = [
    [1024, 64, 1024, 100, 0, 150, 65, 1, 200, 130, 37, 64, 300, 0, 1, 129, 64, 700, 64, 8, 1024, 500, 63, 90],
    [90, 0, 64, 1024, 1, 1024, 200, 64, 65, 7, 0, 3, 640, 64, 128, 66, 40, 1000, 64, 0, 64, 1, 64, 256],
]


def _range_cfg(name):
    return synth.get_config("qwen32b_chunk").with_(
        name=name, batch=2, n_q_heads=32, n_kv_heads=4, q_len=256, tail_len=256,
        n_blocks=len(RANGE_TOKENS[0]), ranks=synth.configs.RankDist("uniform", lo=0, hi=128), seed=31)


def test_chunk_three_blocks_per_range_sharp():
    """Sharp parity where every block range holds three blocks with a short
    or empty middle one, and every U^T / U'^T row carries 16 extra NaN
    padding elements (whole padding chunks past the block end)."""
    cfg = _range_cfg("chunk_ranges_of_3")
    wl = synth.make_workload(cfg, variant="sharp", tokens=RANGE_TOKENS)
    import rank_attention_amd as ra
    dc = ra.DeviceCache(ra.pack(wl, ld_extra=16, shuffle_pool=3), scale=wl.scale)
    nr = chunk_ranges(dc)
    assert nr == 8 and len(RANGE_TOKENS[0]) == 3 * nr, nr
    out, lse = dc.chunk()
    import torch
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    js = [0, 1, 100, 200, 254, 255]
    sel = [(i, j, h) for i in range(2) for j in js for h in range(cfg.n_q_heads)]
    ref_o, ref_l = oracle.attend(wl, sel=sel)
    compare(out, lse, ref_o, ref_l, rows=sel, sharp_gates=True, name=cfg.name)


def one_hot_ranges_workload(d=128):
    """The workload of the one-hot probe below and its exact expected output
    [B][Q][Hq][d] (float32)."""
    from synth.gen import LogicalBlock, bf16_bits_to_f32
    from tests.gpu_util import bf16_bits, custom_workload
    cfg = _range_cfg(f"chunk_onehot_ranges_d{d}").with_(head_dim=d)
    B, Q, Hq, Hkv, d = 2, cfg.q_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = Hq // Hkv
    n_dirs = 16
    rng = np.random.default_rng(5)
    A = 200.0 / cfg.scale

    def code_row(i, g, b, k):
        j = np.arange(d)
        return (((i * 31 + g * 17 + b * 7 + k * 5 + j) % 251) - 125).astype(np.float32)

    direction = lambda j, hl, g: (7 * j + 3 * hl + g) % n_dirs
    q = np.zeros((B, Q, Hq, d), np.float32)
    for j in range(Q):
        for h in range(Hq):
            q[:, j, h, direction(j, h % G, h // G)] = A
    kt = np.zeros((B, Hkv, Q, d), np.float32)
    vt = rng.standard_normal((B, Hkv, Q, d)).astype(np.float32)
    expected_dir = np.zeros((B, Hkv, n_dirs, d), np.float32)
    blocks = []
    for i in range(B):
        toks = RANGE_TOKENS[i]
        nb = len(toks)
        rks = [int(rng.integers(n_dirs, d + 1)) for _ in range(nb)]
        rvs = [int(rng.integers(1, d + 1)) for _ in range(nb)]
        perm = [rng.permutation(d)[:rks[b]] for b in range(nb)]     # W_b[k] = e_perm[b][k]
        ut = [np.zeros((Hkv, rks[b], toks[b]), np.float32) for b in range(nb)]
        w = [np.zeros((Hkv, rks[b], d), np.float32) for b in range(nb)]
        upt = [rng.standard_normal((Hkv, rvs[b], toks[b])).astype(np.float32) for b in range(nb)]
        wp = [np.stack([np.stack([code_row(i, g, b, k) for k in range(rvs[b])]) for g in range(Hkv)])
              for b in range(nb)]
        for b in range(nb):
            w[b][:, np.arange(rks[b]), perm[b]] = 1.0
        for g in range(Hkv):
            used = set()
            for c in range(n_dirs):
                while True:   # a block whose W holds e_c, often a short middle block
                    b = int(rng.integers(nb)) if rng.random() < 0.5 else 3 * int(rng.integers(nb // 3)) + 1
                    if toks[b] == 0 or c not in perm[b]:
                        continue
                    t = int(rng.integers(toks[b]))
                    if (b, t) not in used:
                        break
                used.add((b, t))
                k = int(np.nonzero(perm[b] == c)[0][0])
                kv = int(rng.integers(rvs[b]))
                ut[b][g, k, t] = 1.0
                upt[b][g, :, t] = 0.0
                upt[b][g, kv, t] = 1.0
                expected_dir[i, g, c] = wp[b][g, kv]
        blocks.append([LogicalBlock(toks[b], rks[b], rvs[b], bf16_bits(ut[b]), bf16_bits(w[b]),
                                    bf16_bits(upt[b]), bf16_bits(wp[b])) for b in range(nb)])
    wl = custom_workload(cfg, blocks, bf16_bits(q), bf16_bits(kt), bf16_bits(vt), [Q, Q])
    exp = np.zeros((B, Q, Hq, d), np.float32)
    for j in range(Q):
        for h in range(Hq):
            exp[:, j, h] = expected_dir[:, h // G, direction(j, h % G, h // G)]
    return wl, bf16_bits_to_f32(bf16_bits(exp))


@pytest.mark.parametrize("d", [128, 64])
def test_chunk_one_hot_ranges_of_three(d):
    """Bit-exact indexing on the chunk path with three blocks per range.
    Query row (j, h) looks along one of 16 directions c; every block's W rows
    are distinct unit vectors (a per-block permutation), so a block scores
    through its own W only.  For each (sequence, KV head, c) one token of one
    block carries the key e_k with W_b[k] = e_c (score gap 200 nats) and the
    value one-hot on a rank row of W' whose integers encode (sequence, KV
    head, block, rank); the row's output must equal that W' row exactly.
    At head_dim 64 the kernel's 128-wide tiles carry zero padding."""
    wl, exp = one_hot_ranges_workload(d)
    import rank_attention_amd as ra
    dc = ra.DeviceCache(ra.pack(wl, ld_extra=8, shuffle_pool=9), scale=wl.scale)
    assert chunk_ranges(dc) == 8
    out, _ = dc.chunk()
    import torch
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    bad = np.argwhere(np.any(out != exp, axis=-1))
    assert len(bad) == 0, f"{len(bad)} rows differ, first {bad[:4].tolist()}"
    B, _, Hq, _ = exp.shape
    sel = [(i, j, h) for i in range(B) for j in (0, 37, 255) for h in range(0, Hq, 5)]
    ref_o, _ = oracle.attend(wl, sel=sel)
    idx = tuple(np.array(sel).T)
    np.testing.assert_allclose(ref_o[idx], exp[idx], rtol=0, atol=1e-9)


@pytest.mark.parametrize("hq,hkv,q_len", [(16, 1, 24), (32, 2, 9)])
def test_chunk_large_group(hq, hkv, q_len):
    """Group sizes 9-16 on the chunked path: more query rows per KV head."""
    cfg = small_chunk_cfg(name=f"chunk_large_group_{hq}_{hkv}", batch=2, n_q_heads=hq, n_kv_heads=hkv,
                          q_len=q_len, tail_len=q_len + 40, seed=62)
    wl = synth.make_workload(cfg, variant="sharp", tail_len=[q_len + 40, q_len])
    out, lse = run_hip(wl, path="chunk", ld_extra=8)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)
