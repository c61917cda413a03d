"""Host-side packing of logical factors into the pool layout of milo_attn.h."""
import numpy as np

import rank_attention_amd as ra
import synth


def unpack_block(pc, k, g):
    b = pc.blocks[k]
    off, T, ld, rk, rv = (int(b[f]) for f in ("off", "n_tok", "ld_tok", "rank_k", "rank_v"))
    d = pc.head_dim
    base = off + g * (rk + rv) * (ld + d)
    ut = pc.pool[base:base + rk * ld].reshape(rk, ld)
    w = pc.pool[base + rk * ld: base + rk * ld + rk * d].reshape(rk, d)
    o = base + rk * (ld + d)
    upt = pc.pool[o:o + rv * ld].reshape(rv, ld)
    wp = pc.pool[o + rv * ld: o + rv * ld + rv * d].reshape(rv, d)
    return ut, w, upt, wp, T


def test_pool_roundtrip_and_poison():
    cfg = synth.get_config("qwen05b_16k").with_(batch=3, n_blocks=3)
    tokens = [[37, 512, 8], [1, 16, 100], [64, 65, 7]]
    wl = synth.make_workload(cfg, tokens=tokens, n_blocks=[3, 3, 3], tail_len=[128, 0, 5])
    pc = ra.pack(wl, shuffle_pool=5)
    assert pc.pool.dtype == np.uint16
    assert list(pc.seq_blocks) == [0, 3, 6, 9]
    assert np.all(pc.blocks["off"] % 8 == 0) and np.all(pc.blocks["ld_tok"] % 8 == 0)
    k = 0
    for i in range(3):
        for b in wl.blocks[i]:
            for g in range(cfg.n_kv_heads):
                ut, w, upt, wp, T = unpack_block(pc, k, g)
                np.testing.assert_array_equal(ut[:, :T], b.ut[g])
                np.testing.assert_array_equal(w, b.w[g])
                np.testing.assert_array_equal(upt[:, :T], b.upt[g])
                np.testing.assert_array_equal(wp, b.wp[g])
                assert np.all(ut[:, T:] == 0x7FC0) and np.all(upt[:, T:] == 0x7FC0)
            k += 1
    # blocks do not overlap and the gaps hold NaN
    spans = sorted((int(b["off"]), int(b["off"]) + cfg.n_kv_heads * (int(b["rank_k"]) + int(b["rank_v"])) *
                    (int(b["ld_tok"]) + cfg.head_dim)) for b in pc.blocks)
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 < b0
        assert np.all(pc.pool[a1:b0] == 0x7FC0)
    # tail entries beyond tail_len are poisoned
    assert np.all(pc.k_tail[1] == 0x7FC0)
    assert np.all(pc.v_tail[2, :, 5:] == 0x7FC0)
    np.testing.assert_array_equal(pc.k_tail[2, :, :5], wl.k_tail[2, :, :5])


def test_f32_pool():
    wl = synth.make_workload(synth.get_config("tiny"))
    pc = ra.pack(wl)
    assert pc.pool.dtype == np.float32
    ut, w, upt, wp, T = unpack_block(pc, 3, 0)
    np.testing.assert_array_equal(ut[:, :T], wl.blocks[0][3].ut[0])
    assert pc.max_blocks == 4


def test_decode_plan_tails_first_then_largest_first():
    cfg = synth.get_config("qwen7b_64k").with_(batch=3, n_blocks=5)
    wl = synth.make_workload(cfg, n_blocks=[5, 2, 0], tail_len=[256, 0, 17])
    pc = ra.pack(wl, max_blocks=6)
    order = pc.unit_order
    S = pc.max_blocks + 1
    units = cfg.batch * cfg.n_kv_heads * S
    assert sorted(order.tolist()) == list(range(units))
    d = cfg.head_dim

    def key(u):
        """(class, -cost): non-empty tails, then blocks by size, then empty slots."""
        i, rest = divmod(u, cfg.n_kv_heads * S)
        g, slot = divmod(rest, S)
        nb = int(pc.seq_blocks[i + 1] - pc.seq_blocks[i])
        if slot == pc.max_blocks:
            L = int(pc.tail_len[i])
            return (0, -2 * L * d) if L > 0 else (2, 0)
        if slot >= nb:
            return (2, 0)
        b = pc.blocks[pc.seq_blocks[i] + slot]
        return (1, -(int(b["rank_k"]) + int(b["rank_v"])) * (int(b["n_tok"]) + d))

    keys = [key(int(u)) for u in order]
    assert keys == sorted(keys)
    n_tails = sum(1 for k in keys if k[0] == 0)
    assert n_tails == 2 * cfg.n_kv_heads            # sequences 0 and 2 have a tail
    # ties keep the natural order
    for a, b in zip(order, order[1:]):
        if key(int(a)) == key(int(b)):
            assert a < b
