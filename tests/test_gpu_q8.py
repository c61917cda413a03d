"""GPU parity of 8-bit token-factor storage (MILO_BF16_Q8): the quantise
kernel's codes, scales and biases bit-exact against the oracle's fp32
quantisation, and the decode path over the 8-bit pool against the fp64
oracle on the dequantized factors."""
import numpy as np
import pytest

import oracle
import synth
from oracle import quant
from tests.gpu_util import compare, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def device_caches(wl, **packkw):
    import rank_attention_amd as ra
    pc = ra.pack(wl, **packkw)
    dc = ra.DeviceCache(pc, scale=wl.scale)
    note(f"q8 cfg={wl.cfg.name} variant={wl.variant} B={wl.batch} Hq={wl.cfg.n_q_heads} "
         f"Hkv={wl.cfg.n_kv_heads} d={wl.cfg.head_dim} max_blocks={pc.max_blocks} tail_cap={pc.k_tail.shape[2]}")
    return dc, dc.quantized()


def run_q8(wl, repeat=1, plan=True, **packkw):
    import torch
    _, qc = device_caches(wl, plan=plan, **packkw)
    outs = []
    for _ in range(repeat):
        out, lse = qc.decode()
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)))
    return outs if repeat > 1 else outs[0]


def parse_q8(pool: np.ndarray, desc, n_kv_heads: int, d: int):
    """Per block and KV head: (n_tok, key codes [rank_k][n_tok] (stored
    token-major), W bits, value codes [rank_v][ld_tok] (stored in 64-token
    tiles), W' bits, (a, b) rows) read from the 8-bit pool by the layout the
    header states."""
    out = []
    for blk in desc:
        off, T, ld, r, rv = (int(blk[k]) for k in ("off", "n_tok", "ld_tok", "rank_k", "rank_v"))
        rk16 = (r + 15) // 16 * 16
        head = T * rk16 + rv * ld + 2 * (r + rv) * d + (8 * (r + rv) + 15) // 16 * 16
        heads = []
        for g in range(n_kv_heads):
            o = off + g * head
            ku = pool[o:o + T * rk16].reshape(T, rk16); o += T * rk16
            assert np.all(ku[:, r:] == 0), "key code padding not 0"
            ck = np.ascontiguousarray(ku[:, :r].T)
            w = pool[o:o + 2 * r * d].view(np.uint16).reshape(r, d); o += 2 * r * d
            # value codes in 64-token tiles [ld / 64][rv][64]
            cv = pool[o:o + rv * ld].reshape(ld // 64, rv, 64).transpose(1, 0, 2).reshape(rv, ld); o += rv * ld
            wp = pool[o:o + 2 * rv * d].view(np.uint16).reshape(rv, d); o += 2 * rv * d
            sb = pool[o:o + 8 * (r + rv)].view(np.float32).reshape(r + rv, 2)
            heads.append((T, ck, w, cv, wp, sb))
        out.append(heads)
    return out


# --------------------------------------------------------------------------
# quantise kernel: bit-exact codes, scales and biases
# --------------------------------------------------------------------------
def _check_quantised(wl):
    import torch
    _, qc = device_caches(wl)
    torch.cuda.synchronize()
    pool = qc.pool.cpu().numpy()
    flat = [b for s in wl.blocks for b in s]
    parsed = parse_q8(pool, qc.blocks_host, wl.cfg.n_kv_heads, wl.cfg.head_dim)
    for bi, (blk, heads) in enumerate(zip(flat, parsed)):
        for g, (T, ck, w, cv, wp, sb) in enumerate(heads):
            for X, codes, rows in ((blk.ut[g], ck, sb[:blk.rank_k]), (blk.upt[g], cv, sb[blk.rank_k:])):
                c, a, b = quant.quantize_rows(synth.gen.bf16_bits_to_f32(X))
                assert np.array_equal(codes[:, :T], c), f"block {bi} head {g}: codes differ"
                assert np.all(codes[:, T:] == 0), f"block {bi} head {g}: padding codes not 0"
                assert np.array_equal(rows[:, 0], a), f"block {bi} head {g}: scales differ"
                assert np.array_equal(rows[:, 1], b), f"block {bi} head {g}: biases differ"
            assert np.array_equal(w, blk.w[g]) and np.array_equal(wp, blk.wp[g])


def test_quantise_bit_exact_seeded():
    for cfg in (synth.get_config("qwen05b_16k").with_(batch=2, n_blocks=3),
                synth.get_config("qwen7b_64k").with_(batch=1, n_blocks=4)):
        _check_quantised(synth.make_workload(cfg, variant="sharp"))


def test_quantise_bit_exact_edges():
    # ragged and empty blocks, zero and full ranks, constant and two-valued rows
    cfg = synth.get_config("qwen7b_64k").with_(name="q8_edges", batch=1, n_q_heads=14, n_kv_heads=2,
                                               ranks=synth.configs.RankDist("list", values=(128, 0, 1, 5, 64, 3)),
                                               v_rank_equals_k=False, seed=21)
    toks = [[37, 0, 1, 1024, 1000, 17]]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[6], tokens=toks)
    blk = wl.blocks[0][4]
    blk.ut[0, 0, :] = synth.gen.f32_to_bf16_bits(np.full(blk.n_tok, 1.5, np.float32))        # constant row
    blk.upt[1, 2, :] = synth.gen.f32_to_bf16_bits(np.where(np.arange(blk.n_tok) % 2, 3.0, -1.0).astype(np.float32))
    _check_quantised(wl)


# --------------------------------------------------------------------------
# decode over the 8-bit pool against the oracle on dequantized factors
# --------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_decode_q8_qwen05b_16k_full(variant):
    wl = synth.make_workload(synth.get_config("qwen05b_16k"), variant=variant)
    out, lse = run_q8(wl)
    ref_o, ref_l = quant.attend_q8(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=(variant == "sharp"), name=f"q8 qwen05b_16k/{variant}")


@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_decode_q8_qwen7b_64k_sampled(variant):
    """The full 64k workload on the GPU; the oracle on two whole sequences."""
    cfg = synth.get_config("qwen7b_64k")
    wl = synth.make_workload(cfg, variant=variant)
    out, lse = run_q8(wl)
    seqs = [0, cfg.batch - 1]
    ref_o, ref_l = quant.attend_q8(wl, seq_index=seqs)
    compare(out[seqs], lse[seqs], ref_o, ref_l, sharp_gates=(variant == "sharp"), name=f"q8 qwen7b_64k/{variant}")


def test_decode_q8_qwen7b_128k_sampled():
    """The largest workload (bimodal ranks: both rank classes of the kernel);
    the oracle on two whole sequences."""
    cfg = synth.get_config("qwen7b_128k")
    wl = synth.make_workload(cfg, variant="sharp")
    out, lse = run_q8(wl)
    seqs = [0, 17]
    ref_o, ref_l = quant.attend_q8(wl, seq_index=seqs)
    compare(out[seqs], lse[seqs], ref_o, ref_l, sharp_gates=True, name="q8 qwen7b_128k/sharp")


RAGGED = [(128, 7, 1), (128, 8, 1), (128, 10, 2), (64, 12, 4), (64, 3, 3), (128, 12, 2), (128, 6, 2),
          (64, 14, 2), (128, 4, 2), (64, 16, 2), (64, 8, 2)]


@pytest.mark.parametrize("d,hq,hkv", RAGGED)
def test_decode_q8_ragged_shapes(d, hq, hkv):
    base = synth.get_config("qwen05b_16k")
    cfg = base.with_(name=f"q8_ragged_{d}_{hq}_{hkv}", batch=4, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                     dtype="bf16", tail_len=70, ranks=synth.configs.RankDist("uniform", lo=0, hi=d), seed=11)
    toks = [[1, 37, 1024, 2049, 8], [], [511, 7], [3000]]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[len(t) for t in toks], tokens=toks,
                             tail_len=[70, 0, 1, 33])
    out, lse = run_q8(wl, shuffle_pool=3, max_blocks=6)
    ref_o, ref_l = quant.attend_q8(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)
    assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))


def test_decode_q8_extreme_ranks_and_constant_rows():
    cfg = synth.get_config("qwen7b_64k").with_(name="q8_rank_extremes", batch=2, n_blocks=4,
                                               ranks=synth.configs.RankDist("list", values=(128, 1, 0, 127)),
                                               v_rank_equals_k=False, seed=12)
    wl = synth.make_workload(cfg, variant="sharp", tail_len=[256, 13])
    blk = wl.blocks[1][0]
    blk.ut[2, 5, :] = synth.gen.f32_to_bf16_bits(np.full(blk.n_tok, -0.75, np.float32))
    blk.upt[0, 9, :] = synth.gen.f32_to_bf16_bits(np.full(blk.n_tok, 2.0, np.float32))
    out, lse = run_q8(wl)
    ref_o, ref_l = quant.attend_q8(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name="q8_rank_extremes")


def test_decode_q8_grid_factors_match_the_unquantised_oracle():
    """Factors already on a per-row 256-level grid quantise exactly: the 8-bit
    path then meets the plain oracle at the same gate."""
    cfg = synth.get_config("qwen7b_64k").with_(name="q8_grid", batch=2, n_blocks=3, seed=13)
    wl = synth.make_workload(cfg, variant="sharp")
    rng = np.random.default_rng(5)
    for seq in wl.blocks:
        for blk in seq:
            for arr in (blk.ut, blk.upt):
                for g in range(arr.shape[0]):
                    k = rng.integers(0, 256, size=arr.shape[1:])
                    k[:, 0], k[:, -1] = 0, 255
                    step = 2.0 ** rng.integers(-7, -4, size=(arr.shape[1], 1))
                    x = (-128 * step + step * k).astype(np.float32)
                    arr[g] = synth.gen.f32_to_bf16_bits(x)
    out, lse = run_q8(wl)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name="q8_grid")


def test_decode_q8_schedule_and_determinism():
    cfg = synth.get_config("qwen7b_64k").with_(batch=3, n_blocks=6)
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[6, 1, 4], tail_len=[256, 3, 0])
    (o1, l1), (o2, l2) = run_q8(wl, repeat=2, plan=True)
    o3, l3 = run_q8(wl, plan=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_validate_q8_tables():
    import torch
    wl = synth.make_workload(synth.get_config("qwen05b_16k").with_(batch=2, n_blocks=3), variant="base")
    _, qc = device_caches(wl)
    assert qc.validate() is None
    bad = qc.blocks_host.copy()
    bad["off"][1] += 8                          # a multiple of 8 but not of 16
    qc.blocks = torch.from_numpy(bad.view(np.uint8).copy()).to(qc.pool.device)
    assert qc.validate() == ("offset", 1)
    bad = qc.blocks_host.copy()
    bad["off"][2] = qc.pool.numel() - 16        # factors run past the end of the pool
    qc.blocks = torch.from_numpy(bad.view(np.uint8).copy()).to(qc.pool.device)
    assert qc.validate() == ("pool_bounds", 2)
