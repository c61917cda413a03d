"""GPU parity of KIVI-style token-factor storage (MILO_BF16_KV4 and
MILO_BF16_KV2): the quantise kernel's codes, scales and biases bit-exact
against the oracle's fp32 quantisation (oracle/kivi.py), and the decode path
over the quantised pool against the fp64 oracle on the dequantized factors."""
import numpy as np
import pytest

import oracle
import synth
from oracle import kivi
from tests.gpu_util import compare, note

pytestmark = pytest.mark.gpu

BITS = [4, 2]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def device_caches(wl, bits, **packkw):
    import rank_attention_amd as ra
    pc = ra.pack(wl, **packkw)
    dc = ra.DeviceCache(pc, scale=wl.scale)
    note(f"kivi{bits} cfg={wl.cfg.name} variant={wl.variant} B={wl.batch} Hq={wl.cfg.n_q_heads} "
         f"Hkv={wl.cfg.n_kv_heads} d={wl.cfg.head_dim} max_blocks={pc.max_blocks} tail_cap={pc.k_tail.shape[2]}")
    return dc, dc.kivi(bits)


def run_kivi(wl, bits, repeat=1, plan=True, **packkw):
    import torch
    _, qc = device_caches(wl, bits, plan=plan, **packkw)
    outs = []
    for _ in range(repeat):
        out, lse = qc.decode()
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)))
    return outs if repeat > 1 else outs[0]


# --------------------------------------------------------------------------
# the pool, read back by the layout milo_attn.h states
# --------------------------------------------------------------------------
def _shift(bits, u, i):
    """Bit position of code i (0..7) of 8-code word u (2-bit words pair up in a dword)."""
    i = np.asarray(i)
    if bits == 4:
        return 4 * np.where(i < 4, 2 * i, 2 * (i - 4) + 1)
    P = 4 * u + i // 2
    return 8 * (2 * (P % 2) + i % 2) + 2 * (P // 2)


def parse_kivi(pool: np.ndarray, desc, n_kv_heads: int, d: int, bits: int):
    """Per block and KV head a dict: header (amax_k, amax_v), key scales and
    biases [nch][8 ng8] (uint16 bits), key codes [64 nch][8 ng8], value
    scales and biases [64 nch][ngv] (uint16 bits), value codes
    [64 nch][16 ntv], W and W' bits."""
    out = []
    i8 = np.arange(8)
    for blk in desc:
        off, T, ld, r, rv = (int(blk[k]) for k in ("off", "n_tok", "ld_tok", "rank_k", "rank_v"))
        assert ld % 64 == 0 and ld >= T and off % 16 == 0
        nch, ng8, ngv, ntv = ld // 64, -(-r // 8), -(-rv // 32), -(-rv // 16)
        H = 16 + nch * (32 * ng8 + 64 * bits * ng8 + 256 * ngv + 128 * bits * ntv) + 2 * d * (r + rv)
        heads = []
        for g in range(n_kv_heads):
            o = off + g * H
            take = lambda n: pool[o:o + n]
            h = {"amax": take(16)[:8].view(np.float32).copy(), "pad": take(16)[8:].copy()}; o += 16
            h["ka"] = take(nch * 16 * ng8).view(np.uint16).reshape(nch, 8 * ng8); o += nch * 16 * ng8
            h["kb"] = take(nch * 16 * ng8).view(np.uint16).reshape(nch, 8 * ng8); o += nch * 16 * ng8
            kc = take(nch * 64 * bits * ng8).view(np.uint32); o += nch * 64 * bits * ng8
            va = take(nch * ngv * 128).view(np.uint16).reshape(nch, ngv, 64); o += nch * ngv * 128
            vb = take(nch * ngv * 128).view(np.uint16).reshape(nch, ngv, 64); o += nch * ngv * 128
            vc = take(nch * 128 * bits * ntv).view(np.uint32); o += nch * 128 * bits * ntv
            h["w"] = take(2 * r * d).view(np.uint16).reshape(r, d); o += 2 * r * d
            h["wp"] = take(2 * rv * d).view(np.uint16).reshape(rv, d); o += 2 * rv * d
            # key codes: word (g8, col, m) = ranks 8 g8 + i of token 16 (col / 4) + 4 m + col % 4
            ck = np.zeros((64 * nch, 8 * ng8), np.uint8)
            kw = kc.reshape(nch, ng8, 16, 4 if bits == 4 else 2)
            for c in range(nch):
                for g8 in range(ng8):
                    for col in range(16):
                        for m in range(4):
                            w = kw[c, g8, col, m] if bits == 4 else kw[c, g8, col, m // 2]
                            u = 0 if bits == 4 else m % 2
                            tok = 64 * c + 16 * (col // 4) + 4 * m + col % 4
                            ck[tok, 8 * g8:8 * g8 + 8] = (w >> _shift(bits, u, i8)) & ((1 << bits) - 1)
            # value codes: tile kt, lane l = rank 16 kt + l % 16 at tokens 16 (l / 16) + 8 s + i
            cv = np.zeros((64 * nch, 16 * ntv), np.uint8)
            vw = vc.reshape(nch, ntv, 64, 2) if bits == 4 else vc.reshape(nch, ntv, 64, 1)
            for c in range(nch):
                for kt in range(ntv):
                    for l in range(64):
                        for s in range(2):
                            w = vw[c, kt, l, s] if bits == 4 else vw[c, kt, l, 0]
                            u = 0 if bits == 4 else s
                            t0 = 64 * c + 16 * (l // 16) + 8 * s
                            cv[t0:t0 + 8, 16 * kt + l % 16] = (w >> _shift(bits, u, i8)) & ((1 << bits) - 1)
            h["ck"], h["cv"] = ck, cv
            h["va"] = va.transpose(0, 2, 1).reshape(64 * nch, ngv)
            h["vb"] = vb.transpose(0, 2, 1).reshape(64 * nch, ngv)
            heads.append(h)
        out.append(heads)
    return out


def _check_quantised(wl, bits):
    import torch
    _, qc = device_caches(wl, bits)
    torch.cuda.synchronize()
    pool = qc.pool.cpu().numpy()
    flat = [b for s in wl.blocks for b in s]
    parsed = parse_kivi(pool, qc.blocks_host, wl.cfg.n_kv_heads, wl.cfg.head_dim, bits)
    for bi, (blk, heads) in enumerate(zip(flat, parsed)):
        T, r, rv = blk.n_tok, blk.rank_k, blk.rank_v
        for g, h in enumerate(heads):
            where = f"block {bi} head {g}"
            U = synth.gen.bf16_bits_to_f32(blk.ut[g]).T[:T]         # [T][r]
            Up = synth.gen.bf16_bits_to_f32(blk.upt[g]).T[:T]       # [T][r']
            ck, ka, kb = kivi.quantize_keys(U, bits)
            cv, va, vb = kivi.quantize_values(Up, bits)
            assert np.array_equal(h["ck"][:T, :r], ck), f"{where}: key codes differ"
            assert np.all(h["ck"][T:] == 0) and np.all(h["ck"][:, r:] == 0), f"{where}: key padding not 0"
            assert np.array_equal(h["ka"][:, :r], ka.view(np.uint16)), f"{where}: key scales differ"
            assert np.array_equal(h["kb"][:, :r], kb.view(np.uint16)), f"{where}: key biases differ"
            assert np.all(h["ka"][:, r:] == 0) and np.all(h["kb"][:, r:] == 0), f"{where}: key scale padding"
            assert np.array_equal(h["cv"][:T, :rv], cv), f"{where}: value codes differ"
            assert np.all(h["cv"][T:] == 0) and np.all(h["cv"][:, rv:] == 0), f"{where}: value padding not 0"
            assert np.array_equal(h["va"][:T], va.view(np.uint16)), f"{where}: value scales differ"
            assert np.array_equal(h["vb"][:T], vb.view(np.uint16)), f"{where}: value biases differ"
            assert np.all(h["va"][T:] == 0) and np.all(h["vb"][T:] == 0), f"{where}: value scale padding"
            amax_k = float(ka.astype(np.float32).max()) if ka.size else 0.0
            amax_v = float(va.astype(np.float32).max()) if va.size else 0.0
            assert h["amax"][0] == amax_k and h["amax"][1] == amax_v, f"{where}: header {h['amax']}"
            assert np.all(h["pad"] == 0)
            assert np.array_equal(h["w"], blk.w[g]) and np.array_equal(h["wp"], blk.wp[g]), f"{where}: W differs"


@pytest.mark.parametrize("bits", BITS)
def test_kivi_quantise_bit_exact_seeded(bits):
    for cfg in (synth.get_config("qwen05b_16k").with_(batch=2, n_blocks=3),
                synth.get_config("qwen7b_64k").with_(batch=1, n_blocks=3)):
        _check_quantised(synth.make_workload(cfg, variant="sharp"), bits)


@pytest.mark.parametrize("bits", BITS)
def test_kivi_quantise_bit_exact_edges(bits):
    # ragged and empty blocks, zero and full ranks, rank counts off the 8/16/32 grids, constant rows
    cfg = synth.get_config("qwen7b_64k").with_(name="kivi_edges", batch=1, n_q_heads=14, n_kv_heads=2,
                                               ranks=synth.configs.RankDist("list", values=(128, 0, 1, 5, 64, 3, 33)),
                                               v_rank_equals_k=False, seed=21)
    toks = [[37, 0, 1, 1024, 1000, 17, 65]]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[7], tokens=toks)
    blk = wl.blocks[0][4]
    blk.ut[0, 0, :] = synth.gen.f32_to_bf16_bits(np.full(blk.n_tok, 1.5, np.float32))        # constant key group
    blk.upt[1, :, 5] = synth.gen.f32_to_bf16_bits(np.full(blk.upt.shape[1], -2.0, np.float32))  # constant value token
    _check_quantised(wl, bits)


# --------------------------------------------------------------------------
# decode over the KIVI-style pool against the oracle on dequantized factors
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_decode_kivi_qwen05b_16k_full(bits, variant):
    wl = synth.make_workload(synth.get_config("qwen05b_16k"), variant=variant)
    out, lse = run_kivi(wl, bits)
    ref_o, ref_l = kivi.attend_kivi(wl, bits)
    compare(out, lse, ref_o, ref_l, sharp_gates=(variant == "sharp"), name=f"kivi{bits} qwen05b_16k/{variant}")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_decode_kivi_qwen7b_64k_sampled(bits, variant):
    """The full 64k workload on the GPU; the oracle on two whole sequences."""
    cfg = synth.get_config("qwen7b_64k")
    wl = synth.make_workload(cfg, variant=variant)
    out, lse = run_kivi(wl, bits)
    seqs = [0, cfg.batch - 1]
    ref_o, ref_l = kivi.attend_kivi(wl, bits, seq_index=seqs)
    compare(out[seqs], lse[seqs], ref_o, ref_l, sharp_gates=(variant == "sharp"),
            name=f"kivi{bits} qwen7b_64k/{variant}")


@pytest.mark.parametrize("bits", BITS)
def test_decode_kivi_qwen7b_128k_sampled(bits):
    """2048-token blocks (two tiles of chunk constants) and bimodal ranks
    (both rank classes of the kernel); the oracle on two whole sequences."""
    cfg = synth.get_config("qwen7b_128k")
    wl = synth.make_workload(cfg, variant="sharp")
    out, lse = run_kivi(wl, bits)
    seqs = [0, 17]
    ref_o, ref_l = kivi.attend_kivi(wl, bits, seq_index=seqs)
    compare(out[seqs], lse[seqs], ref_o, ref_l, sharp_gates=True, name=f"kivi{bits} qwen7b_128k/sharp")


RAGGED = [(128, 7, 1), (128, 8, 1), (64, 12, 4), (64, 3, 3), (128, 6, 2), (64, 8, 2), (128, 4, 2)]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("d,hq,hkv", RAGGED)
def test_decode_kivi_ragged_shapes(bits, d, hq, hkv):
    base = synth.get_config("qwen05b_16k")
    cfg = base.with_(name=f"kivi_ragged_{d}_{hq}_{hkv}", batch=4, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                     dtype="bf16", tail_len=70, ranks=synth.configs.RankDist("uniform", lo=0, hi=d),
                     v_rank_equals_k=False, seed=11)
    toks = [[1, 37, 1024, 2049, 8], [], [511, 7], [3000]]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[len(t) for t in toks], tokens=toks,
                             tail_len=[70, 0, 1, 33])
    out, lse = run_kivi(wl, bits, shuffle_pool=3, max_blocks=6)
    ref_o, ref_l = kivi.attend_kivi(wl, bits)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=f"kivi{bits} {cfg.name}")
    assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("bits", BITS)
def test_decode_kivi_extreme_ranks_and_constant_groups(bits):
    cfg = synth.get_config("qwen7b_64k").with_(name="kivi_rank_extremes", batch=2, n_blocks=5,
                                               ranks=synth.configs.RankDist("list", values=(128, 1, 0, 127, 65)),
                                               v_rank_equals_k=False, seed=12)
    wl = synth.make_workload(cfg, variant="sharp", tail_len=[256, 13])
    blk = wl.blocks[1][0]
    blk.ut[2, 5, :] = synth.gen.f32_to_bf16_bits(np.full(blk.n_tok, -0.75, np.float32))
    blk.upt[0, :, 9] = synth.gen.f32_to_bf16_bits(np.full(blk.upt.shape[1], 2.0, np.float32))
    out, lse = run_kivi(wl, bits)
    ref_o, ref_l = kivi.attend_kivi(wl, bits)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=f"kivi{bits} rank_extremes")


@pytest.mark.parametrize("bits", BITS)
def test_decode_kivi_block_above_8192_tokens(bits):
    """A block of 9000 tokens: 141 chunks, so the chunk constants are made
    again after the first 128."""
    cfg = synth.get_config("qwen7b_64k").with_(name="kivi_long", batch=1, n_q_heads=8, n_kv_heads=2,
                                               ranks=synth.configs.RankDist("list", values=(96, 40)),
                                               v_rank_equals_k=False, seed=14)
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[2], tokens=[[9000, 300]], tail_len=[5])
    out, lse = run_kivi(wl, bits)
    ref_o, ref_l = kivi.attend_kivi(wl, bits)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=f"kivi{bits} long block")


@pytest.mark.parametrize("bits", BITS)
def test_decode_kivi_grid_factors_match_the_unquantised_oracle(bits):
    """Factors already on the KIVI grids (per rank component and 64-token
    chunk for U, per token and 32 ranks for U') quantise exactly: the path
    then meets the plain oracle at the same gate."""
    L = 2 ** bits - 1
    cfg = synth.get_config("qwen7b_64k").with_(name="kivi_grid", batch=2, n_blocks=3, seed=13)
    wl = synth.make_workload(cfg, variant="sharp")
    rng = np.random.default_rng(5)
    for seq in wl.blocks:
        for blk in seq:
            T = blk.n_tok
            for g in range(blk.ut.shape[0]):
                ut = np.zeros(blk.ut[g].shape, np.float32)
                for j in range(0, T, 64):
                    n = min(64, T - j)
                    k = rng.integers(0, L + 1, size=(ut.shape[0], n))
                    k[:, 0], k[:, -1] = 0, L
                    step = 2.0 ** rng.integers(-5, -2, size=(ut.shape[0], 1))
                    ut[:, j:j + n] = -step * (L // 2) + step * k
                upt = np.zeros(blk.upt[g].shape, np.float32)
                for j in range(0, upt.shape[0], 32):
                    n = min(32, upt.shape[0] - j)
                    k = rng.integers(0, L + 1, size=(n, T))
                    k[0, :], k[-1, :] = 0, L
                    step = 2.0 ** rng.integers(-5, -2, size=(1, T))
                    upt[j:j + n] = -step * (L // 2) + step * k
                blk.ut[g] = synth.gen.f32_to_bf16_bits(ut)
                blk.upt[g] = synth.gen.f32_to_bf16_bits(upt)
    out, lse = run_kivi(wl, bits)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=f"kivi{bits} grid")


@pytest.mark.parametrize("bits", BITS)
def test_decode_kivi_schedule_and_determinism(bits):
    cfg = synth.get_config("qwen7b_64k").with_(batch=3, n_blocks=6)
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[6, 1, 4], tail_len=[256, 3, 0])
    (o1, l1), (o2, l2) = run_kivi(wl, bits, repeat=2, plan=True)
    o3, l3 = run_kivi(wl, bits, plan=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


@pytest.mark.parametrize("bits", BITS)
def test_validate_kivi_tables(bits):
    import torch
    wl = synth.make_workload(synth.get_config("qwen05b_16k").with_(batch=2, n_blocks=3), variant="base")
    _, qc = device_caches(wl, bits)
    assert qc.validate() is None
    bad = qc.blocks_host.copy()
    bad["off"][1] += 8                          # a multiple of 8 but not of 16
    qc.blocks = torch.from_numpy(bad.view(np.uint8).copy()).to(qc.pool.device)
    assert qc.validate() == ("offset", 1)
    bad = qc.blocks_host.copy()
    bad["off"][2] = qc.pool.numel() - 16        # factors run past the end of the pool
    qc.blocks = torch.from_numpy(bad.view(np.uint8).copy()).to(qc.pool.device)
    assert qc.validate() == ("pool_bounds", 2)
    # a KV head of 2^32 bytes or more (the decode kernel's table offsets
    # are 32-bit): rule 4, ahead of the pool bound it also breaks
    bad = qc.blocks_host.copy()
    bad["n_tok"][0] = bad["ld_tok"][0] = 2**31 - 64
    bad["rank_k"][0] = bad["rank_v"][0] = 64
    qc.blocks = torch.from_numpy(bad.view(np.uint8).copy()).to(qc.pool.device)
    assert qc.validate() == ("tokens", 0)
