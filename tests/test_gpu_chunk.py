"""GPU parity of the chunked-query path (MFMA kernel through the C ABI)
against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import compare, note, run_hip

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


def test_chunk_qwen32b_sampled():
    """Full 32B-like chunk workload on the GPU; oracle on sampled query rows."""
    cfg = synth.get_config("qwen32b_chunk")
    wl = synth.make_workload(cfg)
    out, lse = run_hip(wl, path="chunk")
    seqs = [0, cfg.batch - 1]
    js = [0, 1, 77, cfg.q_len - 2, cfg.q_len - 1]
    sel = [(si, j, h) for si in range(len(seqs)) for j in js for h in range(cfg.n_q_heads)]
    note(f"oracle on {len(sel)} sampled rows")
    ref_o, ref_l = oracle.attend(wl, seq_index=seqs, sel=sel)
    rows_gpu = [(seqs[si], j, h) for (si, j, h) in sel]
    idx_g = tuple(np.array(rows_gpu).T)
    idx_r = tuple(np.array(sel).T)
    compare(out[idx_g], lse[idx_g], ref_o[idx_r], ref_l[idx_r], name="qwen32b_chunk")
