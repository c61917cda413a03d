"""GPU parity of the shared-context decode path (one compressed context for
the whole batch, read once on the MFMA path; per-sequence tails) against the
fp64 oracle, which attends each sequence over its own copy of the shared
block list."""
import numpy as np
import pytest

import oracle
import rank_attention_amd as ra
import synth
from tests.gpu_util import compare, note, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def shared(wl):
    """Every sequence lists sequence 0's blocks (the oracle reads these lists;
    the shared path reads only sequence 0's)."""
    wl.blocks = [wl.blocks[0] for _ in range(wl.batch)]
    return wl


@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_shared_small(variant):
    cfg = synth.get_config("qwen7b_64k").with_(name="shared_small", batch=5, n_blocks=4)
    wl = shared(synth.make_workload(cfg, variant=variant))
    out, lse = run_hip(wl, path="shared")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=(variant == "sharp"), name=f"shared_small/{variant}")


def test_shared_matches_decode():
    """The regular decode path reads each sequence's own (identical) copy."""
    cfg = synth.get_config("qwen7b_64k").with_(name="shared_vs_decode", batch=6, n_blocks=5)
    wl = shared(synth.make_workload(cfg, variant="sharp"))
    os_, ls = run_hip(wl, path="shared")
    od, ld = run_hip(wl, path="decode")
    compare(os_, ls, od, ld, sharp_gates=True, name="shared_vs_decode")


@pytest.mark.parametrize("batch,hq,hkv", [(3, 15, 3), (40, 28, 4), (1, 8, 1), (19, 40, 8), (5, 32, 2), (9, 12, 1)])
def test_shared_ragged(batch, hq, hkv):
    """Odd row counts (batch * group not a multiple of 16, several 128-row
    tiles), group sizes up to 16, ragged tokens, ranks 0..128, empty and
    short tails, and 16 extra NaN padding elements per token-factor row."""
    cfg = synth.get_config("qwen7b_64k").with_(name=f"shared_ragged_{batch}_{hq}_{hkv}", batch=batch,
                                               n_q_heads=hq, n_kv_heads=hkv,
                                               ranks=synth.configs.RankDist("uniform", lo=0, hi=128),
                                               seed=31)
    toks = [[37, 1000, 64, 65, 130]] + [[8] for _ in range(batch - 1)]
    tails = [(7 * s) % 300 for s in range(batch)]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[len(t) for t in toks], tokens=toks,
                             tail_len=tails)
    wl = shared(wl)
    out, lse = run_hip(wl, path="shared", ld_extra=16)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)


def test_shared_empty_context_and_single_block():
    """No shared blocks (tails only), then one shared block and no tails."""
    cfg = synth.get_config("qwen7b_64k").with_(name="shared_edges", batch=4, n_blocks=1)
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[0, 0, 0, 0], tokens=[[], [], [], []],
                             tail_len=[5, 0, 256, 1])
    out, lse = run_hip(wl, path="shared")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, name="shared_no_blocks")
    wl = shared(synth.make_workload(cfg, variant="sharp", n_blocks=[1, 1, 1, 1], tokens=[[333]] * 4,
                                    tail_len=[0, 0, 0, 0]))
    out, lse = run_hip(wl, path="shared")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, name="shared_one_block")


def test_shared_qwen7b_64k_sampled():
    """Full 7B-like 64k shape with the context shared by all 16 sequences;
    oracle on sampled rows."""
    cfg = synth.get_config("qwen7b_64k").with_(name="qwen7b_64k_shared")
    wl = shared(synth.make_workload(cfg, variant="sharp"))
    out, lse = run_hip(wl, path="shared")
    seqs = [0, 7, cfg.batch - 1]
    sel = [(si, 0, h) for si in range(len(seqs)) for h in (0, 6, 13, 27)]
    note(f"oracle on {len(sel)} sampled rows")
    ref_o, ref_l = oracle.attend(wl, seq_index=seqs, sel=sel)
    rows_gpu = [(seqs[si], j, h) for (si, j, h) in sel]
    idx_g = tuple(np.array(rows_gpu).T)
    idx_r = tuple(np.array(sel).T)
    compare(out[idx_g], lse[idx_g], ref_o[idx_r], ref_l[idx_r], sharp_gates=True, name="qwen7b_64k_shared")
    # every row against the regular decode path over per-sequence copies
    od, ld = run_hip(wl, path="decode")
    compare(out, lse, od, ld, sharp_gates=True, name="qwen7b_64k_shared_vs_decode")


def test_shared_without_tails():
    """tail_cap 0: no tail tensors at all (NULL tail pointers)."""
    cfg = synth.get_config("qwen7b_64k").with_(name="shared_no_tail", batch=9, n_blocks=3, tail_len=0)
    wl = shared(synth.make_workload(cfg, variant="sharp"))
    assert ra.pack(wl).k_tail.shape[2] == 0
    out, lse = run_hip(wl, path="shared")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name="shared_no_tail")
