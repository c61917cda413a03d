"""GPU parity of the matrix-core kernel at head_dim 64 (Qwen2.5-0.5B-like
layers): chunked prefill, the shared pre-encoded context, and decode with
group sizes above 8, all against the fp64 oracle.  The kernel's tiles are
128 wide; W, W', q and the tail rows are zero-padded to 128 on load."""
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


def d64_cfg(**kw):
    """The 0.5B-like layer (14/2 heads, d 64) on the chunked path."""
    base = synth.get_config("qwen05b_16k").with_(name="chunk_d64", path="chunk", batch=2, q_len=48,
                                                  tail_len=100, n_blocks=6,
                                                  ranks=synth.configs.RankDist("uniform", lo=0, hi=64),
                                                  seed=71)
    return base.with_(**kw)


@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_chunk_d64_small(variant):
    cfg = d64_cfg()
    wl = synth.make_workload(cfg, variant=variant)
    out, lse = run_hip(wl, path="chunk")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=(variant == "sharp"), name=f"chunk_d64/{variant}")


def test_chunk_d64_ranges_of_several_blocks():
    """Enough short blocks that each block range holds two or three of them
    (the cross-block W / tile pipeline), ragged lengths, empty and one-token
    blocks, ranks 0..64, NaN row padding, a shuffled pool."""
    from tests.gpu_util import chunk_ranges
    import rank_attention_amd as ra
    rng = np.random.default_rng(5)
    nb = 160
    toks = [[int(rng.choice([0, 1, 63, 64, 65, 128])) if rng.random() < 0.3 else int(rng.integers(2, 200))
             for _ in range(nb)] for _ in range(2)]
    cfg = d64_cfg(name="chunk_d64_ranges", n_blocks=nb, q_len=64, tail_len=64 + 90)
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[nb, nb], tokens=toks, tail_len=[64 + 90, 64])
    dc = ra.DeviceCache(ra.pack(wl, shuffle_pool=9, ld_extra=16), scale=wl.scale)
    nr = chunk_ranges(dc)
    assert nb / nr >= 2, f"{nr} ranges: fewer than two blocks per range"
    note(f"chunk_d64_ranges: {nr} block ranges of {-(-nb // nr)} blocks")
    import torch
    out, lse = dc.chunk()
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)


@pytest.mark.parametrize("hq,hkv,q_len", [(14, 2, 33), (16, 1, 20), (3, 3, 70)])
def test_chunk_d64_ragged(hq, hkv, q_len):
    cfg = d64_cfg(name=f"chunk_d64_ragged_{hq}_{hkv}_{q_len}", batch=3, n_q_heads=hq, n_kv_heads=hkv,
                  q_len=q_len, tail_len=q_len + 9, seed=72)
    toks = [[37, 1000, 64, 65], [], [1, 130, 2049]]
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[len(t) for t in toks], tokens=toks,
                             tail_len=[q_len + 9, q_len, q_len + 100])
    out, lse = run_hip(wl, path="chunk", shuffle_pool=5, max_blocks=5, ld_extra=8)
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)


def _shared(wl):
    wl.blocks = [wl.blocks[0] for _ in range(wl.batch)]
    return wl


@pytest.mark.parametrize("variant", ["base", "sharp"])
def test_shared_d64(variant):
    """The whole 0.5B-like batch (8 queries) over one shared 16k context."""
    cfg = synth.get_config("qwen05b_16k")
    wl = _shared(synth.make_workload(cfg, variant=variant))
    out, lse = run_hip(wl, path="shared")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=(variant == "sharp"), name=f"shared_d64/{variant}")


def test_shared_d64_matches_decode():
    cfg = synth.get_config("qwen05b_16k").with_(name="shared_d64_vs_decode", batch=5, n_blocks=6)
    wl = _shared(synth.make_workload(cfg, variant="sharp"))
    os_, ls = run_hip(wl, path="shared")
    od, ld = run_hip(wl, path="decode")
    compare(os_, ls, od, ld, sharp_gates=True, name="shared_d64_vs_decode")


@pytest.mark.parametrize("hq,hkv", [(32, 2), (12, 1)])
def test_decode_d64_large_group(hq, hkv):
    """Group sizes above 8 at head_dim 64: decode runs on the matrix-core kernel."""
    cfg = synth.get_config("qwen05b_16k").with_(name=f"decode_d64_g{hq // hkv}", batch=3, n_q_heads=hq,
                                                n_kv_heads=hkv, n_blocks=7, seed=73)
    wl = synth.make_workload(cfg, variant="sharp", tail_len=[128, 0, 77])
    out, lse = run_hip(wl, path="decode")
    ref_o, ref_l = oracle.attend(wl)
    compare(out, lse, ref_o, ref_l, sharp_gates=True, name=cfg.name)
