"""GPU test of milo_attn_decode_noalloc, the decode entry point for callers
that cannot allocate (partials in the library's static device buffer): two
calls in a row, the second on a smaller input, each equal bit for bit to
milo_attn_decode (same kernels, same schedule) and within the parity gates
of the fp64 oracle; a call needing more than the static buffer is refused
before any HIP call."""
import numpy as np
import pytest

import oracle
import rank_attention_amd as ra
import synth
from tests.gpu_util import compare, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(wl):
    import torch
    dc = ra.DeviceCache(ra.pack(wl), scale=wl.scale)
    note(f"noalloc cfg={wl.cfg.name} B={wl.batch} blocks={[len(s) for s in wl.blocks]}")
    o_ref, l_ref = dc.decode()
    torch.cuda.synchronize()
    # preallocated outputs: the no-allocation call itself allocates nothing
    out = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    o_na, l_na = dc.decode_noalloc(out=out, lse=lse)
    torch.cuda.synchronize()
    assert o_na.data_ptr() == out.data_ptr() and l_na.data_ptr() == lse.data_ptr()
    return (o_ref.cpu().numpy(), l_ref.cpu().numpy()), (o_na.cpu().numpy(), l_na.cpu().numpy())


def test_noalloc_matches_decode_on_two_calls():
    big = synth.get_config("qwen7b_64k").with_(name="noalloc_big", batch=6, n_blocks=12)
    small = synth.get_config("qwen05b_16k").with_(name="noalloc_small", batch=2, n_blocks=3)
    for cfg in (big, small):          # the second call is smaller: stale partials must not leak in
        wl = synth.make_workload(cfg, variant="sharp")
        (o_ref, l_ref), (o_na, l_na) = _both(wl)
        assert np.array_equal(o_na, o_ref) and np.array_equal(l_na, l_ref), cfg.name
        ref_o, ref_l = oracle.attend(wl)
        compare(o_na.astype(np.float64), l_na.astype(np.float64), ref_o, ref_l, sharp_gates=True, name=cfg.name)
