"""The attention entry points are asynchronous and allocate nothing, so they
can be captured into a HIP graph: each path is captured once (workspace,
out and lse allocated beforehand), replayed several times with eager work
and synchronisations between the replays, and every replay must equal the
eager result bit for bit (the kernels are deterministic for a fixed plan)."""
import numpy as np
import pytest

import rank_attention_amd as ra
import synth
from tests.gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _capture_and_replay(dc, path, fn_name):
    import ctypes
    import torch
    from rank_attention_amd import _lib
    lib = _lib.load()
    B, Q, Hq, d = (int(x) for x in dc.q.shape)
    out = torch.empty((B, Q, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Q, Hq), dtype=torch.float32, device="cuda")
    a = ra.make_args(*dc.tensors(), n_kv_heads=dc.n_kv_heads, scale=dc.scale, max_blocks=dc.max_blocks,
                     out=out, lse=lse, unit_order=dc.unit_order if path == ra.MILO_PATH_DECODE else None)
    need = lib.milo_attn_workspace_bytes(ctypes.byref(a), path)
    ws = torch.empty(int(need), dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), int(need)
    fn = getattr(lib, fn_name)

    def call():
        rc = fn(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, ra.status_str(rc)

    call()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        note(f"{fn_name} replay {rep}: scratch {float(scratch):.3f}")
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"{fn_name}: replay {rep} differs"


def test_decode_graph_replays():
    cfg = synth.get_config("qwen7b_64k").with_(batch=3, n_blocks=6)
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[6, 2, 5], tail_len=[256, 3, 0])
    _capture_and_replay(ra.DeviceCache(ra.pack(wl), scale=wl.scale), ra.MILO_PATH_DECODE, "milo_attn_decode")


def test_chunk_graph_replays():
    cfg = synth.get_config("qwen32b_chunk").with_(batch=2, n_q_heads=10, n_kv_heads=2, n_blocks=4, q_len=40,
                                                   tail_len=60)
    wl = synth.make_workload(cfg, variant="sharp")
    _capture_and_replay(ra.DeviceCache(ra.pack(wl), scale=wl.scale), ra.MILO_PATH_CHUNK, "milo_attn_chunk")


def test_shared_graph_replays():
    cfg = synth.get_config("qwen7b_64k").with_(batch=6, n_blocks=5)
    wl = synth.make_workload(cfg, variant="sharp")
    wl.blocks = [wl.blocks[0] for _ in range(wl.batch)]
    _capture_and_replay(ra.DeviceCache(ra.pack(wl), scale=wl.scale), ra.MILO_PATH_SHARED,
                        "milo_attn_decode_shared")


def test_q8_decode_graph_replays():
    cfg = synth.get_config("qwen7b_64k").with_(batch=3, n_blocks=6)
    wl = synth.make_workload(cfg, variant="sharp", n_blocks=[6, 2, 5], tail_len=[256, 3, 0])
    qc = ra.DeviceCache(ra.pack(wl), scale=wl.scale).quantized()
    _capture_and_replay(qc, ra.MILO_PATH_DECODE, "milo_attn_decode")
