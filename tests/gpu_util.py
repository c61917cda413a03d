"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import rank_attention_amd as ra
import synth
from synth.gen import LogicalBlock, Workload

# Official parity gate (elementwise, numpy isclose convention).
ATOL, RTOL = 2e-3, 1e-2
# Extra gates for workloads whose outputs are not tiny: relative L2 error per
# query row and the log-sum-exp.
REL_L2 = 1e-2
LSE_ATOL, LSE_RTOL = 2e-3, 1e-2


def note(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_hip(wl: Workload, path: str = "decode", repeat: int = 1, **packkw):
    """Pack, upload, run the HIP path; returns (out, lse) float64 numpy arrays."""
    import torch
    pc = ra.pack(wl, **packkw)
    dc = ra.DeviceCache(pc, scale=wl.scale)
    note(f"{path} cfg={wl.cfg.name} variant={wl.variant} B={wl.batch} Q={wl.cfg.q_len} "
         f"Hq={wl.cfg.n_q_heads} Hkv={wl.cfg.n_kv_heads} d={wl.cfg.head_dim} dtype={wl.dtype} "
         f"max_blocks={pc.max_blocks} tail_cap={pc.k_tail.shape[2]}")
    outs = []
    for _ in range(repeat):
        out, lse = {"decode": dc.decode, "chunk": dc.chunk, "shared": dc.decode_shared}[path]()
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)))
    return outs if repeat > 1 else outs[0]


def chunk_ranges(dc, path=None) -> int:
    """Block ranges per (sequence, KV head) the library's chunk split gives
    for this cache, read back from the workspace size it asks for."""
    path = ra.MILO_PATH_CHUNK if path is None else path
    a = ra.make_args(*dc.tensors(), n_kv_heads=dc.n_kv_heads, scale=dc.scale, max_blocks=dc.max_blocks)
    total = ra.workspace_bytes(a, path)
    B, Q, Hq, d = (int(x) for x in dc.q.shape)
    if path == ra.MILO_PATH_SHARED:
        B, Q = B, 1
    rows = Q * (Hq // dc.n_kv_heads)
    def ws(units):                         # o~ rows, then (m, l) per row, each 256-B aligned
        r256 = lambda x: (x + 255) // 256 * 256
        return r256(units * rows * 4 * d) + r256(units * rows * 8)
    units = total // (rows * (4 * d + 8))
    while units > 0 and ws(units) > total:
        units -= 1
    assert ws(units) == total and units % (B * dc.n_kv_heads) == 0, "unexpected workspace layout"
    return int(units // (B * dc.n_kv_heads) - 1)


def compare(out, lse, ref_o, ref_l, rows=None, sharp_gates=False, name=""):
    """Assert the official gate (and the extra gates when asked) on the given
    rows [(i, j, h)] or on every row."""
    if rows is not None:
        idx = tuple(np.array(rows).T)
        out, lse, ref_o, ref_l = out[idx], lse[idx], ref_o[idx], ref_l[idx]
    assert np.all(np.isfinite(out)), f"{name}: non-finite GPU output"
    err = np.abs(out - ref_o)
    bad = err > ATOL + RTOL * np.abs(ref_o)
    assert not bad.any(), (f"{name}: {bad.sum()} of {bad.size} outputs outside atol {ATOL} + rtol {RTOL}; "
                           f"max err {err.max():.3e}")
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse)), f"{name}: lse finiteness differs"
    lerr = np.abs(lse[fin] - ref_l[fin])
    assert np.all(lerr <= LSE_ATOL + LSE_RTOL * np.abs(ref_l[fin])), f"{name}: lse max err {lerr.max():.3e}"
    if sharp_gates:
        num = np.linalg.norm((out - ref_o).reshape(-1, out.shape[-1]), axis=-1)
        den = np.linalg.norm(ref_o.reshape(-1, out.shape[-1]), axis=-1)
        rel = num / np.maximum(den, 1e-30)
        assert np.all(rel <= REL_L2), f"{name}: relative L2 error per row up to {rel.max():.3e}"
    return float(err.max())


def weight_abs_bound(wl, rows):
    """Per query row (i, j, h): ||sum_t a_t |v_t| ||_2 over the row's visible
    tokens (a the exact softmax weights, v_t the reconstructed value rows, in
    fp64) and the softmax mass of each listed block plus the tail (last
    entry).  Rounding every weight by a relative 2^-9 (e in bf16) moves the
    output by at most 2^-9 times the first figure, so it bounds the error of
    a row whose output nearly cancels.  Dense reconstruction: small workloads
    only."""
    from synth.gen import stored_to_f64
    dt, d = wl.dtype, wl.cfg.head_dim
    G = wl.cfg.n_q_heads // wl.cfg.n_kv_heads
    Q = wl.q.shape[1]
    q = stored_to_f64(wl.q, dt)
    cache = {}
    out_b, out_m = [], []
    for (i, j, h) in rows:
        g = h // G
        if (i, g) not in cache:
            Ks, Vs = [], []
            for b in wl.blocks[i]:
                U = stored_to_f64(b.ut[g], dt).T
                Up = stored_to_f64(b.upt[g], dt).T
                Ks.append(U @ stored_to_f64(b.w[g], dt))
                Vs.append(Up @ stored_to_f64(b.wp[g], dt))
            cache[(i, g)] = (Ks, Vs)
        Ks, Vs = cache[(i, g)]
        vis = int(wl.tail_len[i]) - Q + j + 1 if Q > 1 else int(wl.tail_len[i])
        vis = max(vis, 0)
        K = np.concatenate(Ks + [stored_to_f64(wl.k_tail[i, g, :vis], dt)])
        V = np.concatenate(Vs + [stored_to_f64(wl.v_tail[i, g, :vis], dt)])
        s = K @ q[i, j, h] * wl.scale
        a = np.exp(s - s.max())
        a /= a.sum()
        out_b.append(np.linalg.norm(a @ np.abs(V)))
        edges = np.cumsum([0] + [k.shape[0] for k in Ks] + [vis])
        out_m.append(np.add.reduceat(a, edges[:-1]) if len(a) else np.zeros(0))
    return np.array(out_b), out_m


def custom_workload(cfg, blocks, q, k_tail, v_tail, tail_len) -> Workload:
    """A workload from explicit arrays (stored dtype of cfg)."""
    return Workload(cfg=cfg, variant="custom", seqs=list(range(len(blocks))), q=q, blocks=blocks,
                    k_tail=k_tail, v_tail=v_tail, tail_len=np.asarray(tail_len, np.int32),
                    scale=cfg.scale)


def bf16_bits(x):
    return synth.gen.f32_to_bf16_bits(np.asarray(x, np.float32))
