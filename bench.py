#!/usr/bin/env python3
"""Attention benchmark over a block-wise low-rank KV cache on one MI355X.

One step = one call of the attention path (split-K attention kernel + merge
kernel) over the whole batch of one layer, inputs resident in HBM.  Prints one
JSON line.

Decode workloads (the default, qwen7b_64k): context tokens/s for the step and
the attention kernel's achieved HBM bandwidth on algorithmic bytes against the
8 TB/s peak.  Chunked-query workloads (qwen32b_chunk): query tokens/s and the
kernel's algorithmic bf16 FLOP rate against the 2.5 PFLOP/s dense MFMA peak.
Shared-context decode (--shared, on a decode workload): every sequence of the
batch attends to sequence 0's compressed context plus its own tail; context
tokens/s counts each sequence's full context, and the roofline is that of the
MFMA kernel, which reads the shared factors once and each sequence's tail
(HBM-bound while the batch's query rows per KV head stay under the 312
FLOP/byte ridge).
Kernel time comes from HIP events recorded on the launch stream around the
attention kernel alone; the fp64 CPU oracle is timed on a bounded sample.

8-bit token factors (--q8, on a decode workload): the bf16 pool is quantised
once (milo_quantize_factors, outside the timed region) and the decode path
reads the 8-bit pool; algorithmic bytes are the codes, the bf16 W/W' and the
per-row (scale, bias) pairs plus the tails.

KIVI-style token factors (--kivi 4 or --kivi 2, on a decode workload): the
bf16 pool is quantised once (milo_quantize_kivi) and the decode path reads
the 4- or 2-bit pool; algorithmic bytes are the codes at their width, one
fp16 (scale, bias) pair per key group (rank component x 64-token chunk) and
per value group (token x 32 rank components), the bf16 W/W' and the tails.

Encode (--encode, workload enc_qwen7b_64k): one step runs the encode
workflow over the dense keys and values of one 64k-token context (spectra,
entropy-driven ranks at a 50% budget, host layout, factors); context
tokens/s, and the spectrum kernel's algorithmic fp32 rate against the 157.3
TFLOP/s vector peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen7b_64k] [--shared | --q8 | --kivi 4|2]
    python bench.py --encode [--workload enc_qwen7b_64k]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

ENCODE_METRIC = "low-rank-KV encode: context tokens/s factorised (dense K/V -> per-block truncated SVD factors)"
FP32_VECTOR_PEAK_TFLOPS = 157.3
METRIC = "low-rank-KV decode attn: context tokens/s and % of HBM peak (7B, 64k)"
Q8_METRIC = "low-rank-KV decode attn, 8-bit token factors: context tokens/s and % of HBM peak (7B, 64k)"
KIVI_METRIC = ("low-rank-KV decode attn, KIVI-style {bits}-bit token factors: context tokens/s and % of HBM peak "
               "(7B, 64k)")
SHARED_METRIC = "low-rank-KV shared-context decode attn: context tokens/s (7B, 64k context shared by the batch)"
CHUNK_METRIC = "low-rank-KV chunked-query attn: query tokens/s and % of bf16 MFMA peak (32B, Q=256)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
LAST_LEVEL_CACHE_BYTES = 256 << 20   # MI355X Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "decode": ["rank_attention_amd/csrc/decode.hip", "rank_attention_amd/csrc/decode_kivi.inc",
               "rank_attention_amd/csrc/device_common.h"],
    "chunk": ["rank_attention_amd/csrc/chunk.hip", "rank_attention_amd/csrc/device_common.h"],
    "encode": ["rank_attention_amd/csrc/encode.hip", "rank_attention_amd/csrc/device_common.h"],
}


def kernel_source_sha(path: str = "decode") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[path]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (timing plumbing)."""

    def __init__(self):
        import torch  # noqa: F401  (loads the HIP runtime)
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, ev: int) -> None:
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def traffic_from_profiles(workload: str, path: str = "decode"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    fn = os.path.join(PROFILES, f"{path}_{workload}_traffic.json")
    if not os.path.exists(fn):
        return None
    rec = json.load(open(fn))
    if rec.get("kernel_source_sha") != kernel_source_sha(path):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_ceiling_gbs(lib, torch, gib: int = 2, reps: int = 5) -> float:
    """HBM read rate of the library's streaming-read probe (the decode
    kernel's load form) over a fresh `gib` GiB buffer, mean of `reps` runs."""
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        lib.milo_read_probe(buf.data_ptr(), n, sink.data_ptr(), 4096, ctypes.c_void_p(stream))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        rc = lib.milo_read_probe(buf.data_ptr(), n, sink.data_ptr(), 4096, ctypes.c_void_p(stream))
        b.record()
        if rc != 0:
            raise RuntimeError("milo_read_probe failed")
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / reps
    del buf
    return n / (ms * 1e-3) / 1e9


def chunk_flops(wl, shared: bool = False) -> int:
    """Algorithmic FLOPs of one chunked-query launch: per block and KV head
    2*M*(r + r')*(T + d) for the four factor products (M = Q*G query rows),
    and 4*d per visible (query row, tail token) pair of the causal tail.
    Shared context: M = batch*G rows over sequence 0's blocks, plus each
    sequence's G rows over its own tail."""
    cfg = wl.cfg
    G = cfg.n_q_heads // cfg.n_kv_heads
    Q, d = cfg.q_len, cfg.head_dim
    M = Q * G
    total = 0
    if shared:
        return (sum(2 * wl.batch * G * (b.rank_k + b.rank_v) * (b.n_tok + d) * cfg.n_kv_heads
                    for b in wl.blocks[0]) + 4 * d * G * cfg.n_kv_heads * int(wl.tail_len.sum()))
    for i, seq in enumerate(wl.blocks):
        for b in seq:
            total += 2 * M * (b.rank_k + b.rank_v) * (b.n_tok + d) * cfg.n_kv_heads
        L = int(wl.tail_len[i])
        vis = sum(max(0, min(L, L - Q + j + 1)) for j in range(Q))
        total += 4 * d * vis * G * cfg.n_kv_heads
    return total


def encode_flops(ctx) -> int:
    """Algorithmic FLOPs of encoding a context: per (block, head, K/V)
    matrix of T tokens at rank r, the Gram matrix (2 T d^2), a symmetric
    eigen-decomposition with vectors at the textbook count (9 d^3:
    tridiagonalisation plus implicit QR with accumulated rotations) and the
    projection U = X W^T (2 T d r)."""
    d, h = ctx.cfg.head_dim, ctx.cfg.n_kv_heads
    total = 0
    for b in range(len(ctx.n_tok)):
        T = int(ctx.n_tok[b])
        for kv in range(2):
            total += h * (2 * T * d * d + 9 * d ** 3 + 2 * T * d * int(ctx.ranks[b][kv]))
    return total


def cpu_baseline_encode(ctx, seconds: float):
    """fp64 SVD oracle on whole blocks of the context until `seconds` pass."""
    from oracle import encode as oenc
    toks, elapsed, done = 0, 0.0, 0
    for b in range(len(ctx.n_tok)):
        t0 = time.perf_counter()
        for g in range(ctx.cfg.n_kv_heads):
            for kv in range(2):
                oenc.encode_block(ctx.dense_f64(kv, b, g), int(ctx.ranks[b][kv]))
        elapsed += time.perf_counter() - t0
        toks += int(ctx.n_tok[b])
        done += 1
        if elapsed >= seconds:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    return {"value": toks / elapsed, "unit": "context tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{done} of {len(ctx.n_tok)} blocks (all {ctx.cfg.n_kv_heads} KV heads, K and V), "
                      f"numpy fp64 SVD, {elapsed:.1f} s"}


def run_encode(args) -> int:
    """The encode workflow per step: spectra (Gram + tridiagonal QL), entropy-driven
    ranks at a 50% rank budget for keys and for values (r_min 8), the pool
    layout on the host, then the factors at those ranks."""
    import numpy as np
    import torch
    import rank_attention_amd as ra
    import synth
    from rank_attention_amd import _lib
    from rank_attention_amd.encode import DeviceContext, allocate_ranks, layout

    if not os.path.exists(ra.library_path):
        import __graft_entry__
        __graft_entry__.build()
    lib = _lib.load()
    name = args.workload if args.workload.startswith("enc_") else "enc_qwen7b_64k"
    cfg = synth.get_encode_config(name)
    t0 = time.time()
    ctx = synth.make_dense_context(cfg)
    nb, d, h = len(ctx.n_tok), cfg.head_dim, cfg.n_kv_heads
    r_min, frac = 8, 0.5
    budget = int(nb * d * frac)
    dc = DeviceContext(ctx.k, ctx.v, ctx.tok_start, ctx.n_tok, dtype=cfg.dtype, device="cuda:0")
    dense_bytes = 2 * dc.k.numel() * dc.k.element_size()
    copies = max(args.copies, -(-3 * LAST_LEVEL_CACHE_BYTES // max(1, dense_bytes)))
    kvs = [(dc.k, dc.v)] + [(dc.k.clone(), dc.v.clone()) for _ in range(copies - 1)]
    sigma, iters = dc.spectrum()            # sizes the workspace
    _, full_elems = layout(ctx.n_tok, [d] * nb, [d] * nb, h, d)
    pool = torch.empty(full_elems, dtype=torch.int16 if cfg.dtype == "bf16" else torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    sw = iters.cpu().numpy()
    spec_blocks = dc._spectrum_blocks
    print(f"[bench] {cfg.desc}: dense K/V {dense_bytes / 1e6:.1f} MB, {copies} copies, QL iterations "
          f"{sw.min()}..{sw.max()} (mean {sw.mean():.1f}), rank budget {budget} per K/V (50%), r_min {r_min}, "
          f"setup {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    def step(k, evs=None):
        dc.k, dc.v = kvs[k % len(kvs)]
        rec = (lambda i: evs[i].record()) if evs is not None else (lambda i: None)
        rec(0)
        rc = lib.milo_encode_spectrum(ctypes.byref(dc._args(spec_blocks, sigma=sigma, iters=iters)),
                                      ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"milo_encode_spectrum failed: {ra.status_str(rc)}")
        rec(1)
        ranks, _ = allocate_ranks(sigma, budget, budget, r_min, 1)
        rec(2)
        rk = ranks.cpu().numpy()                 # the pool layout is a host step
        blocks, _ = layout(ctx.n_tok, rk[:, 0], rk[:, 1], h, d)
        bdev = torch.from_numpy(blocks.view(np.uint8).copy()).to("cuda:0", non_blocking=False)
        rec(3)
        rc = lib.milo_encode_factors(ctypes.byref(dc._args(bdev, pool=pool)), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"milo_encode_factors failed: {ra.status_str(rc)}")
        rec(4)
        return rk

    stream = torch.cuda.current_stream().cuda_stream
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for k in range(args.steps):
        rk = step(k, evs[k])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    spec_ms = [e[0].elapsed_time(e[1]) for e in evs]
    alloc_ms = [e[1].elapsed_time(e[2]) for e in evs]
    fac_ms = [e[3].elapsed_time(e[4]) for e in evs]
    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    kmean = sum(spec_ms) / len(spec_ms)
    amean = sum(alloc_ms) / len(alloc_ms)
    fmean = sum(fac_ms) / len(fac_ms)
    spec_flops = sum(h * 2 * (2 * int(T) * d * d + 9 * d ** 3) for T in ctx.n_tok)
    achieved = spec_flops / (kmean * 1e-3) / 1e12
    tokens = int(ctx.n_tok.sum())
    print(f"[bench] spectrum kernel mean {kmean * 1e3:.1f} us, rank allocation {amean * 1e3:.1f} us, factors "
          f"kernel mean {fmean * 1e3:.1f} us, step {ms_per_step * 1e3:.1f} us; {achieved:.2f} TFLOP/s "
          f"algorithmic in the spectrum kernel; allocated ranks K {rk[:, 0].min()}..{rk[:, 0].max()}, "
          f"V {rk[:, 1].min()}..{rk[:, 1].max()}", file=sys.stderr, flush=True)
    res = {
        "metric": ENCODE_METRIC, "value": tokens / (ms_per_step * 1e-3), "unit": "context tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "desc": cfg.desc, "n_blocks": nb, "block_tokens": cfg.block_tokens,
                   "n_kv_heads": h, "head_dim": d, "context_tokens_per_step": tokens, "copies": copies,
                   "rank_budget": budget, "r_min": r_min, "ql_iterations_mean": float(sw.mean())},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_VECTOR_PEAK_TFLOPS,
                     "traffic": traffic_from_profiles(cfg.name, "encode"),
                     "kernel": "milo_encode_spectrum_kernel", "kernel_us_mean": kmean * 1e3,
                     "rank_allocation_us_mean": amean * 1e3, "factors_kernel_us_mean": fmean * 1e3,
                     "algorithmic_flops_per_launch": spec_flops,
                     "algorithmic_bytes_per_launch": dense_bytes,
                     "kernel_source_sha": kernel_source_sha("encode")},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_encode(ctx, args.cpu_seconds),
    }
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline_chunk(wl, seconds: float):
    """fp64 oracle on sampled query positions (all heads) of sequence 0 of the
    chunk workload, grown until `seconds` pass; reported per query token."""
    import oracle
    q, blocks, kt, vt, tl = oracle.logical_from_workload(wl, [0])
    Q, Hq = wl.cfg.q_len, wl.cfg.n_q_heads
    js, elapsed, n = [], 0.0, 1
    order = [Q - 1 - (k * 37) % Q for k in range(Q)]
    while elapsed < seconds and len(js) < Q:
        new = order[len(js):len(js) + n]
        sel = [(0, j, h) for j in new for h in range(Hq)]
        t0 = time.perf_counter()
        oracle.attend_logical(q, blocks, kt, vt, tl, wl.scale, sel=sel)
        elapsed += time.perf_counter() - t0
        js += new
        n *= 2
    return {"value": len(js) / elapsed, "unit": "query tokens/s", "cores": oracle.threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{len(js)} of {Q} query positions x all {Hq} heads of sequence 0 "
                      f"({sum(b.n_tok for b in wl.blocks[0]) + int(wl.tail_len[0])} context tokens), "
                      f"fp64 reconstruct-then-attend, {elapsed:.1f} s"}


def kivi_factor_bytes(wl, bits: int) -> int:
    """Algorithmic bytes of the KIVI-style factors: per block and KV head the
    codes at `bits` per element, an fp16 (scale, bias) pair per key group
    (rank component x 64-token chunk) and per value group (token x 32 rank
    components), and the bf16 W and W'."""
    d, h = wl.cfg.head_dim, wl.cfg.n_kv_heads
    total = 0
    for s_ in wl.blocks:
        for b in s_:
            T, r, rv = b.n_tok, b.rank_k, b.rank_v
            codes = (T * (r + rv) * bits + 7) // 8
            groups = -(-T // 64) * r + T * -(-rv // 32)
            total += h * (codes + 4 * groups + 2 * d * (r + rv))
    return total


def cpu_baseline(wl, seconds: float, q8: bool = False, kivi_bits: int = 0):
    """fp64 oracle on whole sequences of the same workload, in order and again
    from the first when the batch is done, until `seconds` pass (q8 or
    kivi_bits: the oracle's quantisation of the token factors, then attention
    over the dequantized factors, both timed)."""
    import oracle
    from oracle import kivi, quant
    toks, elapsed, done = 0, 0.0, 0
    while wl.batch > 0 and elapsed < seconds:
        i = done % wl.batch
        q, blocks, kt, vt, tl = oracle.logical_from_workload(wl, [i])
        t0 = time.perf_counter()
        if q8:
            blocks = quant.quantize_logical_blocks(blocks)
        if kivi_bits:
            blocks = kivi.quantize_logical_blocks(blocks, kivi_bits)
        oracle.attend_logical(q, blocks, kt, vt, tl, wl.scale)
        elapsed += time.perf_counter() - t0
        toks += sum(b.n_tok for b in wl.blocks[i]) + int(wl.tail_len[i])
        done += 1
    return {"value": toks / elapsed, "unit": "context tokens/s", "cores": oracle.threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{done} sequence evaluations over the {wl.batch} of the workload ({toks} context "
                      f"tokens, all {wl.cfg.n_q_heads} query heads), {'fp32 8-bit quantisation, ' if q8 else ''}"
                      f"{f'fp32 KIVI-style {kivi_bits}-bit quantisation, ' if kivi_bits else ''}"
                      f"fp64 reconstruct-then-attend, {elapsed:.1f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first few dozen launches run slower (about 175 us against 167 us at
    # qwen7b_64k) while the device settles, so the default warmup covers them
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="qwen7b_64k")
    ap.add_argument("--variant", default="base")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch (sequences)")
    ap.add_argument("--q-heads", type=int, default=0, help="override the query heads (group size)")
    ap.add_argument("--encode", action="store_true",
                    help="encode step: factorise the dense K/V of one context (enc_* workloads)")
    ap.add_argument("--shared", action="store_true",
                    help="shared-context decode: the batch attends to sequence 0's context")
    ap.add_argument("--q8", action="store_true",
                    help="decode over 8-bit token factors (the bf16 pool quantised once before timing)")
    ap.add_argument("--kivi", type=int, default=0, choices=(0, 2, 4),
                    help="decode over KIVI-style 4- or 2-bit token factors (quantised once before timing)")
    ap.add_argument("--copies", type=int, default=2,
                    help="pool copies read in rotation so no step finds the last one's bytes in cache")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-plan", action="store_true", help="natural work-unit order (no schedule)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true", help="skip the measured read-ceiling probe")
    ap.add_argument("--dump-steps", action="store_true", help="print each timed step's kernel time")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        return 2

    import torch

    if args.encode or args.workload.startswith("enc_"):
        return run_encode(args)

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return 0

    import rank_attention_amd as ra
    import synth
    from rank_attention_amd import _lib

    if not os.path.exists(ra.library_path):
        import __graft_entry__
        __graft_entry__.build()
    lib = _lib.load()

    cfg = synth.get_config(args.workload)
    if args.batch:
        cfg = cfg.with_(batch=args.batch, desc=f"{cfg.desc}; batch set to {args.batch}")
    if args.q_heads:
        cfg = cfg.with_(n_q_heads=args.q_heads, desc=f"{cfg.desc}; {args.q_heads} query heads")
    is_chunk = cfg.path == "chunk"
    shared = args.shared
    q8 = args.q8
    kv = args.kivi
    if kv and (q8 or is_chunk or shared or cfg.dtype != "bf16"):
        print("--kivi needs a bf16 decode workload (and neither --shared nor --q8)", file=sys.stderr)
        return 2
    if shared and is_chunk:
        print("--shared needs a decode workload", file=sys.stderr)
        return 2
    if q8 and (is_chunk or shared or cfg.dtype != "bf16"):
        print("--q8 needs a bf16 decode workload (and not --shared)", file=sys.stderr)
        return 2
    path_code = (_lib.MILO_PATH_CHUNK if is_chunk else
                 _lib.MILO_PATH_SHARED if shared else _lib.MILO_PATH_DECODE)
    entry = (lib.milo_attn_chunk if is_chunk else
             lib.milo_attn_decode_shared if shared else lib.milo_attn_decode)
    t0 = time.time()
    if shared:
        # only sequence 0's blocks are packed: the shared path reads no other list
        wl = synth.make_workload(cfg, variant=args.variant, n_blocks=[cfg.n_blocks] + [0] * (cfg.batch - 1))
    else:
        wl = synth.make_workload(cfg, variant=args.variant)
    pc = ra.pack(wl)
    dc = ra.DeviceCache(pc, device="cuda:0", scale=wl.scale)
    if q8:
        dc = dc.quantized()
        torch.cuda.synchronize()
    if kv:
        dc = dc.kivi(kv)
        torch.cuda.synchronize()
    copies = args.copies
    if shared:
        # the shared factors and the tails are small: rotate enough copies of
        # both that a step never finds the previous steps' bytes in the
        # last-level cache
        step_bytes = dc.pool.numel() * dc.pool.element_size()
        if dc.k_tail is not None:
            step_bytes += 2 * dc.k_tail.numel() * dc.k_tail.element_size()
        copies = max(copies, -(-3 * LAST_LEVEL_CACHE_BYTES // max(1, step_bytes)))
    pools = [dc.pool] + [dc.pool.clone() for _ in range(max(0, copies - 1))]
    tails = [(dc.k_tail, dc.v_tail)] * len(pools)
    if shared and dc.k_tail is not None:
        tails = [(dc.k_tail, dc.v_tail)] + [(dc.k_tail.clone(), dc.v_tail.clone()) for _ in pools[1:]]
    B, Q, Hq, d = (int(x) for x in dc.q.shape)
    out = torch.empty((B, Q, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Q, Hq), dtype=torch.float32, device="cuda:0")
    a0 = ra.make_args(*dc.tensors(), n_kv_heads=dc.n_kv_heads, scale=dc.scale, max_blocks=dc.max_blocks,
                      out=out, lse=lse, storage=dc.storage)
    need = lib.milo_attn_workspace_bytes(ctypes.byref(a0), path_code)
    ws = torch.empty(int(need), dtype=torch.uint8, device="cuda:0")
    argsets = []
    for pool, (kt, vt) in zip(pools, tails):
        a = ra.make_args(dc.q, pool, dc.blocks, dc.seq_blocks, kt, vt, dc.tail_len,
                         n_kv_heads=dc.n_kv_heads, scale=dc.scale, max_blocks=dc.max_blocks, out=out,
                         lse=lse, workspace=ws,
                         unit_order=None if (args.no_plan or is_chunk or shared) else dc.unit_order,
                         storage=dc.storage)
        argsets.append(a)
    stream = torch.cuda.current_stream().cuda_stream
    setup_s = time.time() - t0
    shared_factor_bytes = wl.factor_bytes()
    if shared:
        wl.blocks = [wl.blocks[0] for _ in range(wl.batch)]   # what every sequence attends to
    print(f"[bench] {cfg.desc}: factor {wl.factor_bytes() / 1e6:.1f} MB, tail {wl.tail_bytes() / 1e6:.1f} MB, "
          f"setup {setup_s:.1f} s", file=sys.stderr, flush=True)

    def step(k, evs=None):
        a = argsets[k % len(argsets)]
        if evs is not None:
            a.prof_events[0], a.prof_events[1] = evs
        else:
            a.prof_events[0] = a.prof_events[1] = None
        rc = entry(ctypes.byref(a), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"{'milo_attn_decode_shared' if shared else 'milo_attn_' + cfg.path} "
                               f"failed: {ra.status_str(rc)}")

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    hip = HipEvents()
    evs = [(hip.create(), hip.create()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(k, evs[k])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    kern_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    if args.dump_steps:
        print("[bench] kernel us per step: " + " ".join(f"{x * 1e3:.1f}" for x in kern_ms),
              file=sys.stderr, flush=True)
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)

    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    kmean = sum(kern_ms) / len(kern_ms)
    kern_sorted = sorted(kern_ms)

    def pct(q):
        return kern_sorted[min(len(kern_sorted) - 1, int(q * (len(kern_sorted) - 1) + 0.5))] * 1e3

    # the shared path reads sequence 0's factors once for the whole batch
    factor_bytes = shared_factor_bytes if shared else wl.factor_bytes()
    if q8:
        # per KV head and row: n_tok codes, d bf16 of W or W', one fp32 (scale, bias) pair
        factor_bytes = sum(cfg.n_kv_heads * (b.rank_k + b.rank_v) * (b.n_tok + 2 * d + 8)
                           for s_ in wl.blocks for b in s_)
    if kv:
        factor_bytes = kivi_factor_bytes(wl, kv)
    alg_bytes = factor_bytes + wl.tail_bytes()
    es = 2 if cfg.dtype == "bf16" else 4
    # every byte a step moves: factors + tails + q, partials written and read, out and lse
    all_bytes = (factor_bytes + wl.tail_bytes() + B * Q * Hq * d * es + 2 * int(need)
                 + B * Q * Hq * (d + 1) * 4)
    prof_key = ((cfg.name + "_shared", "chunk") if shared else (cfg.name + "_q8", "decode") if q8
                else (cfg.name + f"_kv{kv}", "decode") if kv else (cfg.name, cfg.path))
    if shared:
        flops = chunk_flops(wl, shared=True)
        alg_bytes = shared_factor_bytes + wl.tail_bytes()
        t_hbm, t_mfma = alg_bytes / HBM_PEAK_GBS / 1e9, flops / MFMA_BF16_PEAK_TFLOPS / 1e12
        if t_mfma > t_hbm:
            achieved = flops / (kmean * 1e-3) / 1e12
            peak, unit, bound = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
        else:
            achieved = alg_bytes / (kmean * 1e-3) / 1e9
            peak, unit, bound = HBM_PEAK_GBS, "GB/s", "hbm"
        value, vunit, metric = wl.context_tokens() / (ms_per_step * 1e-3), "context tokens/s", SHARED_METRIC
        kname = "milo_chunk_kernel"
        print(f"[bench] shared-context block kernel: mean {kmean * 1e3:.1f} us, median "
              f"{kern_sorted[len(kern_sorted) // 2] * 1e3:.1f} us, min {kern_sorted[0] * 1e3:.1f} us; "
              f"step {ms_per_step * 1e3:.1f} us; {flops / (kmean * 1e-3) / 1e12:.0f} TFLOP/s on "
              f"{flops / 1e9:.2f} GFLOP, {alg_bytes / (kmean * 1e-3) / 1e9:.0f} GB/s on "
              f"{alg_bytes / 1e6:.1f} MB shared factors + tails ({flops / max(1, alg_bytes):.0f} FLOP/B); "
              f"{copies} pool copies", file=sys.stderr, flush=True)
    elif is_chunk:
        flops = chunk_flops(wl)
        achieved = flops / (kmean * 1e-3) / 1e12
        peak, unit, bound = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
        value, vunit, metric = B * Q / (ms_per_step * 1e-3), "query tokens/s", CHUNK_METRIC
        kname = "milo_chunk_kernel"
        print(f"[bench] attention kernel: mean {kmean * 1e3:.1f} us, median "
              f"{kern_sorted[len(kern_sorted) // 2] * 1e3:.1f} us, min {kern_sorted[0] * 1e3:.1f} us; "
              f"step {ms_per_step * 1e3:.1f} us; {achieved:.0f} TFLOP/s on {flops / 1e9:.1f} GFLOP, "
              f"{alg_bytes / (kmean * 1e-3) / 1e9:.0f} GB/s of factor+tail bytes", file=sys.stderr, flush=True)
    else:
        achieved = alg_bytes / (kmean * 1e-3) / 1e9
        peak, unit, bound = HBM_PEAK_GBS, "GB/s", "hbm"
        value, vunit, metric = (wl.context_tokens() / (ms_per_step * 1e-3), "context tokens/s",
                                Q8_METRIC if q8 else KIVI_METRIC.format(bits=kv) if kv else METRIC)
        kname = "milo_decode_q8_kernel" if q8 else "milo_decode_kv_kernel" if kv else "milo_decode_kernel"
        print(f"[bench] attention kernel: mean {kmean * 1e3:.1f} us, median "
              f"{kern_sorted[len(kern_sorted) // 2] * 1e3:.1f} us, min {kern_sorted[0] * 1e3:.1f} us; "
              f"step {ms_per_step * 1e3:.1f} us; {achieved:.0f} GB/s on {alg_bytes / 1e6:.1f} MB",
              file=sys.stderr, flush=True)

    res = {
        "metric": metric,
        "value": value,
        "unit": vunit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+u8" if q8 else f"bf16+u{kv}" if kv else cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "desc": cfg.desc, "batch": cfg.batch, "q_len": cfg.q_len,
                   "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "blocks_per_seq": cfg.n_blocks, "block_tokens": cfg.block_tokens,
                   "tail_len": cfg.tail_len, "context_tokens_per_step": wl.context_tokens(),
                   "variant": args.variant, "pool_copies": len(pools), "shared_context": shared,
                   "factor_storage": ("u8 token factors, bf16 W/W'" if q8 else
                                      f"KIVI-style u{kv} token factors, fp16 group scales, bf16 W/W'" if kv
                                      else cfg.dtype)},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic_from_profiles(*prof_key),
                     "kernel": kname, "kernel_us_mean": kmean * 1e3,
                     "kernel_us_p10": pct(0.1), "kernel_us_median": pct(0.5), "kernel_us_p90": pct(0.9),
                     "algorithmic_bytes_per_launch": alg_bytes, "all_bytes_per_step": all_bytes,
                     "algorithmic_factor_bytes_per_launch": factor_bytes,
                     "achieved_factor_only": factor_bytes / (kmean * 1e-3) / 1e9,
                     "kernel_source_sha": kernel_source_sha(prof_key[1])},
        "cpu_baseline": None,
    }
    if is_chunk or shared:
        res["roofline"]["algorithmic_flops_per_launch"] = flops
    if bound == "hbm" and not args.no_read_probe:
        ceil = read_ceiling_gbs(lib, torch)
        res["roofline"]["measured_read_ceiling_gbs"] = ceil
        res["roofline"]["frac_of_measured_ceiling"] = achieved / ceil
        print(f"[bench] streaming-read probe: {ceil:.0f} GB/s; kernel at {100 * achieved / ceil:.1f}% of it",
              file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = (cpu_baseline_chunk(wl, args.cpu_seconds) if is_chunk
                               else cpu_baseline(wl, args.cpu_seconds, q8=q8, kivi_bits=kv))
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
