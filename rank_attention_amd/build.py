"""Build the HIP library ``libmilo_attn.so`` for gfx950 with hipcc.

Every kernel translation unit is compiled in parallel, then linked with the
host library into one shared object next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmilo_attn.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are kept out of every kernel.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + INCLUDE, "-I" + CSRC]

# (source, extra defines, object name)
UNITS = [
    ("decode.hip", ["-DMILO_INST_DT=0", "-DMILO_INST_D=64"], "decode_f32_64.o"),
    ("decode.hip", ["-DMILO_INST_DT=0", "-DMILO_INST_D=128"], "decode_f32_128.o"),
    ("decode.hip", ["-DMILO_INST_DT=1", "-DMILO_INST_D=64"], "decode_bf16_64.o"),
    ("decode.hip", ["-DMILO_INST_DT=1", "-DMILO_INST_D=128"], "decode_bf16_128.o"),
    ("decode.hip", ["-DMILO_INST_DT=2", "-DMILO_INST_D=64"], "decode_q8_64.o"),
    ("decode.hip", ["-DMILO_INST_DT=2", "-DMILO_INST_D=128"], "decode_q8_128.o"),
    ("decode.hip", ["-DMILO_INST_DT=3", "-DMILO_INST_D=64"], "decode_kv4_64.o"),
    ("decode.hip", ["-DMILO_INST_DT=3", "-DMILO_INST_D=128"], "decode_kv4_128.o"),
    ("decode.hip", ["-DMILO_INST_DT=4", "-DMILO_INST_D=64"], "decode_kv2_64.o"),
    ("decode.hip", ["-DMILO_INST_DT=4", "-DMILO_INST_D=128"], "decode_kv2_128.o"),
    ("merge.hip", [], "merge.o"),
    ("chunk.hip", [], "chunk.o"),
    ("encode.hip", [], "encode.o"),
    ("rank.hip", [], "rank.o"),
    ("validate.hip", [], "validate.o"),
    ("probe.hip", [], "probe.o"),
    ("quant.hip", [], "quant.o"),
    ("kivi.hip", [], "kivi.o"),
    ("noalloc.hip", [], "noalloc.o"),
    ("milo_attn.cpp", [], "milo_attn.o"),
    ("milo_encode.cpp", [], "milo_encode.o"),
]


def _compile(unit, extra_flags):
    src, defs, obj = unit
    out = os.path.join(BUILD, obj)
    cmd = [HIPCC] + COMMON + defs + extra_flags + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} {defs}:\n{msgs}")
    return out, msgs


def build(jobs: int | None = None, extra_flags=None, verbose: bool = False) -> str:
    """Compile every kernel for gfx950 and link libmilo_attn.so (always rebuilds)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    os.makedirs(BUILD, exist_ok=True)
    extra_flags = list(extra_flags or [])
    jobs = jobs or min(len(UNITS), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        res = list(ex.map(lambda u: _compile(u, extra_flags), UNITS))
    if verbose:
        for _, msgs in res:
            if msgs.strip():
                print(msgs)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [o for o, _ in res]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(verbose="-v" in sys.argv))
