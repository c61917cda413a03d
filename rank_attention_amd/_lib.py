"""ctypes view of the C ABI in include/milo_attn.h and include/milo_encode.h
(argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmilo_attn.so")

MILO_OK, MILO_ERR_INVALID, MILO_ERR_UNSUPPORTED, MILO_ERR_WORKSPACE, MILO_ERR_DEVICE = range(5)
MILO_F32, MILO_BF16, MILO_BF16_Q8, MILO_BF16_KV4, MILO_BF16_KV2 = 0, 1, 2, 3, 4
MILO_PATH_DECODE, MILO_PATH_CHUNK, MILO_PATH_SHARED = 0, 1, 2
MILO_NOALLOC_SCRATCH_BYTES = 32 << 20   # static scratch of milo_attn_decode_noalloc
EXPORTS = ("milo_attn_workspace_bytes", "milo_attn_decode", "milo_attn_chunk", "milo_attn_decode_shared",
           "milo_attn_plan_decode", "milo_status_str", "milo_abi_version",
           "milo_encode_workspace_bytes", "milo_encode_spectrum", "milo_encode_factors", "milo_encode_layout",
           "milo_rank_workspace_bytes", "milo_rank_allocate", "milo_attn_validate", "milo_read_probe",
           "milo_quant_layout", "milo_quantize_factors", "milo_attn_decode_noalloc", "milo_kivi_layout",
           "milo_quantize_kivi")
TABLE_RULES = {1: "seq_range", 2: "too_many_blocks", 3: "rank", 4: "tokens", 5: "offset", 6: "pool_bounds",
               7: "tail_len", 8: "unit_order"}


class MiloBlock(ctypes.Structure):
    _fields_ = [("off", ctypes.c_int64), ("n_tok", ctypes.c_int32), ("ld_tok", ctypes.c_int32),
                ("rank_k", ctypes.c_int32), ("rank_v", ctypes.c_int32)]


class MiloAttnArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("pool", ctypes.c_void_p),
        ("blocks", ctypes.c_void_p),
        ("seq_blocks", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("tail_cap", ctypes.c_int32),
        ("k_tail", ctypes.c_void_p),
        ("v_tail", ctypes.c_void_p),
        ("tail_len", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("prof_events", ctypes.c_void_p * 2),
        ("unit_order", ctypes.c_void_p),
    ]


class MiloEncodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("n_tokens", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("tok_start", ctypes.c_void_p),
        ("blocks", ctypes.c_void_p),
        ("sigma", ctypes.c_void_p),
        ("iters", ctypes.c_void_p),
        ("pool", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MiloRankArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("budget_k", ctypes.c_int32),
        ("budget_v", ctypes.c_int32),
        ("r_min", ctypes.c_int32),
        ("unit", ctypes.c_int32),
        ("sigma", ctypes.c_void_p),
        ("ranks", ctypes.c_void_p),
        ("entropy", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MiloQuantArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("src_pool", ctypes.c_void_p),
        ("src_blocks", ctypes.c_void_p),
        ("dst_pool", ctypes.c_void_p),
        ("dst_blocks", ctypes.c_void_p),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the built HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        # Stream handles and device pointers from torch cross the boundary, so
        # the library must run on torch's HIP runtime.  torch bundles its own
        # libamdhip64 with the same soname as the system one the library
        # names; loading torch first makes that dependency resolve to torch's
        # copy instead of a second runtime (which would not know torch's
        # streams and, on some hosts, finds no device).
        import torch  # noqa: F401
        lib = ctypes.CDLL(LIB_PATH)
        lib.milo_attn_workspace_bytes.argtypes = [ctypes.POINTER(MiloAttnArgs), ctypes.c_int32]
        lib.milo_attn_workspace_bytes.restype = ctypes.c_size_t
        for fn in (lib.milo_attn_decode, lib.milo_attn_chunk, lib.milo_attn_decode_shared,
                   lib.milo_attn_decode_noalloc):
            fn.argtypes = [ctypes.POINTER(MiloAttnArgs), ctypes.c_void_p]
            fn.restype = ctypes.c_int
        lib.milo_attn_validate.argtypes = [ctypes.POINTER(MiloAttnArgs), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.milo_attn_validate.restype = ctypes.c_int
        lib.milo_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p]
        lib.milo_read_probe.restype = ctypes.c_int
        lib.milo_attn_plan_decode.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        lib.milo_attn_plan_decode.restype = ctypes.c_int
        lib.milo_status_str.argtypes = [ctypes.c_int]
        lib.milo_status_str.restype = ctypes.c_char_p
        lib.milo_encode_workspace_bytes.argtypes = [ctypes.POINTER(MiloEncodeArgs)]
        lib.milo_encode_workspace_bytes.restype = ctypes.c_size_t
        for fn in (lib.milo_encode_spectrum, lib.milo_encode_factors):
            fn.argtypes = [ctypes.POINTER(MiloEncodeArgs), ctypes.c_void_p]
            fn.restype = ctypes.c_int
        lib.milo_encode_layout.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_int64)]
        lib.milo_encode_layout.restype = ctypes.c_int
        lib.milo_rank_workspace_bytes.argtypes = [ctypes.POINTER(MiloRankArgs)]
        lib.milo_rank_workspace_bytes.restype = ctypes.c_size_t
        lib.milo_rank_allocate.argtypes = [ctypes.POINTER(MiloRankArgs), ctypes.c_void_p]
        lib.milo_rank_allocate.restype = ctypes.c_int
        lib.milo_quant_layout.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
        lib.milo_quant_layout.restype = ctypes.c_int
        lib.milo_quantize_factors.argtypes = [ctypes.POINTER(MiloQuantArgs), ctypes.c_void_p]
        lib.milo_quantize_factors.restype = ctypes.c_int
        lib.milo_kivi_layout.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
        lib.milo_kivi_layout.restype = ctypes.c_int
        lib.milo_quantize_kivi.argtypes = [ctypes.POINTER(MiloQuantArgs), ctypes.c_int32, ctypes.c_void_p]
        lib.milo_quantize_kivi.restype = ctypes.c_int
        lib.milo_abi_version.argtypes = []
        lib.milo_abi_version.restype = ctypes.c_int32
        _lib = lib
    return _lib
