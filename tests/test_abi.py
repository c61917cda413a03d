"""The C-ABI library: it loads, exports every declared symbol, and rejects
host-checkable faults before any HIP call (so these run without a GPU)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import rank_attention_amd as ra
from rank_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

FAKE = 0x10000  # 64 KiB-aligned non-null address; never dereferenced by these calls


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(milo_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_struct_size():
    assert ra.abi_version() == 5
    # 7 int32 + float, 4 pointers, 2 int32, 6 pointers, size_t, 3 pointers; the
    # C side agrees, or the batch-0 call below would fail its struct_size check
    assert ctypes.sizeof(_lib.MiloAttnArgs) == 8 * 4 + 4 * 8 + 2 * 4 + 6 * 8 + 8 + 3 * 8
    assert ctypes.sizeof(_lib.MiloBlock) == 24 == ra.BLOCK_DTYPE.itemsize


def test_status_strings():
    for code in range(5):
        assert isinstance(ra.status_str(code), str) and ra.status_str(code)
    assert ra.status_str(99) == "unknown status"


def good_args(**over):
    a = _lib.MiloAttnArgs()
    a.struct_size = ctypes.sizeof(_lib.MiloAttnArgs)
    a.dtype = _lib.MILO_BF16
    a.batch, a.q_len, a.n_q_heads, a.n_kv_heads, a.head_dim = 2, 1, 14, 2, 64
    a.scale = 0.125
    a.q = a.pool = a.blocks = a.seq_blocks = FAKE
    a.max_blocks_per_seq = 4
    a.tail_cap = 16
    a.k_tail = a.v_tail = a.tail_len = FAKE
    a.out = a.lse = FAKE
    a.workspace = FAKE
    for k, v in over.items():
        setattr(a, k, v)
    return a


def call(a, path=_lib.MILO_PATH_DECODE):
    lib = _lib.load()
    fn = lib.milo_attn_decode if path == _lib.MILO_PATH_DECODE else lib.milo_attn_chunk
    return fn(ctypes.byref(a), None)


def test_workspace_query():
    lib = _lib.load()
    a = good_args()
    need = lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_DECODE)
    # units = B * Hkv * (max_blocks + 1), rows per unit = G, (d + 2) floats per row
    units, rows = 2 * 2 * 5, 7
    exp_o = -(-units * rows * 64 * 4 // 256) * 256
    exp_ml = -(-units * rows * 2 * 4 // 256) * 256
    assert need == exp_o + exp_ml
    bad = good_args(head_dim=96)
    assert lib.milo_attn_workspace_bytes(ctypes.byref(bad), _lib.MILO_PATH_DECODE) == 0
    assert lib.milo_attn_workspace_bytes(None, _lib.MILO_PATH_DECODE) == 0
    assert lib.milo_attn_workspace_bytes(ctypes.byref(a), 7) == 0


@pytest.mark.parametrize("over,code", [
    ({"struct_size": 8}, _lib.MILO_ERR_INVALID),
    ({"dtype": 7}, _lib.MILO_ERR_UNSUPPORTED),
    ({"n_q_heads": 15}, _lib.MILO_ERR_INVALID),
    ({"head_dim": 96}, _lib.MILO_ERR_UNSUPPORTED),
    ({"n_q_heads": 34, "n_kv_heads": 2}, _lib.MILO_ERR_UNSUPPORTED),   # group size 17
    ({"n_q_heads": 32, "n_kv_heads": 2, "dtype": _lib.MILO_F32}, _lib.MILO_ERR_UNSUPPORTED),  # G 16, fp32
    ({"scale": math.nan}, _lib.MILO_ERR_INVALID),
    ({"scale": math.inf}, _lib.MILO_ERR_INVALID),
    ({"q_len": 2}, _lib.MILO_ERR_INVALID),
    ({"batch": -1}, _lib.MILO_ERR_INVALID),
    ({"n_kv_heads": 0}, _lib.MILO_ERR_INVALID),
    ({"max_blocks_per_seq": -1}, _lib.MILO_ERR_INVALID),
    ({"batch": 1 << 20, "max_blocks_per_seq": 1 << 10}, _lib.MILO_ERR_UNSUPPORTED),  # 32-bit indices
    ({"q": None}, _lib.MILO_ERR_INVALID),
    ({"out": None}, _lib.MILO_ERR_INVALID),
    ({"seq_blocks": None}, _lib.MILO_ERR_INVALID),
    ({"pool": None}, _lib.MILO_ERR_INVALID),
    ({"q": FAKE + 2}, _lib.MILO_ERR_INVALID),
    ({"out": FAKE + 4}, _lib.MILO_ERR_INVALID),
    ({"pool": FAKE + 8}, _lib.MILO_ERR_INVALID),
    ({"k_tail": None}, _lib.MILO_ERR_INVALID),
    ({"tail_len": None}, _lib.MILO_ERR_INVALID),
    ({"tail_cap": 0}, _lib.MILO_ERR_INVALID),          # tail pointers set with no capacity
    ({"workspace": None}, _lib.MILO_ERR_WORKSPACE),
    ({"workspace": FAKE + 16}, _lib.MILO_ERR_WORKSPACE),
])
def test_decode_rejects_before_any_hip_call(over, code):
    a = good_args(**over)
    lib = _lib.load()
    a.workspace_bytes = 1 << 30
    assert call(a) == code


@pytest.mark.parametrize("over,code", [
    ({"dtype": _lib.MILO_F32}, _lib.MILO_ERR_UNSUPPORTED),   # the MFMA path is bf16 only
    ({"head_dim": 96}, _lib.MILO_ERR_UNSUPPORTED),           # head_dim 64 or 128
    ({"q_len": 2}, _lib.MILO_ERR_INVALID),                  # one query token per sequence
    ({"n_q_heads": 34, "n_kv_heads": 2}, _lib.MILO_ERR_UNSUPPORTED),   # group size 17
    ({"workspace": None}, _lib.MILO_ERR_WORKSPACE),
])
def test_shared_rejects_before_any_hip_call(over, code):
    lib = _lib.load()
    a = good_args(**{"head_dim": 128, **over})
    a.workspace_bytes = 1 << 30
    assert lib.milo_attn_decode_shared(ctypes.byref(a), None) == code
    assert lib.milo_attn_decode_shared(None, None) == _lib.MILO_ERR_INVALID


def test_shared_workspace_query():
    """Shared path: the batch's B * G query rows form one tile set per KV head;
    slots = block ranges + the tail's pieces (one per 64-token tile of the
    tail capacity, at most 8; 1 without tails) per (sequence, KV head), G
    rows each."""
    lib = _lib.load()
    for cap, pieces in ((0, 1), (256, 4), (100, 2), (4096, 8)):
        a = good_args(head_dim=128, batch=16, n_q_heads=28, n_kv_heads=4, max_blocks_per_seq=64, tail_cap=cap)
        need = lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_SHARED)
        # 16 * 7 = 112 rows -> one 128-row tile; 4 KV heads -> base 4 workgroups;
        # ranges = min(64, ceil(1024 / 4)) = 64 of one block each
        units, rows = 16 * 4 * (64 + pieces), 7
        exp_o = -(-units * rows * 128 * 4 // 256) * 256
        exp_ml = -(-units * rows * 2 * 4 // 256) * 256
        assert need == exp_o + exp_ml, (cap, need, exp_o + exp_ml)
    # head_dim 64 (the kernel pads its tiles to 128): the same slots, 64 floats per row
    a = good_args(head_dim=64, batch=16, n_q_heads=28, n_kv_heads=4, max_blocks_per_seq=64, tail_cap=256)
    units, rows = 16 * 4 * (64 + 4), 7
    exp = -(-units * rows * 64 * 4 // 256) * 256 + -(-units * rows * 2 * 4 // 256) * 256
    assert lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_SHARED) == exp
    assert lib.milo_attn_workspace_bytes(ctypes.byref(good_args(head_dim=96)), _lib.MILO_PATH_SHARED) == 0


def test_group_sizes_above_eight():
    """Group sizes 9-16 are served by the MFMA kernel (bf16 storage, head_dim
    64 or 128); decode then takes the chunked path's workspace layout (block
    ranges + a tail slot per (sequence, KV head), G rows each).  Other
    storage and groups above 16 are unsupported."""
    lib = _lib.load()
    for path in (_lib.MILO_PATH_DECODE, _lib.MILO_PATH_CHUNK, _lib.MILO_PATH_SHARED):
        q_len = 5 if path == _lib.MILO_PATH_CHUNK else 1
        for hd in (64, 128):
            a = good_args(head_dim=hd, n_q_heads=32, n_kv_heads=2, q_len=q_len)
            assert lib.milo_attn_workspace_bytes(ctypes.byref(a), path) > 0
        for over in ({"dtype": _lib.MILO_F32}, {"n_q_heads": 34}):
            b = good_args(**{"head_dim": 128, "n_q_heads": 32, "n_kv_heads": 2, "q_len": q_len, **over})
            assert lib.milo_attn_workspace_bytes(ctypes.byref(b), path) == 0
            assert call(b, path) if path != _lib.MILO_PATH_SHARED else True
    # decode, G = 16, batch 2, 4 blocks: 16 rows -> 1 query tile; base 2 * 2 * 1 = 4;
    # ranges = min(4, 256) = 4 of one block, + 1 tail slot
    a = good_args(head_dim=128, n_q_heads=32, n_kv_heads=2, batch=2, max_blocks_per_seq=4)
    units, rows = 2 * 2 * (4 + 1), 16
    exp = -(-units * rows * 128 * 4 // 256) * 256 + -(-units * rows * 2 * 4 // 256) * 256
    assert lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_DECODE) == exp
    b = good_args(head_dim=128, n_q_heads=32, n_kv_heads=2, dtype=_lib.MILO_F32)
    b.workspace_bytes = 1 << 30
    assert call(b) == _lib.MILO_ERR_UNSUPPORTED


def test_small_workspace_is_rejected():
    lib = _lib.load()
    a = good_args()
    need = lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_DECODE)
    a.workspace_bytes = need - 1
    assert call(a) == _lib.MILO_ERR_WORKSPACE


def test_null_args_and_empty_batch():
    lib = _lib.load()
    assert lib.milo_attn_decode(None, None) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_chunk(None, None) == _lib.MILO_ERR_INVALID
    a = good_args(batch=0, q=None, out=None, seq_blocks=None, workspace=None)
    assert call(a) == _lib.MILO_OK   # nothing to do, nothing launched


def test_python_binding_raises_without_a_built_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_noalloc_decode_checks_before_any_hip_call():
    """milo_attn_decode_noalloc ignores the workspace fields, applies every
    other check of milo_attn_decode, and refuses a call whose partials exceed
    its static buffer, all before any HIP call."""
    lib = _lib.load()
    a = good_args()
    a.workspace, a.workspace_bytes = None, 0
    bad = good_args(q=None)
    assert lib.milo_attn_decode_noalloc(ctypes.byref(bad), None) == _lib.MILO_ERR_INVALID
    bad = good_args(q_len=2)
    assert lib.milo_attn_decode_noalloc(ctypes.byref(bad), None) == _lib.MILO_ERR_INVALID
    a.batch, a.n_q_heads, a.n_kv_heads, a.head_dim, a.max_blocks_per_seq = 64, 28, 4, 128, 64
    need = lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_DECODE)
    assert need > _lib.MILO_NOALLOC_SCRATCH_BYTES      # 64 x 4 x 65 units x 7 rows: 60 MB
    assert lib.milo_attn_decode_noalloc(ctypes.byref(a), None) == _lib.MILO_ERR_WORKSPACE
    a.batch = 0
    assert lib.milo_attn_decode_noalloc(ctypes.byref(a), None) == _lib.MILO_OK


def test_plan_rejects_bad_arguments():
    lib = _lib.load()
    out = (ctypes.c_int32 * 8)()
    sb = (ctypes.c_int32 * 2)(0, 0)
    assert lib.milo_attn_plan_decode(None, 0, sb, None, -1, 1, 0, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, 0, None, None, 1, 1, 0, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, 2, sb, None, 1, 1, 2, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, 0, sb, None, 1, 0, 0, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, -1, sb, None, 1, 1, 0, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, 0, sb, None, 1, 1, 0, 64, out) == _lib.MILO_OK
    assert out[0] == 0
    # a negative or decreasing block range, or one past the descriptor table,
    # is refused before any descriptor is read
    blk = (_lib.MiloBlock * 2)()
    for bad in ((-1, 1), (1, 0), (0, 3), (2, 3)):
        sb2 = (ctypes.c_int32 * 2)(*bad)
        assert lib.milo_attn_plan_decode(blk, 2, sb2, None, 1, 1, 2, 64, out) == _lib.MILO_ERR_INVALID
    sb2 = (ctypes.c_int32 * 2)(0, 2)
    assert lib.milo_attn_plan_decode(blk, 2, sb2, None, 1, 1, 2, 64, out) == _lib.MILO_OK
    # unit indices are 32-bit
    big = (ctypes.c_int32 * 2)(0, 0)
    assert lib.milo_attn_plan_decode(blk, 2, big, None, 1, 1 << 16, 1 << 16, 64, out) == _lib.MILO_ERR_UNSUPPORTED


# --------------------------------------------------------------------------
# encode ABI (include/milo_encode.h)
# --------------------------------------------------------------------------
def enc_args(**over):
    a = _lib.MiloEncodeArgs()
    a.struct_size = ctypes.sizeof(_lib.MiloEncodeArgs)
    a.dtype = _lib.MILO_BF16
    a.n_blocks, a.n_kv_heads, a.head_dim, a.n_tokens = 3, 2, 128, 1000
    a.k = a.v = a.tok_start = a.blocks = a.pool = FAKE
    a.sigma = a.iters = FAKE
    a.workspace, a.workspace_bytes = FAKE, 1 << 30
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_encode_struct_size_and_workspace():
    assert ctypes.sizeof(_lib.MiloEncodeArgs) == 6 * 4 + 8 * 8 + 8
    lib = _lib.load()
    # 3 blocks x 2 heads x (K, V) matrices of 128 x 128 fp32 singular vectors
    assert lib.milo_encode_workspace_bytes(ctypes.byref(enc_args())) == 12 * 128 * 128 * 4
    assert lib.milo_encode_workspace_bytes(ctypes.byref(enc_args(head_dim=96))) == 0
    assert lib.milo_encode_workspace_bytes(None) == 0


@pytest.mark.parametrize("over,code", [
    ({"struct_size": 8}, _lib.MILO_ERR_INVALID),
    ({"dtype": 5}, _lib.MILO_ERR_UNSUPPORTED),
    ({"head_dim": 96}, _lib.MILO_ERR_UNSUPPORTED),
    ({"n_blocks": -1}, _lib.MILO_ERR_INVALID),
    ({"n_kv_heads": 0}, _lib.MILO_ERR_INVALID),
    ({"n_tokens": -5}, _lib.MILO_ERR_INVALID),
    ({"k": None}, _lib.MILO_ERR_INVALID),
    ({"k": FAKE + 8}, _lib.MILO_ERR_INVALID),
    ({"tok_start": None}, _lib.MILO_ERR_INVALID),
    ({"blocks": FAKE + 4}, _lib.MILO_ERR_INVALID),
    ({"workspace": None}, _lib.MILO_ERR_WORKSPACE),
    ({"workspace_bytes": 100}, _lib.MILO_ERR_WORKSPACE),
    ({"workspace": FAKE + 64}, _lib.MILO_ERR_WORKSPACE),
    ({"n_blocks": 1 << 30}, _lib.MILO_ERR_UNSUPPORTED),   # more matrices than one grid holds
])
def test_encode_rejects_before_any_hip_call(over, code):
    lib = _lib.load()
    a = enc_args(**over)
    assert lib.milo_encode_spectrum(ctypes.byref(a), None) == code
    assert lib.milo_encode_factors(ctypes.byref(a), None) == code


def test_encode_specific_pointer_checks():
    lib = _lib.load()
    assert lib.milo_encode_spectrum(ctypes.byref(enc_args(sigma=FAKE + 2)), None) == _lib.MILO_ERR_INVALID
    assert lib.milo_encode_factors(ctypes.byref(enc_args(pool=None)), None) == _lib.MILO_ERR_INVALID
    assert lib.milo_encode_factors(ctypes.byref(enc_args(pool=FAKE + 8)), None) == _lib.MILO_ERR_INVALID
    assert lib.milo_encode_spectrum(None, None) == _lib.MILO_ERR_INVALID
    # nothing to encode: no pointer is needed and nothing is launched
    empty = enc_args(n_blocks=0, k=None, v=None, tok_start=None, blocks=None, workspace=None, pool=None)
    assert lib.milo_encode_spectrum(ctypes.byref(empty), None) == _lib.MILO_OK
    assert lib.milo_encode_factors(ctypes.byref(empty), None) == _lib.MILO_OK


def test_encode_layout():
    from rank_attention_amd import encode as enc
    blocks, elems = enc.layout([37, 1024, 0], [5, 128, 0], [3, 1, 7], n_kv_heads=2, head_dim=128)
    assert list(blocks["ld_tok"]) == [40, 1024, 0]
    assert list(blocks["off"]) == [0, 2 * 8 * (40 + 128), 2 * 8 * (40 + 128) + 2 * 129 * (1024 + 128)]
    assert elems == blocks["off"][2] + 2 * 7 * 128
    assert all(o % 8 == 0 for o in blocks["off"])
    for bad in ([[1], [129], [0]], [[-1], [0], [0]], [[4], [0], [-2]]):
        with pytest.raises(ra.MiloError):
            enc.layout(*bad, n_kv_heads=1, head_dim=128)
    lib = _lib.load()
    assert lib.milo_encode_layout(None, None, None, 1, 1, 128, None, None) == _lib.MILO_ERR_INVALID


def rank_args(**over):
    a = _lib.MiloRankArgs()
    a.struct_size = ctypes.sizeof(_lib.MiloRankArgs)
    a.n_blocks, a.n_kv_heads, a.head_dim = 10, 2, 128
    a.budget_k, a.budget_v, a.r_min, a.unit = 10 * 8 + 320, 10 * 8 + 160, 8, 1
    a.sigma = a.ranks = a.entropy = FAKE
    a.workspace, a.workspace_bytes = FAKE, 1 << 20
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_rank_struct_and_workspace():
    assert ctypes.sizeof(_lib.MiloRankArgs) == 8 * 4 + 5 * 8
    lib = _lib.load()
    # 2 x 10 blocks x 120 units of fp32 gains
    assert lib.milo_rank_workspace_bytes(ctypes.byref(rank_args())) == -(-2 * 10 * 120 * 4 // 256) * 256
    assert lib.milo_rank_workspace_bytes(ctypes.byref(rank_args(unit=16))) == -(-2 * 10 * 7 * 4 // 256) * 256
    assert lib.milo_rank_workspace_bytes(ctypes.byref(rank_args(budget_k=5))) == 0


@pytest.mark.parametrize("over,code", [
    ({"struct_size": 4}, _lib.MILO_ERR_INVALID),
    ({"head_dim": 96}, _lib.MILO_ERR_UNSUPPORTED),
    ({"unit": 0}, _lib.MILO_ERR_INVALID),
    ({"r_min": 129}, _lib.MILO_ERR_INVALID),
    ({"r_min": -1}, _lib.MILO_ERR_INVALID),
    ({"budget_k": 79}, _lib.MILO_ERR_INVALID),              # below n_blocks * r_min
    ({"budget_v": 10 * 128 + 1}, _lib.MILO_ERR_INVALID),    # more than every block at full rank
    ({"unit": 16, "budget_k": 80 + 17}, _lib.MILO_ERR_INVALID),   # not whole units
    ({"sigma": None}, _lib.MILO_ERR_INVALID),
    ({"ranks": FAKE + 2}, _lib.MILO_ERR_INVALID),
    ({"workspace": None}, _lib.MILO_ERR_WORKSPACE),
    ({"workspace_bytes": 16}, _lib.MILO_ERR_WORKSPACE),
])
def test_rank_rejects_before_any_hip_call(over, code):
    assert _lib.load().milo_rank_allocate(ctypes.byref(rank_args(**over)), None) == code


def test_rank_empty_and_null():
    lib = _lib.load()
    assert lib.milo_rank_allocate(None, None) == _lib.MILO_ERR_INVALID
    empty = rank_args(n_blocks=0, budget_k=0, budget_v=0, sigma=None, ranks=None, workspace=None)
    assert lib.milo_rank_allocate(ctypes.byref(empty), None) == _lib.MILO_OK


def test_validate_rejects_bad_host_arguments():
    lib = _lib.load()
    a = good_args()
    assert lib.milo_attn_validate(ctypes.byref(a), _lib.MILO_PATH_DECODE, 4, 1000, None, None) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_validate(ctypes.byref(a), _lib.MILO_PATH_DECODE, 4, 1000, FAKE + 4, None) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_validate(ctypes.byref(a), _lib.MILO_PATH_DECODE, -1, 1000, FAKE, None) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_validate(ctypes.byref(a), _lib.MILO_PATH_DECODE, 4, -5, FAKE, None) == _lib.MILO_ERR_INVALID
    b = good_args(seq_blocks=None)
    assert lib.milo_attn_validate(ctypes.byref(b), _lib.MILO_PATH_DECODE, 4, 1000, FAKE, None) == _lib.MILO_ERR_INVALID
    c = good_args(head_dim=96)
    assert lib.milo_attn_validate(ctypes.byref(c), _lib.MILO_PATH_DECODE, 4, 1000, FAKE, None) == _lib.MILO_ERR_UNSUPPORTED
    assert lib.milo_attn_validate(None, _lib.MILO_PATH_DECODE, 4, 1000, FAKE, None) == _lib.MILO_ERR_INVALID


def test_quant_layout():
    from rank_attention_amd import encode as enc
    src = np.zeros(3, ra.BLOCK_DTYPE)
    src["n_tok"], src["rank_k"], src["rank_v"] = [37, 1024, 0], [5, 128, 0], [3, 1, 7]
    src["off"], src["ld_tok"] = [8, 1000, 5000], [40, 1024, 0]       # the source's placement is irrelevant
    blocks, nbytes = enc.quant_layout(src, n_kv_heads=2, head_dim=128)
    assert list(blocks["ld_tok"]) == [64, 1024, 0]
    assert list(blocks["n_tok"]) == [37, 1024, 0] and list(blocks["rank_k"]) == [5, 128, 0]
    # per head: n_tok * rk16 key codes, rank_v * ld value codes, bf16 W and W', then 8 bytes of
    # (a, b) per row padded to 16
    h0 = 37 * 16 + 3 * 64 + 8 * 256 + 64
    h1 = 1024 * 128 + 1 * 1024 + 129 * 256 + (8 * 129 + 15) // 16 * 16
    h2 = 0 * 0 + 7 * 0 + 7 * 256 + 64
    assert list(blocks["off"]) == [0, 2 * h0, 2 * h0 + 2 * h1]
    assert nbytes == 2 * (h0 + h1 + h2)
    assert all(o % 16 == 0 for o in blocks["off"])
    bad = src.copy()
    bad["rank_k"][0] = 129
    with pytest.raises(ra.MiloError):
        enc.quant_layout(bad, n_kv_heads=2, head_dim=128)
    lib = _lib.load()
    out = ctypes.c_int64(0)
    assert lib.milo_quant_layout(None, 1, 1, 128, None, ctypes.byref(out)) == _lib.MILO_ERR_INVALID
    assert lib.milo_quant_layout(None, 0, 1, 128, None, ctypes.byref(out)) == _lib.MILO_OK and out.value == 0


def quant_args(**over):
    a = _lib.MiloQuantArgs()
    a.struct_size = ctypes.sizeof(_lib.MiloQuantArgs)
    a.n_blocks, a.n_kv_heads, a.head_dim = 3, 2, 128
    a.src_pool = a.src_blocks = a.dst_pool = a.dst_blocks = FAKE
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    ({"struct_size": 8}, _lib.MILO_ERR_INVALID),
    ({"head_dim": 96}, _lib.MILO_ERR_UNSUPPORTED),
    ({"n_blocks": -1}, _lib.MILO_ERR_INVALID),
    ({"n_kv_heads": 0}, _lib.MILO_ERR_INVALID),
    ({"src_pool": None}, _lib.MILO_ERR_INVALID),
    ({"dst_blocks": None}, _lib.MILO_ERR_INVALID),
    ({"dst_pool": FAKE + 8}, _lib.MILO_ERR_INVALID),
    ({"n_blocks": 0, "src_pool": None}, _lib.MILO_OK),
])
def test_quantize_rejects_before_any_hip_call(over, code):
    assert ctypes.sizeof(_lib.MiloQuantArgs) == 4 * 4 + 4 * 8
    assert _lib.load().milo_quantize_factors(ctypes.byref(quant_args(**over)), None) == code
    assert _lib.load().milo_quantize_factors(None, None) == _lib.MILO_ERR_INVALID


def test_q8_storage_is_decode_only():
    lib = _lib.load()
    a = good_args(dtype=_lib.MILO_BF16_Q8)
    assert lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_DECODE) > 0
    c = good_args(dtype=_lib.MILO_BF16_Q8, head_dim=128, q_len=4, n_q_heads=4)
    for path in (_lib.MILO_PATH_CHUNK, _lib.MILO_PATH_SHARED):
        assert lib.milo_attn_workspace_bytes(ctypes.byref(c), path) == 0
    assert lib.milo_attn_chunk(ctypes.byref(c), None) == _lib.MILO_ERR_UNSUPPORTED
    d = good_args(dtype=_lib.MILO_BF16_Q8, head_dim=128, n_q_heads=4)
    assert lib.milo_attn_decode_shared(ctypes.byref(d), None) == _lib.MILO_ERR_UNSUPPORTED


def test_kivi_layout():
    """Sizes from the layout milo_attn.h states: per head a 16-byte header,
    per 64-token chunk 32 ng8 bytes of key scales and biases, 8 BITS ng8 x 8
    bytes of key codes, 256 ngv bytes of value scales and biases and
    16 BITS ntv x 8 bytes of value codes, then bf16 W and W'."""
    from rank_attention_amd import encode as enc
    src = np.zeros(3, ra.BLOCK_DTYPE)
    src["n_tok"], src["rank_k"], src["rank_v"] = [37, 1024, 0], [5, 128, 0], [33, 1, 7]
    src["off"], src["ld_tok"] = [8, 1000, 5000], [40, 1024, 0]
    for bits in (4, 2):
        blocks, nbytes = enc.kivi_layout(src, n_kv_heads=2, head_dim=128, bits=bits)
        assert list(blocks["ld_tok"]) == [64, 1024, 0]
        assert list(blocks["rank_k"]) == [5, 128, 0] and list(blocks["rank_v"]) == [33, 1, 7]
        def head(nch, r, rv):
            ng8, ngv, ntv = -(-r // 8), -(-rv // 32), -(-rv // 16)
            return 16 + nch * (32 * ng8 + 64 * bits * ng8 + 256 * ngv + 128 * bits * ntv) + 256 * (r + rv)
        h0, h1, h2 = head(1, 5, 33), head(16, 128, 1), head(0, 0, 7)
        assert h0 == 16 + (32 + 64 * bits + 512 + 128 * bits * 3) + 256 * 38
        assert list(blocks["off"]) == [0, 2 * h0, 2 * h0 + 2 * h1]
        assert nbytes == 2 * (h0 + h1 + h2)
        assert all(o % 16 == 0 for o in blocks["off"])
    bad = src.copy()
    bad["rank_v"][0] = 129
    with pytest.raises(ra.MiloError):
        enc.kivi_layout(bad, n_kv_heads=2, head_dim=128, bits=4)
    with pytest.raises(ra.MiloError):
        enc.kivi_layout(src, n_kv_heads=2, head_dim=128, bits=3)
    lib = _lib.load()
    out = ctypes.c_int64(0)
    assert lib.milo_kivi_layout(None, 1, 1, 128, 4, None, ctypes.byref(out)) == _lib.MILO_ERR_INVALID
    assert lib.milo_kivi_layout(None, 0, 1, 128, 2, None, ctypes.byref(out)) == _lib.MILO_OK and out.value == 0


@pytest.mark.parametrize("over,code", [
    ({"struct_size": 8}, _lib.MILO_ERR_INVALID),
    ({"head_dim": 96}, _lib.MILO_ERR_UNSUPPORTED),
    ({"n_blocks": -1}, _lib.MILO_ERR_INVALID),
    ({"src_pool": None}, _lib.MILO_ERR_INVALID),
    ({"dst_pool": FAKE + 8}, _lib.MILO_ERR_INVALID),
    ({"n_blocks": 0, "src_pool": None}, _lib.MILO_OK),
])
def test_quantize_kivi_rejects_before_any_hip_call(over, code):
    lib = _lib.load()
    for bits in (4, 2):
        assert lib.milo_quantize_kivi(ctypes.byref(quant_args(**over)), bits, None) == code
    for bits in (0, 1, 3, 8):
        assert lib.milo_quantize_kivi(ctypes.byref(quant_args()), bits, None) == _lib.MILO_ERR_INVALID
    assert lib.milo_quantize_kivi(None, 4, None) == _lib.MILO_ERR_INVALID


@pytest.mark.parametrize("dtype", [_lib.MILO_BF16_KV4, _lib.MILO_BF16_KV2])
def test_kivi_storage_is_decode_only_with_groups_up_to_eight(dtype):
    lib = _lib.load()
    for d in (64, 128):
        a = good_args(dtype=dtype, head_dim=d)
        assert lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_DECODE) > 0
    c = good_args(dtype=dtype, head_dim=128, q_len=4, n_q_heads=4)
    for path in (_lib.MILO_PATH_CHUNK, _lib.MILO_PATH_SHARED):
        assert lib.milo_attn_workspace_bytes(ctypes.byref(c), path) == 0
    assert lib.milo_attn_chunk(ctypes.byref(c), None) == _lib.MILO_ERR_UNSUPPORTED
    d = good_args(dtype=dtype, head_dim=128, n_q_heads=4)
    assert lib.milo_attn_decode_shared(ctypes.byref(d), None) == _lib.MILO_ERR_UNSUPPORTED
    g9 = good_args(dtype=dtype, head_dim=128, n_q_heads=9, n_kv_heads=1)
    assert lib.milo_attn_workspace_bytes(ctypes.byref(g9), _lib.MILO_PATH_DECODE) == 0
    assert lib.milo_attn_decode(ctypes.byref(g9), None) == _lib.MILO_ERR_UNSUPPORTED
    bad = good_args(dtype=5)
    assert lib.milo_attn_decode(ctypes.byref(bad), None) == _lib.MILO_ERR_UNSUPPORTED


def test_library_binds_to_torchs_hip_runtime():
    """A process that opens the library before touching torch must still have
    one HIP runtime: torch's bundled copy, which shares the soname of the ROCm
    one the library links.  Two runtimes would give the library a runtime that
    knows none of torch's streams."""
    import subprocess
    import sys
    code = ("from rank_attention_amd import _lib; _lib.load(); import torch; "
            "maps = open('/proc/self/maps').read().split(chr(10)); "
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert res.returncode == 0, res.stderr[-2000:]
    import ast
    libs = ast.literal_eval(res.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs
    import torch
    assert os.path.realpath(libs[0]).startswith(os.path.realpath(os.path.dirname(torch.__file__))), libs
