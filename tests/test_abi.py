"""The C-ABI library: it loads, exports every declared symbol, and rejects
host-checkable faults before any HIP call (so these run without a GPU)."""
import ctypes
import math
import os
import re

import pytest

import rank_attention_amd as ra
from rank_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "milo_attn.h")

FAKE = 0x10000  # 64 KiB-aligned non-null address; never dereferenced by these calls


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(milo_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_struct_size():
    assert ra.abi_version() == 2
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
    ({"n_q_heads": 32, "n_kv_heads": 2}, _lib.MILO_ERR_UNSUPPORTED),
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
    ({"head_dim": 64}, _lib.MILO_ERR_UNSUPPORTED),           # and head_dim 128 only
    ({"q_len": 2}, _lib.MILO_ERR_INVALID),                  # one query token per sequence
    ({"n_q_heads": 32, "n_kv_heads": 2}, _lib.MILO_ERR_UNSUPPORTED),
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
    slots = block ranges + 1 tail slot per (sequence, KV head), G rows each."""
    lib = _lib.load()
    a = good_args(head_dim=128, batch=16, n_q_heads=28, n_kv_heads=4, max_blocks_per_seq=64)
    need = lib.milo_attn_workspace_bytes(ctypes.byref(a), _lib.MILO_PATH_SHARED)
    # 16 * 7 = 112 rows -> one 128-row tile; 4 KV heads -> base 4 workgroups;
    # ranges = min(64, ceil(1024 / 4)) = 64 of one block each
    units, rows = 16 * 4 * (64 + 1), 7
    exp_o = -(-units * rows * 128 * 4 // 256) * 256
    exp_ml = -(-units * rows * 2 * 4 // 256) * 256
    assert need == exp_o + exp_ml
    assert lib.milo_attn_workspace_bytes(ctypes.byref(good_args(head_dim=64)), _lib.MILO_PATH_SHARED) == 0


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


def test_plan_rejects_bad_arguments():
    lib = _lib.load()
    out = (ctypes.c_int32 * 8)()
    sb = (ctypes.c_int32 * 2)(0, 0)
    assert lib.milo_attn_plan_decode(None, sb, None, -1, 1, 0, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, None, None, 1, 1, 0, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, sb, None, 1, 1, 2, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, sb, None, 1, 0, 0, 64, out) == _lib.MILO_ERR_INVALID
    assert lib.milo_attn_plan_decode(None, sb, None, 1, 1, 0, 64, out) == _lib.MILO_OK
    assert out[0] == 0
