"""GPU test of the device-side table check (milo_attn_validate): a packed
cache passes; each contract rule, broken on purpose in a copy of the host
tables (the attention kernels are never run on them), is reported with the
offending index; several violations report the smallest rule."""
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


@pytest.fixture(scope="module")
def packed():
    cfg = synth.get_config("qwen7b_64k").with_(name="validate", batch=4, n_blocks=5, seed=51)
    wl = synth.make_workload(cfg, n_blocks=[5, 2, 0, 5], tail_len=[256, 0, 3, 100])
    return ra.pack(wl)


def check(pc, path=ra.MILO_PATH_DECODE, blocks=None, seq_blocks=None, tail_len=None, max_blocks=None,
          unit_order=None):
    import torch
    dc = ra.DeviceCache(pc)
    if blocks is not None:
        dc.blocks = torch.from_numpy(np.ascontiguousarray(blocks).view(np.uint8)).to("cuda")
    if seq_blocks is not None:
        dc.seq_blocks = torch.from_numpy(np.ascontiguousarray(seq_blocks, np.int32)).to("cuda")
    if tail_len is not None:
        dc.tail_len = torch.from_numpy(np.ascontiguousarray(tail_len, np.int32)).to("cuda")
    if max_blocks is not None:
        dc.max_blocks = max_blocks
    if unit_order is not None:
        dc.unit_order = torch.from_numpy(np.ascontiguousarray(unit_order, np.int32)).to("cuda")
    note(f"validate path={path}")
    return dc.validate(path)


def test_packed_cache_is_valid(packed):
    assert check(packed) is None
    assert check(packed, path=ra.MILO_PATH_SHARED) is None


@pytest.mark.parametrize("field,value,idx,rule", [
    ("rank_k", 129, 3, "rank"), ("rank_v", -1, 6, "rank"),
    ("ld_tok", 1000, 2, "tokens"), ("n_tok", -3, 0, "tokens"),
    ("off", 12, 4, "offset"), ("off", -8, 1, "offset"),
    ("off", 1 << 40, 7, "pool_bounds"),
])
def test_descriptor_rules(packed, field, value, idx, rule):
    blocks = packed.blocks.copy()
    blocks[idx][field] = value
    assert check(packed, blocks=blocks) == (rule, idx)


def test_csr_and_tail_rules(packed):
    sb = packed.seq_blocks.copy()
    sb[2] = sb[1] - 1                                  # sequence 1 ends before it starts
    assert check(packed, seq_blocks=sb) == ("seq_range", 1)
    sb = packed.seq_blocks.copy()
    sb[-1] = len(packed.blocks) + 5                    # last list runs past the table
    assert check(packed, seq_blocks=sb)[0] == "seq_range"
    assert check(packed, max_blocks=4) == ("too_many_blocks", 0)
    tl = packed.tail_len.copy()
    tl[2] = packed.k_tail.shape[2] + 1
    assert check(packed, tail_len=tl) == ("tail_len", 2)


def test_smallest_rule_wins_and_shared_checks_sequence_zero_only(packed):
    blocks = packed.blocks.copy()
    blocks[8]["rank_k"] = 500
    blocks[3]["off"] = 4
    assert check(packed, blocks=blocks) == ("rank", 8)
    sb = packed.seq_blocks.copy()
    sb[3] = sb[2] - 1                                  # breaks sequence 2's list only
    assert check(packed, seq_blocks=sb) == ("seq_range", 2)
    assert check(packed, path=ra.MILO_PATH_SHARED, seq_blocks=sb) is None


def test_schedule_rule(packed):
    """The decode schedule (unit_order) must be a permutation of the units:
    an entry out of range, or a unit named twice, is reported at the
    smallest offending position."""
    order = packed.unit_order.copy()
    assert check(packed, unit_order=order) is None
    n = len(order)
    bad = order.copy()
    bad[17] = n                                         # out of range
    assert check(packed, unit_order=bad) == ("unit_order", 17)
    bad = order.copy()
    bad[40] = -3
    assert check(packed, unit_order=bad) == ("unit_order", 40)
    bad = order.copy()
    bad[30] = bad[9]                                    # unit named at 9 and 30; unit bad[30] unlisted
    assert check(packed, unit_order=bad) == ("unit_order", 9)
    # a descriptor rule (smaller rule number) still wins over the schedule rule
    blocks = packed.blocks.copy()
    blocks[2]["rank_v"] = 1000
    assert check(packed, blocks=blocks, unit_order=bad) == ("rank", 2)
