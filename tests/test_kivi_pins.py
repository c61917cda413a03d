"""Pins of the KIVI-style quantisation oracle (oracle/kivi.py): the
round-trip bound, grid points, ties, the group boundaries along tokens (keys)
and along rank components (values), the fp16 scale and bias that decide the
codes, and attention over factors that the grid represents exactly."""
import numpy as np
import pytest

from oracle import kivi


@pytest.mark.parametrize("bits", [2, 4])
def test_round_trip_error_is_within_half_a_step(bits):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((30, 200)) * rng.uniform(0.05, 8, (30, 1))).astype(np.float32)
    c, a, b = kivi.quantize_groups(x, bits)
    lo = x.min(axis=1).astype(np.float64)
    err = np.abs(kivi.dequantize_groups(c, a, b) - x.astype(np.float64))
    # half a step, the fp16 rounding of the bias (codes saturate at 0 and L,
    # so a bias below or above lo costs at most that distance) and the fp32
    # rounding before the integer decision
    bound = a.astype(np.float64)[:, None] * (0.5 + 1e-3) + np.abs(b.astype(np.float64) - lo)[:, None]
    # the top of the range: (hi - b) / a may exceed L by the fp16 rounding of a
    bound = bound + (2 ** bits - 1) * np.abs(a.astype(np.float64) - (x.max(1) - x.min(1)) / (2 ** bits - 1))[:, None]
    assert np.all(err <= bound)
    assert np.all(c.max(axis=1) == 2 ** bits - 1) and np.all(c.min(axis=1) == 0)
    assert c.max() <= 2 ** bits - 1


@pytest.mark.parametrize("bits", [2, 4])
def test_grid_points_are_exact(bits):
    L = 2 ** bits - 1
    lo, step = np.float32(-1.5), np.float32(0.25)          # exact in fp16 and fp32
    k = np.arange(L + 1, dtype=np.float32)
    x = np.stack([lo + step * k, lo + step * k[::-1]]).astype(np.float32)
    c, a, b = kivi.quantize_groups(x, bits)
    assert np.all(a == np.float16(step)) and np.all(b == np.float16(lo))
    assert list(c[0]) == list(range(L + 1)) and list(c[1]) == list(range(L, -1, -1))
    assert np.array_equal(kivi.dequantize_groups(c, a, b), x.astype(np.float64))


def test_half_way_codes_round_to_even():
    # 4 bits, range 15 -> scale 1, bias 0: (x - b) / a = x
    x = np.array([[0.0, 0.5, 1.5, 2.5, 13.5, 15.0]], np.float32)
    c, a, b = kivi.quantize_groups(x, 4)
    assert a[0] == 1 and b[0] == 0 and list(c[0]) == [0, 0, 2, 2, 14, 15]


def test_constant_and_empty_groups():
    c, a, b = kivi.quantize_groups(np.full((2, 7), -2.25, np.float32), 2)
    assert np.all(c == 0) and np.all(a == 0) and np.all(kivi.dequantize_groups(c, a, b) == -2.25)
    c, a, b = kivi.quantize_groups(np.zeros((3, 0), np.float32), 4)
    assert c.shape == (3, 0)


def test_codes_are_decided_with_the_stored_fp16_scale():
    # range 1 over 15 levels: fp32 scale 0.0666667 rounds to fp16 0.06665039;
    # x = 0.5 then gives (0.5 - 0) / 0.06665039 = 7.5018 -> 8 with the fp16
    # scale, while the fp32 scale gives exactly 7.4999995 -> 7
    x = np.array([[0.0, 0.5, 1.0]], np.float32)
    c, a, b = kivi.quantize_groups(x, 4)
    assert a[0] == np.float16(1.0 / 15.0) and float(a[0]) != np.float32(1.0) / np.float32(15.0)
    assert c[0, 1] == 8
    assert np.float32(0.5) / (np.float32(1.0) / np.float32(15.0)) < 7.5   # the fp32 path would round to 7


def test_key_groups_run_along_tokens_per_rank_component():
    """Keys: each rank component has its own scale in each 64-token group:
    a component that is tiny everywhere stays accurate next to a large one,
    and a jump in range at token 64 starts a new group."""
    rng = np.random.default_rng(5)
    T, r = 150, 3
    U = rng.standard_normal((T, r)).astype(np.float32)
    U[:, 1] *= 1e-3                     # a small component
    U[64:128, 2] *= 100.0               # the second token group of component 2 is large
    codes, sc, bi = kivi.quantize_keys(U, 4)
    assert codes.shape == (T, r) and sc.shape == (3, r)
    deq = kivi.dequantize_keys(codes, sc, bi)
    for j, (t0, t1) in enumerate([(0, 64), (64, 128), (128, 150)]):
        for k in range(r):
            seg = U[t0:t1, k].astype(np.float64)
            step = (seg.max() - seg.min()) / 15
            assert np.max(np.abs(deq[t0:t1, k] - seg)) <= step * 0.51 + 1e-3 * abs(seg).max()
    assert float(sc[1, 2]) > 50 * float(sc[0, 2])       # group boundary at token 64


def test_value_groups_run_along_rank_components_per_token():
    """Values: each token has its own scale per run of 32 rank components:
    a token with a large entry loses precision only in its own group."""
    rng = np.random.default_rng(6)
    T, rv = 10, 70
    Up = rng.standard_normal((T, rv)).astype(np.float32)
    Up[4, 3] = 500.0                     # token 4, first rank group
    codes, sc, bi = kivi.quantize_values(Up, 4)
    assert sc.shape == (T, 3)
    deq = kivi.dequantize_values(codes, sc, bi)
    err = np.abs(deq - Up)
    assert err[4, :32].max() > 1.0                        # the outlier's group is coarse
    assert err[4, 32:].max() < 0.5 and np.delete(err, 4, axis=0).max() < 0.5   # the rest is not


def _grid_workload(bits):
    """A small bf16 workload whose key factors lie, per rank component and
    64-token group, and whose value factors lie, per token and 32-rank group,
    on their own 2^bits-level grids (steps and offsets exact in bf16 and fp16)."""
    import synth
    L = 2 ** bits - 1
    cfg = synth.get_config("tiny").with_(dtype="bf16", n_kv_heads=2, n_q_heads=4)
    wl = synth.make_workload(cfg, variant="sharp")
    rng = np.random.default_rng(8)
    for blk in wl.blocks[0]:
        T = blk.n_tok
        for g in range(cfg.n_kv_heads):
            ut = np.zeros(blk.ut[g].shape, np.float32)     # [r][T]
            for j in range(0, T, 64):
                n = min(64, T - j)
                k = rng.integers(0, L + 1, size=(ut.shape[0], n))
                k[:, 0], k[:, -1] = 0, L
                step = 2.0 ** rng.integers(-4, 0, size=(ut.shape[0], 1))
                lo = -step * rng.integers(0, L + 1, size=(ut.shape[0], 1))
                ut[:, j:j + n] = lo + step * k
            upt = np.zeros(blk.upt[g].shape, np.float32)   # [r'][T]
            for j in range(0, upt.shape[0], 32):
                n = min(32, upt.shape[0] - j)
                k = rng.integers(0, L + 1, size=(n, T))
                k[0, :], k[-1, :] = 0, L
                step = 2.0 ** rng.integers(-4, 0, size=(1, T))
                lo = -step * rng.integers(0, L + 1, size=(1, T))
                upt[j:j + n] = lo + step * k
            blk.ut[g] = synth.gen.f32_to_bf16_bits(ut)
            blk.upt[g] = synth.gen.f32_to_bf16_bits(upt)
            assert np.array_equal(synth.gen.bf16_bits_to_f32(blk.ut[g]), ut)
    return wl


@pytest.mark.parametrize("bits", [2, 4])
def test_grid_factors_quantise_exactly_and_attention_is_unchanged(bits):
    import oracle
    wl = _grid_workload(bits)
    o1, l1 = oracle.attend(wl)
    o2, l2 = kivi.attend_kivi(wl, bits)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_generic_factors_move_the_attention_more_at_two_bits():
    import oracle, synth
    cfg = synth.get_config("tiny").with_(dtype="bf16")
    wl = synth.make_workload(cfg, variant="sharp")
    o, _ = oracle.attend(wl)
    e4 = np.abs(kivi.attend_kivi(wl, 4)[0] - o).max()
    e2 = np.abs(kivi.attend_kivi(wl, 2)[0] - o).max()
    assert 1e-4 < e4 < e2 < 1.0


def test_codes_saturate_and_follow_the_stored_fp16_bias():
    # lo = 1000.3 rounds to the fp16 bias 1000.5 (spacing 0.5 there), above the
    # whole range 1000.3 .. 1000.315: every code decided against the stored
    # bias is negative before clamping and saturates at 0, so every value
    # dequantises to the bias; a decision against the fp32 minimum would give
    # codes 0 .. 15 instead
    x = (np.float32(1000.3) + np.float32(0.001) * np.arange(16, dtype=np.float32))[None, :]
    c, a, b = kivi.quantize_groups(x, 4)
    assert float(b[0]) == 1000.5 and float(a[0]) > 0
    assert np.all(c == 0)
    assert np.all(kivi.dequantize_groups(c, a, b) == 1000.5)


@pytest.mark.parametrize("bits", [2, 4])
def test_quantised_factors_take_at_most_2_to_the_bits_values_per_group(bits):
    """Counting, not arithmetic: after quantisation every key group (one rank
    component over 64 tokens) and every value group (one token over 32 rank
    components) of every block holds at most 2^bits distinct values, some
    hold exactly that many, and W and W' pass through unchanged."""
    import oracle, synth
    cfg = synth.get_config("tiny").with_(dtype="bf16", n_kv_heads=2, n_q_heads=4)
    wl = synth.make_workload(cfg, variant="sharp")
    _, blocks, _, _, _ = oracle.logical_from_workload(wl)
    qb = kivi.quantize_logical_blocks(blocks, bits)
    full = 0
    for seq, qseq in zip(blocks, qb):
        for (U, W, Up, Wp), (Uq, Wq, Upq, Wpq) in zip(seq, qseq):
            assert np.array_equal(W, Wq) and np.array_equal(Wp, Wpq)
            assert Uq.shape == U.shape and Upq.shape == Up.shape
            for g in range(U.shape[0]):
                for t0 in range(0, U.shape[1], 64):
                    for k in range(U.shape[2]):
                        n = len(np.unique(Uq[g, t0:t0 + 64, k]))
                        assert n <= 2 ** bits
                        full += n == 2 ** bits
                for t in range(Up.shape[1]):
                    for k0 in range(0, Up.shape[2], 32):
                        n = len(np.unique(Upq[g, t, k0:k0 + 32]))
                        assert n <= 2 ** bits
                        full += n == 2 ** bits
    assert full > 100
