"""Pins of the 8-bit row quantisation oracle: the round-trip bound, grid
points, constant and empty rows, and where each code comes from."""
import numpy as np
import pytest

from oracle import quant


def test_round_trip_error_is_at_most_half_a_step():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((20, 300)) * rng.uniform(0.01, 10, (20, 1))).astype(np.float32)
    c, s, b = quant.quantize_rows(x)
    err = np.abs(quant.dequantize_rows(c, s, b) - x.astype(np.float64))
    # half a step, plus the fp32 rounding of (x - lo) / scale before it is rounded to an integer
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5))
    assert np.all(c.min(axis=1) == 0) and np.all(c.max(axis=1) == 255)   # extremes hit both ends


def test_grid_points_are_exact():
    lo, step = np.float32(-3.0), np.float32(0.0625)                      # binary: every step exact
    k = np.array([0, 1, 2, 100, 200, 254, 255], np.float32)
    x = (lo + step * k)[None, :].astype(np.float32)
    x = np.concatenate([x, np.array([[lo + step * 255]], np.float32)], axis=1)
    c, s, b = quant.quantize_rows(x)
    assert s[0] == step and b[0] == lo
    assert list(c[0]) == [0, 1, 2, 100, 200, 254, 255, 255]
    assert np.array_equal(quant.dequantize_rows(c, s, b)[0], x[0].astype(np.float64))


def test_half_way_codes_round_to_even():
    lo, step = np.float32(0.0), np.float32(1.0)
    x = np.array([[0.0, 0.5, 1.5, 2.5, 255.0]], np.float32)               # scale = 1: (x - lo) / scale = x
    c, s, b = quant.quantize_rows(x)
    assert s[0] == 1.0 and list(c[0]) == [0, 0, 2, 2, 255]


def test_constant_and_empty_rows():
    c, s, b = quant.quantize_rows(np.full((2, 5), 1.25, np.float32))
    assert np.all(c == 0) and np.all(s == 0) and np.all(b == np.float32(1.25))
    assert np.all(quant.dequantize_rows(c, s, b) == 1.25)
    c, s, b = quant.quantize_rows(np.zeros((3, 0), np.float32))
    assert c.shape == (3, 0) and np.all(s == 0)


def test_codes_follow_each_rows_own_range():
    x = np.array([[0.0, 10.0, 5.0], [-1.0, -1.0, 1.0]], np.float32)
    c, s, b = quant.quantize_rows(x)
    assert list(b) == [0.0, -1.0]
    np.testing.assert_allclose(s, [10 / 255, 2 / 255], rtol=1e-7)
    # exactly 127.5 in real arithmetic, but fp32 10/255 rounds up, so 5/scale is
    # 127.49999 and the code is 127: the decision is the fp32 one
    assert list(c[0]) == [0, 255, 127] and list(c[1]) == [0, 0, 255]


def _grid_rows(rng, rows, n):
    """Rows whose values lie on their own 256-level grid lo + step * k, k in
    [0, 255] with both ends hit, steps and offsets exact in bf16 and fp32."""
    k = rng.integers(0, 256, size=(rows, n))
    k[:, 0], k[:, -1] = 0, 255
    step = 2.0 ** rng.integers(-9, -5, size=(rows, 1))          # differs per row
    lo = -step * rng.integers(0, 256, size=(rows, 1))
    return lo + step * k


def _grid_workload():
    import synth
    cfg = synth.get_config("tiny").with_(dtype="bf16", n_kv_heads=2, n_q_heads=4)
    wl = synth.make_workload(cfg, variant="sharp")
    rng = np.random.default_rng(7)
    for b in wl.blocks[0]:
        for g in range(cfg.n_kv_heads):
            for arr in (b.ut, b.upt):
                x = _grid_rows(rng, arr.shape[1], arr.shape[2]).astype(np.float32)
                arr[g] = synth.gen.f32_to_bf16_bits(x)
                assert np.array_equal(synth.gen.bf16_bits_to_f32(arr[g]), x)   # exact in bf16
    return wl


def test_grid_factors_quantise_exactly_and_attention_is_unchanged():
    import oracle
    wl = _grid_workload()
    o1, l1 = oracle.attend(wl)
    o2, l2 = quant.attend_q8(wl)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_off_grid_factors_change_the_attention_within_the_step_bound():
    # generic factors: every dequantized element within half a step of the
    # original, and the attention moved (so the quantised path is really taken)
    import oracle, synth
    cfg = synth.get_config("tiny").with_(dtype="bf16")
    wl = synth.make_workload(cfg, variant="sharp")
    _, blocks, _, _, _ = oracle.logical_from_workload(wl)
    qb = quant.quantize_logical_blocks(blocks)
    for (U, W, Up, Wp), (Uq, Wq, Upq, Wpq) in zip(blocks[0], qb[0]):
        assert Wq is W and Wpq is Wp
        for X, Xq in ((U, Uq), (Up, Upq)):
            step = (X.max(axis=1) - X.min(axis=1)) / 255      # per rank component (column of U)
            assert np.all(np.abs(Xq - X) <= step[:, None, :] * (0.5 + 1e-5))
            assert np.mean(Xq != X) > 0.5                      # generic values are off the grid
    o1, _ = oracle.attend(wl)
    o2, _ = quant.attend_q8(wl)
    assert 1e-4 < np.abs(o1 - o2).max() < 5e-2
