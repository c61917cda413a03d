"""The 8-bit quantisation pins catch plausible mistakes in its oracle (each
planted in a copy of ``oracle/quant.py`` loaded as its own module)."""
import types

import pytest

from oracle import quant as real
from tests import test_quant_pins as pins

MUTANTS = {
    "floor_not_round": ("q = np.rint((x[k] - lo[k]) / scale[k])", "q = np.floor((x[k] - lo[k]) / scale[k])"),
    "round_half_up": ("q = np.rint((x[k] - lo[k]) / scale[k])", "q = np.floor((x[k] - lo[k]) / scale[k] + np.float32(0.5))"),
    "256_levels": ("scale = (hi - lo) / np.float32(255.0)", "scale = (hi - lo) / np.float32(256.0)"),
    "symmetric_no_bias": ("return codes, scale.astype(np.float32), lo.astype(np.float32)",
                          "return codes, scale.astype(np.float32), np.zeros_like(lo, dtype=np.float32)"),
    "float64_decision": ("    x = np.asarray(x, dtype=np.float32)", "    x = np.asarray(x, dtype=np.float64)"),
    "groups_per_token": ("Uq[g] = dequantize_rows(*quantize_rows(U[g].T.astype(np.float32))).T",
                         "Uq[g] = dequantize_rows(*quantize_rows(U[g].astype(np.float32)))"),
    "values_not_quantised": ("Upq[g] = dequantize_rows(*quantize_rows(Up[g].T.astype(np.float32))).T",
                             "Upq[g] = Up[g]"),
    "bias_dropped_on_dequantize": ("            + np.asarray(bias, np.float64)[:, None])", "            + 0.0)"),
}

PINS = [
    pins.test_round_trip_error_is_at_most_half_a_step,
    pins.test_grid_points_are_exact,
    pins.test_half_way_codes_round_to_even,
    pins.test_constant_and_empty_rows,
    pins.test_codes_follow_each_rows_own_range,
    pins.test_grid_factors_quantise_exactly_and_attention_is_unchanged,
    pins.test_off_grid_factors_change_the_attention_within_the_step_bound,
]


def _mutant(old, new):
    src = open(real.__file__).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("quant_mutant")
    exec(compile(src.replace(old, new, 1), "quant_mutant", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_the_real_oracle():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(pins, "quant", _mutant(*MUTANTS[name]))
    failed = 0
    for pin in PINS:
        try:
            pin()
        except Exception:
            failed += 1
    assert failed > 0, f"no pin caught mutant {name}"
