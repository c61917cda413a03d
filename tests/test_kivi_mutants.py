"""The KIVI-style quantisation pins catch plausible mistakes in its oracle
(each planted in a copy of ``oracle/kivi.py`` loaded as its own module)."""
import types

import pytest

from oracle import kivi as real
from tests import test_kivi_pins as pins

MUTANTS = {
    "floor_not_round": ("q = np.rint((x - b[:, None])", "q = np.floor((x - b[:, None])"),
    "round_half_up": ("q = np.rint((x - b[:, None]) / np.where(ok, a, np.float32(1))[:, None])",
                      "q = np.floor((x - b[:, None]) / np.where(ok, a, np.float32(1))[:, None] + np.float32(0.5))"),
    "2_to_the_bits_levels": ("return (1 << bits) - 1", "return 1 << bits"),
    "symmetric_no_bias": ("b16 = lo.astype(np.float16)", "b16 = np.zeros_like(lo, dtype=np.float16)"),
    "fp32_scale_decides": ("a = a16.astype(np.float32)", "a = (hi - lo) / L"),
    "fp32_bias_decides": ("b = b16.astype(np.float32)", "b = lo"),
    "no_clamp": ("codes = np.where(ok[:, None], np.clip(q, 0, L), 0).astype(np.uint8)",
                 "codes = np.where(ok[:, None], q, 0).astype(np.int64).astype(np.uint8)"),
    "keys_grouped_per_token": ("Uq[g] = dequantize_keys(*quantize_keys(U[g], bits))",
                               "Uq[g] = dequantize_values(*quantize_values(U[g], bits))"),
    "values_grouped_per_channel": ("Upq[g] = dequantize_values(*quantize_values(Up[g], bits))",
                                   "Upq[g] = dequantize_keys(*quantize_keys(Up[g], bits))"),
    "keys_not_quantised": ("Uq[g] = dequantize_keys(*quantize_keys(U[g], bits))", "Uq[g] = U[g]"),
    "values_not_quantised": ("Upq[g] = dequantize_values(*quantize_values(Up[g], bits))", "Upq[g] = Up[g]"),
    "key_groups_of_128": ("KEY_GROUP_TOKENS = 64", "KEY_GROUP_TOKENS = 128"),
    "key_groups_of_32": ("KEY_GROUP_TOKENS = 64", "KEY_GROUP_TOKENS = 32"),
    "value_groups_of_64": ("VALUE_GROUP_RANKS = 32", "VALUE_GROUP_RANKS = 64"),
    "value_groups_of_16": ("VALUE_GROUP_RANKS = 32", "VALUE_GROUP_RANKS = 16"),
    "bias_dropped_on_dequantize": ("            + np.asarray(bias, np.float64)[:, None])", "            + 0.0)"),
    "scale_squared_on_dequantize": ("return (np.asarray(scale, np.float64)[:, None] * np.asarray(codes, np.float64)",
                                    "return (np.asarray(scale, np.float64)[:, None] ** 2 * np.asarray(codes, np.float64)"),
}


def _pins():
    out = []
    for name in dir(pins):
        f = getattr(pins, name)
        if name.startswith("test_") and callable(f):
            out.append(f)
    return out


def _call(pin):
    """Run one pin; parametrised pins run at both widths."""
    import inspect
    if "bits" in inspect.signature(pin).parameters:
        for bits in (2, 4):
            pin(bits)
    else:
        pin()


def _mutant(old, new):
    src = open(real.__file__).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("kivi_mutant")
    exec(compile(src.replace(old, new, 1), "kivi_mutant", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_the_real_oracle():
    for pin in _pins():
        _call(pin)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(pins, "kivi", _mutant(*MUTANTS[name]))
    failed = []
    for pin in _pins():
        try:
            _call(pin)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
