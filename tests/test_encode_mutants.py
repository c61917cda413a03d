"""The encode pins catch plausible mistakes in the encode oracle.

Each case plants one mistake in a copy of ``oracle/encode.py`` (loaded as a
separate module, on the CPU) and checks that at least one pin of
``test_encode_pins`` fails when the pins run against the mutant.
"""
import importlib.util
import os
import types

import pytest

from oracle import encode as real
from tests import test_encode_pins as pins

SRC = real.__file__

MUTANTS = {
    "smallest_directions": ("    w = vt[:r]\n", "    w = vt[::-1][:r]\n"),
    "basis_columns_not_rows": ("    w = vt[:r]\n", "    w = vt.T[:r]\n"),
    "u_without_sigma": ("    u = x @ w.T\n",
                        "    u = x @ w.T\n    u = u / np.maximum(np.linalg.norm(u, axis=0), 1e-300)\n"),
    "sigma_squared": ("    sf[:len(s)] = s\n", "    sf[:len(s)] = s ** 2\n"),
    "sigma_padded_at_front": ("    sf[:len(s)] = s\n", "    sf[d - len(s):] = s\n"),
    "one_rank_short": ("    w = vt[:r]\n", "    w = vt[:max(r - 1, 0)]\n"),
    "values_from_keys": ("                a[g, kv] = approx(ctx.dense_f64(kv, b, g), int(ranks[b][kv]))",
                         "                a[g, kv] = approx(ctx.dense_f64(0, b, g), int(ranks[b][kv]))"),
}

PINS = [
    pins.test_rank1_matches_brute_force_direction_search,
    pins.test_rank2_of_three_columns_matches_brute_force_normal_search,
    lambda: [pins.test_known_singular_value_decomposition(T, d) for T, d in [(40, 8), (8, 8), (5, 8)]],
    pins.test_factor_shapes_orthonormal_rows_and_u_equals_xwt,
    pins.test_full_rank_reproduces_block_and_rank_zero_is_empty,
    pins.test_empty_block,
    pins.test_column_permutation_equivariance,
    pins.test_planted_context_is_recovered_to_rounding,
    pins.test_context_helpers_agree_with_block_calls,
]


def _mutant(old, new) -> types.ModuleType:
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("encode_mutant")
    exec(compile(src.replace(old, new, 1), "encode_mutant", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_the_real_oracle():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(pins, "enc", _mutant(*MUTANTS[name]))
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"no pin caught mutant {name}"
