"""The rank-allocation pins catch plausible mistakes in its oracle (each
planted in a copy of ``oracle/rank_alloc.py`` loaded as its own module)."""
import types

import pytest

from oracle import rank_alloc as real
from tests import test_rank_alloc_pins as pins

MUTANTS = {
    "gain_without_entropy": ("    return H * float(p[r:r + unit].sum())", "    return float(p[r:r + unit].sum())"),
    "next_component_off_by_one": ("p[r:r + unit]", "p[r + 1:r + unit + 1]"),
    "argmin": ("            if g > best_g:", "            if best < 0 or g < best_g:"),
    "ties_to_highest_index": ("            if g > best_g:", "            if g >= best_g:"),
    "no_renormalisation": ("    tot = p.sum()\n    if tot > 0:\n        p /= tot\n", ""),
    "energy_not_squared": ("        e = s[g] ** 2", "        e = np.abs(s[g])"),
    "one_unit_short": ("    for _ in range(extra // unit):", "    for _ in range(extra // unit - 1):"),
    "entropy_log2": ("    H = float(-(nz * np.log(nz)).sum())", "    H = float(-(nz * np.log2(nz)).sum())"),
}

PINS = [
    pins.test_entropy_closed_forms,
    pins.test_head_averaging_and_empty_heads,
    pins.test_worked_allocation,
    pins.test_worked_allocation_where_entropy_decides,
    lambda: [pins.test_greedy_equals_exhaustive_optimum(r, u) for r, u in [(0, 1), (1, 1), (0, 2), (1, 2)]],
    pins.test_budget_conservation_and_bounds,
    pins.test_slowly_decaying_spectrum_gets_more_rank,
    pins.test_scale_invariance_and_tie_break,
    pins.test_zero_energy_block_keeps_minimum_until_others_are_full,
    pins.test_invalid_budgets,
]


def _mutant(old, new):
    src = open(real.__file__).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("rank_alloc_mutant")
    exec(compile(src.replace(old, new, 1), "rank_alloc_mutant", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_the_real_oracle():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(pins, "ra_", _mutant(*MUTANTS[name]))
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, Exception):
            failed += 1
    assert failed > 0, f"no pin caught mutant {name}"
