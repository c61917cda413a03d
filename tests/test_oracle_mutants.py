"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), loads the mutant in place of the real oracle and
checks that at least one pin of ``test_oracle_pins`` fails on it.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "milo_oracle.c")

MUTANTS = {
    "transposed_W": ("kr[c] += u * wr[c];", "kr[c] += u * W[(size_t)c * r + k];"),
    "drop_value_term": ("for (int k = 0; k < rv; ++k) {", "for (int k = 0; k < rv - 1; ++k) {"),
    "causal_off_by_one": ("int64_t vis_tail = (int64_t)L - Q + j + 1;", "int64_t vis_tail = (int64_t)L - Q + j;"),
    "gqa_modulo": ("const int j = row / G, h = g * G + row % G;", "const int j = row / G, h = g + Hkv * (row % G);"),
    "scale_outside_exp": ("s[t] = scale * acc;", "s[t] = acc;"),
    "no_max_shift_in_lse": ("*lse = mx + log(z);", "*lse = log(z);"),
    "tail_dropped": ("attend_row(a->q + qi * d, K, V, nblk_tok + vis_tail,", "attend_row(a->q + qi * d, K, V, nblk_tok,"),
    "tail_from_wrong_head": ("const size_t src = (((size_t)i * Hkv + g) * a->tail_cap + t) * d;",
                             "const size_t src = (((size_t)i * Hkv + 0) * a->tail_cap + t) * d;"),
    "values_from_key_factor": ("const double u = Up[(size_t)t * rv + k];", "const double u = U[(size_t)t * rv + k];"),
    "exp_without_shift": ("s[t] = exp(s[t] - mx); z += s[t];", "s[t] = exp(s[t]); z += s[t];"),
}

PIN_TESTS = [
    lambda: [pins.test_full_rank_identity_matches_sdpa(Q, L) for Q, L in
             [(1, [4, 0, 7]), (3, [3, 5, 6]), (5, [5, 9, 5])]],
    pins.test_absorbed_order_plain_loops,
    pins.test_weights_sum_to_one,
    pins.test_zero_query_gives_mean_of_visible_rows,
    pins.test_single_visible_token,
    pins.test_linear_in_value_projection,
    pins.test_empty_context,
    pins.test_rank_zero_block_counts_in_normaliser,
    pins.test_split_merge_permute_invariance,
    pins.test_planted_future_token_is_masked,
    pins.test_gqa_head_reads_group_h_over_G,
]


def _build_mutant(tmp, old, new):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    path = os.path.join(tmp, "m.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    so = os.path.join(tmp, "m.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, path, "-lm"],
                   check=True)
    lib = ctypes.CDLL(so)
    lib.milo_oracle_attend.argtypes = [ctypes.POINTER(oracle._Args)]
    lib.milo_oracle_attend.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    real = oracle._load()
    with tempfile.TemporaryDirectory() as tmp:
        mutant = _build_mutant(tmp, old, new)
        oracle._lib = mutant
        try:
            failed = []
            for t in PIN_TESTS:
                try:
                    t()
                except (AssertionError, ValueError, RuntimeError) as e:
                    failed.append(getattr(t, "__name__", "sdpa"))
        finally:
            oracle._lib = real
    assert failed, f"no pin caught mutant {name}"


def test_real_oracle_passes_all_pins():
    for t in PIN_TESTS:
        t()
