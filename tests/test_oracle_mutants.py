"""Shows that the oracle's pins have teeth: each plausible slip, planted in a copy of the
oracle's C source and compiled on the CPU, makes at least one pin in test_oracle.py fail."""
import os

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "verify_attn_oracle.c")

# (name, original text, planted text)
MUTANTS = [
    ("rope dims dropped from the score", "for (int64_t d = 0; d < D; ++d)",
     "for (int64_t d = 0; d < Dl; ++d)"),
    ("softmax scale not applied", "s[j] = scale * dot;", "s[j] = dot;"),
    ("mask indexed by tail position", "mrow[j] != 0", "mrow[j - P] != 0"),
    ("tree mask ignored", "vis[j] = (unsigned char)(j < P || mrow[j] != 0);", "vis[j] = 1;"),
    ("prefix columns read from the mask", "vis[j] = (unsigned char)(j < P || mrow[j] != 0);",
     "vis[j] = (unsigned char)(mrow[j] != 0);"),
    ("argmax ties broken high", "if (s[j] > m) {", "if (s[j] >= m) {"),
    ("value taken from the last Dl dims", "acc[c] += w * elem(kv_buffer, in_dtype, kbase + c);",
     "acc[c] += w * elem(kv_buffer, in_dtype, kbase + Dr + c);"),
    ("lse missing the max", "lse[n] = m + log(lam);", "lse[n] = log(lam);"),
    ("mask offset of request 0 for every request",
     "custom_mask + mask_indptr[r] + i * L", "custom_mask + i * L"),
    ("mask row stride T instead of L", "custom_mask + mask_indptr[r] + i * L",
     "custom_mask + mask_indptr[r] + i * T"),
    ("exponent sign flipped", "exp(s[j] - m)", "exp(m - s[j])"),
    ("denominator dropped", "o[c] = acc[c] / lam;", "o[c] = acc[c];"),
    ("key rows of request 0 for every request", "return kv_indices[kv_indptr[r] + j];",
     "return kv_indices[j];"),
    ("tree slots of request 0 for every request", "out_cache_loc[qo_indptr[r] + (j - P)]",
     "out_cache_loc[j - P]"),
    ("tree keys left out of the split layout's key count",
     "return out_cache_loc ? n + (qo_indptr[r + 1] - qo_indptr[r]) : n;", "return n;"),
    ("query row of head 0 for every head", "const int64_t qbase = (t * H + h) * D;",
     "const int64_t qbase = (t * H) * D;"),
]

PINS = [
    lambda: pins.test_brute_force_fuzz(1),
    lambda: pins.test_brute_force_fuzz(4),
    pins.test_brute_force_tiny_workload,
    lambda: pins.test_identical_rows_return_that_row("bf16"),
    lambda: pins.test_self_only_at_zero_prefix("bf16"),
    pins.test_prefix_permutation_invariance,
    pins.test_tree_node_permutation_equivariance,
    pins.test_prefix_mask_columns_and_invisible_rows_are_ignored,
    pins.test_mask_is_indexed_by_global_key_position_and_request,
    pins.test_zero_query_gives_mean_of_visible_values,
    pins.test_two_visible_keys_closed_form,
    pins.test_duplicate_slots_are_separate_keys_and_ties_break_low,
    pins.test_empty_visible_set,
    pins.test_rope_shift_invariance,
    pins.test_latent_is_the_value_and_rope_only_scores,
    lambda: pins.test_split_layout_brute_force(0),
]


def _caught(lib) -> bool:
    saved = oracle._lib
    oracle._lib = lib
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, oracle.OracleError, ValueError, FloatingPointError):
                return True
        return False
    finally:
        oracle._lib = saved


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, orig, planted, tmp_path):
    src = open(SRC).read()
    assert orig in src, f"mutation anchor vanished: {orig!r}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(orig, planted))
    so = str(tmp_path / "libmutant.so")
    oracle.build(src=str(mutated), out=so)
    lib = oracle.load(so)
    assert _caught(lib), f"no pin caught: {name}"


def test_unmutated_oracle_passes_every_pin():
    assert not _caught(oracle.load())
