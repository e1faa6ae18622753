"""Plant plausible slips in the CPU oracle and check that the pins catch each one.

A mistake in the oracle's arithmetic is planted in the C++ oracle itself
(oracle.cfm_oracle.set_mutation names one of the slips compiled into
oracle/cfm_oracle.cpp for this purpose), so it also reaches every internal use
(the batch forward, the sketch build, ...). Slips in the byte count, which is
Python, and in a function's result are planted with monkeypatch. One of the
pin tests in test_oracle_pins.py must then fail. All on the CPU.
"""
import contextlib

import numpy as np
import pytest

from oracle import cfm_oracle as O
import test_oracle_pins as P


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


@contextlib.contextmanager
def planted(name):
    O.set_mutation(name)
    try:
        yield
    finally:
        O.set_mutation("")


# ----------------------------------------------------------------------------- sketch

def test_threshold_inclusive_is_caught(golden_dir):
    with planted("threshold_inclusive"):            # '>=' instead of '>' at the TWN threshold
        _fails(P.test_twn_worked_example, golden_dir)


def test_wrong_threshold_factor_is_caught():
    with planted("twn_delta_half"):                 # 0.5 mean|w| instead of 0.7
        _fails(P.test_twn_nonzero_fraction_on_gaussian_rows)


def test_dropped_signs_are_caught():
    with planted("rotate_ignores_signs"):
        _fails(P.test_sketch_round_trip_on_ternary_rows, 64, 1)


def test_unsigned_scale_mean_is_caught():
    with planted("scale_mean_all"):                 # scale = mean |w~| over all values
        _fails(P.test_twn_scale_is_least_squares_for_its_pattern)


def test_swapped_gate_up_in_sketch_build_is_caught(monkeypatch):
    real = O.sketch_build

    def swapped(wg, wu, d):                         # the up sketch returned as the gate sketch and back
        tg, tu, sg, su = real(wg, wu, d)
        return tu, tg, su, sg
    monkeypatch.setattr(O, "sketch_build", swapped)
    _fails(P.test_sketch_build_feeds_the_screen_in_gate_up_order)


def test_swapped_flag_bits_are_caught(golden_dir):
    with planted("pack_sign_swap"):
        _fails(P.test_pack_golden, golden_dir)


def test_natural_bit_order_is_caught(golden_dir):
    with planted("pack_natural_order"):             # 4 codes per byte, LSB first, 01 = +1, 11 = -1
        _fails(P.test_pack_golden, golden_dir)


# ----------------------------------------------------------------------------- activations and selection

def test_silu_sign_slip_is_caught():
    with planted("silu_sign"):                      # z / (1 + e^z)
        _fails(P.test_silu_matches_scipy)
        _fails(P.test_dense_matches_torch_swiglu)


def test_topk_tie_to_higher_index_is_caught():
    with planted("topk_tie_high"):
        _fails(P.test_topk_brute_force_with_ties)


def test_transposed_down_rows_are_caught():
    with planted("gate_up_swapped"):
        _fails(P.test_dense_matches_torch_swiglu)


def test_recovery_over_unscreened_only_is_caught():
    """Dropping the screened-in-but-not-kept channels from the recovery sum must be caught."""
    with planted("recovery_unscreened_only"):
        _fails(P.test_kept_part_and_recovery_are_separate_terms)


def test_exact_scores_from_sketch_are_caught():
    """Keeping the top-k by sketch score instead of the exact BF16 score must be caught."""
    with planted("keep_by_sketch_score"):
        _fails(P.test_kept_part_and_recovery_are_separate_terms)


def test_candidates_exact_ignored_is_caught(monkeypatch):
    """A variant flag that falls back to the sketch activations must be caught."""
    orig = O.select_pair
    monkeypatch.setattr(O, "select_pair", lambda *a, **kw: orig(*a))
    _fails(P.test_candidates_exact_all_screened_full_rank_is_dense, 5)


def test_candidates_exact_on_every_skipped_channel_is_caught():
    """Giving every skipped channel (not only the dropped candidates) its exact activation must be caught."""
    with planted("candidates_exact_everywhere"):
        _fails(P.test_candidates_exact_changes_only_dropped_candidates)


def test_map_without_singular_values_is_caught():
    with planted("map_without_singular_values"):
        _fails(P.test_lowrank_eckart_young_and_orthonormal, (96, 40))
        _fails(P.test_lowrank_eckart_young_and_orthonormal, (40, 96))


# ----------------------------------------------------------------------------- envelope

def test_router_lowest_probabilities_are_caught():
    with planted("router_lowest"):
        _fails(P.test_router_matches_torch_softmax_topk)


def test_rmsnorm_without_weight_is_caught():
    with planted("rmsnorm_without_weight"):
        _fails(P.test_rmsnorm_matches_torch)


def test_residual_rounded_separately_is_caught():
    with planted("residual_rounded_separately"):
        _fails(P.test_layer_all_kept_matches_torch_envelope, False)


# ----------------------------------------------------------------------------- threshold keep rule

def test_threshold_strict_comparison_is_caught():
    with planted("threshold_strict"):
        _fails(P.test_threshold_set_brute_force_with_ties)


def test_threshold_calibration_off_by_one_is_caught():
    with planted("calibration_off_by_one"):        # the (k n + 1)-th largest instead of the (k n)-th
        _fails(P.test_calibrate_threshold_worked_example)


def test_threshold_ignored_by_select_pair_is_caught(monkeypatch):
    orig = O.select_pair
    monkeypatch.setattr(O, "select_pair", lambda *a, tau=None, **kw: orig(*a, **kw))
    _fails(P.test_select_pair_threshold_equals_topk_of_the_same_size)


# ----------------------------------------------------------------------------- byte count (Python)

def test_candidate_rows_billed_at_k0_is_caught(monkeypatch):
    """Billing candidate rows that nothing reads (k = 0, default recovery) must be caught."""
    orig = O.read_bytes
    monkeypatch.setattr(O, "read_bytes", lambda *a, **kw: orig(*a, **dict(kw, recovery="candidates_exact")))
    _fails(P.test_read_bytes_candidate_rows_only_when_exact_activations_are_used)


def test_threshold_rule_billed_like_topk_is_caught(monkeypatch):
    orig = O.read_bytes
    monkeypatch.setattr(O, "read_bytes", lambda *a, threshold=False, **kw: orig(*a, **kw))
    _fails(P.test_read_bytes_threshold_counts_the_kept_sets)


def test_no_mutation_is_left_planted():
    """The pins pass again once the switch is cleared."""
    with planted("silu_sign"):
        pass
    P.test_silu_matches_scipy()
    P.test_dense_matches_torch_swiglu()
