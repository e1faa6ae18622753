"""Plant plausible slips in the CPU oracle and check that the pins catch each one.

Every mutation is applied with monkeypatch to the oracle module on the CPU, and
one of the pin tests in test_oracle_pins.py must then fail.
"""
import numpy as np
import pytest

from oracle import cfm_oracle as O
import test_oracle_pins as P


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_threshold_inclusive_is_caught(monkeypatch, golden_dir):
    orig = O.ternarize

    def bad(wt):   # '>=' instead of '>' at the threshold
        wt = np.asarray(wt, np.float64)
        codes, _ = orig(wt)
        delta = O.TWN_DELTA * np.sum(np.abs(wt), -1) / wt.shape[-1]
        codes[wt >= delta[..., None]] = 1
        nz = codes != 0
        alpha = np.where(nz.sum(-1) > 0, np.sum(np.where(nz, np.abs(wt), 0), -1) / np.maximum(nz.sum(-1), 1), 0)
        return codes, alpha
    monkeypatch.setattr(O, "ternarize", bad)
    _fails(P.test_twn_worked_example, golden_dir)


def test_wrong_threshold_factor_is_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(O, "TWN_DELTA", 0.5)
    _fails(P.test_twn_nonzero_fraction_on_gaussian_rows)


def test_dropped_signs_are_caught(monkeypatch):
    orig = O.rotate
    monkeypatch.setattr(O, "rotate", lambda v, signs: orig(v, np.ones_like(signs)))
    _fails(P.test_sketch_round_trip_on_ternary_rows, 64, 1)


def test_unsigned_scale_mean_is_caught(monkeypatch):
    orig = O.ternarize

    def bad(wt):   # scale = mean |wt| over all values instead of over the kept ones
        codes, _ = orig(wt)
        return codes, np.mean(np.abs(np.asarray(wt, np.float64)), -1)
    monkeypatch.setattr(O, "ternarize", bad)
    _fails(P.test_twn_scale_is_least_squares_for_its_pattern)


def test_swapped_flag_bits_are_caught(monkeypatch, golden_dir):
    orig = O.pack_codes
    monkeypatch.setattr(O, "pack_codes", lambda codes: orig(-np.asarray(codes)))   # nz/neg mix-up on sign
    _fails(P.test_pack_golden, golden_dir)


def test_natural_bit_order_is_caught(monkeypatch, golden_dir):
    def natural(codes):   # 4 codes per byte, LSB first, 01 = +1, 11 = -1
        codes = np.asarray(codes)
        c = np.where(codes == 1, 1, np.where(codes == -1, 3, 0)).astype(np.uint8)
        c = c.reshape(c.shape[0], -1, 4)
        return (c[..., 0] | c[..., 1] << 2 | c[..., 2] << 4 | c[..., 3] << 6).astype(np.uint8)
    monkeypatch.setattr(O, "pack_codes", natural)
    _fails(P.test_pack_golden, golden_dir)


def test_silu_sign_slip_is_caught(monkeypatch):
    monkeypatch.setattr(O, "silu", lambda z: np.asarray(z, np.float64) / (1 + np.exp(np.asarray(z, np.float64))))
    _fails(P.test_silu_matches_scipy)
    _fails(P.test_dense_matches_torch_swiglu)


def test_topk_tie_to_higher_index_is_caught(monkeypatch):
    def bad(scores, k):
        s = np.nan_to_num(np.asarray(scores, np.float64))
        order = np.lexsort((-np.arange(s.size), -s))
        return np.sort(order[:k])
    monkeypatch.setattr(O, "topk_set", bad)
    _fails(P.test_topk_brute_force_with_ties)


def test_recovery_over_unscreened_only_is_caught(monkeypatch):
    """Dropping the screened-in-but-not-kept channels from the recovery sum must be caught."""
    orig = O.select_pair

    def bad(x_bits, e, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c, **kw):
        d = orig(x_bits, e, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c, **kw)
        lost = [j for j in d["C"] if j not in set(d["S"])]
        if A.shape[-1] and lost:
            corr = O.as_f64(A[e]) @ sum(d["hhat"][j] * O.as_f64(Bt[e][j]) for j in lost)
            d["y"] = d["y"] - corr
        return d
    monkeypatch.setattr(O, "select_pair", bad)
    _fails(P.test_kept_part_and_recovery_are_separate_terms)


def test_exact_scores_from_sketch_are_caught(monkeypatch):
    """Keeping the top-k by sketch score instead of the exact BF16 score must be caught."""
    orig = O.select_pair

    def bad(x_bits, e, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c, **kw):
        d = orig(x_bits, e, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c, **kw)
        d["S"] = d["C"][O.topk_set(np.abs(d["hhat"][d["C"]]), k)]
        return d
    monkeypatch.setattr(O, "select_pair", bad)
    _fails(P.test_kept_part_and_recovery_are_separate_terms)


def test_transposed_down_rows_are_caught(monkeypatch):
    orig = O.exact_activations
    monkeypatch.setattr(O, "exact_activations", lambda x, g, u: orig(x, u, g))   # gate/up swapped
    _fails(P.test_dense_matches_torch_swiglu)


def test_map_without_singular_values_is_caught(monkeypatch):
    orig = O.lowrank

    def bad(w, r):
        A, Bt = orig(w, r)
        return A / np.maximum(np.linalg.norm(A, axis=0), 1e-300), Bt
    monkeypatch.setattr(O, "lowrank", bad)
    _fails(P.test_lowrank_eckart_young_and_orthonormal)


def test_candidates_exact_ignored_is_caught(monkeypatch):
    """A variant flag that falls back to the sketch activations must be caught."""
    orig = O.select_pair
    monkeypatch.setattr(O, "select_pair", lambda *a, **kw: orig(*a))
    _fails(P.test_candidates_exact_all_screened_full_rank_is_dense, 5)


def test_candidates_exact_on_every_skipped_channel_is_caught(monkeypatch):
    """Giving every skipped channel (not only the dropped candidates) its exact activation must be caught."""
    orig = O.select_pair

    def bad(x_bits, e, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c, recovery="sketch"):
        d = orig(x_bits, e, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c, recovery=recovery)
        if recovery == "candidates_exact" and A.shape[-1]:
            outside = [j for j in range(w_gate.shape[1]) if j not in set(d["C"])]
            if outside:
                d["y"] = d["y"] + O.as_f64(A[e]) @ sum((d["h_all"][j] - d["hhat"][j]) * O.as_f64(Bt[e][j])
                                                       for j in outside)
        return d
    monkeypatch.setattr(O, "select_pair", bad)
    _fails(P.test_candidates_exact_changes_only_dropped_candidates)


def test_candidate_rows_billed_at_k0_is_caught(monkeypatch):
    """Billing candidate rows that nothing reads (k = 0, default recovery) must be caught."""
    orig = O.read_bytes
    monkeypatch.setattr(O, "read_bytes", lambda *a, **kw: orig(*a, **dict(kw, recovery="candidates_exact")))
    _fails(P.test_read_bytes_candidate_rows_only_when_exact_activations_are_used)


def test_router_lowest_probabilities_are_caught(monkeypatch):
    orig = O.router

    def bad(x_bits, w_router_bits, K, renorm):
        ids, w, logits = orig(x_bits, -O.as_f64(w_router_bits), K, renorm)
        return ids, w, -logits
    monkeypatch.setattr(O, "router", bad)
    _fails(P.test_router_matches_torch_softmax_topk)


def test_rmsnorm_without_weight_is_caught(monkeypatch):
    orig = O.rmsnorm
    monkeypatch.setattr(O, "rmsnorm", lambda h, g, eps: orig(h, O.f64_to_bf16(np.ones(np.shape(g))), eps))
    _fails(P.test_rmsnorm_matches_torch)


def test_residual_rounded_separately_is_caught(monkeypatch):
    orig = O.combine

    def bad(ys, w, resid=None):
        out = orig(ys, w)
        if resid is None:
            return out
        return O.f64_to_bf16(O.bf16_to_f64(out) + O.bf16_to_f64(resid))
    monkeypatch.setattr(O, "combine", bad)
    _fails(P.test_layer_all_kept_matches_torch_envelope, False)


# ----------------------------------------------------------------------------- threshold keep rule

def test_threshold_strict_comparison_is_caught(monkeypatch):
    monkeypatch.setattr(O, "threshold_set",
                        lambda scores, tau: np.flatnonzero(np.nan_to_num(np.asarray(scores, np.float64)) > tau))
    _fails(P.test_threshold_set_brute_force_with_ties)


def test_threshold_calibration_off_by_one_is_caught(monkeypatch):
    def bad(score_sets, k):   # the (k n + 1)-th largest instead of the (k n)-th
        pooled = np.sort(np.concatenate([np.asarray(s, np.float64) for s in score_sets]))[::-1]
        m = k * len(score_sets)
        return float("inf") if m <= 0 else float(pooled[min(m, pooled.size - 1)])
    monkeypatch.setattr(O, "calibrate_threshold", bad)
    _fails(P.test_calibrate_threshold_worked_example)


def test_threshold_ignored_by_select_pair_is_caught(monkeypatch):
    orig = O.select_pair
    monkeypatch.setattr(O, "select_pair", lambda *a, tau=None, **kw: orig(*a, **kw))
    _fails(P.test_select_pair_threshold_equals_topk_of_the_same_size)


def test_threshold_rule_billed_like_topk_is_caught(monkeypatch):
    orig = O.read_bytes
    monkeypatch.setattr(O, "read_bytes", lambda *a, threshold=False, **kw: orig(*a, **kw))
    _fails(P.test_read_bytes_threshold_counts_the_kept_sets)
