"""Comparison rules between the HIP library and the CPU oracle.

Index sets: the library must return exactly the oracle's set, or a set whose
symmetric difference with it consists only of near-ties: items whose oracle
score lies within 1e-3 (relative) of the oracle's boundary score (the k-th
largest). The library scores in float32 and the oracle in float64, so a swap
of two items that tie to within rounding is a valid answer too.

Outputs: relative L2 error per token <= 2e-2 on the BF16 result.
"""
from __future__ import annotations

import numpy as np

from oracle import cfm_oracle as O

NEAR_TIE = 1e-3
OUT_TOL = 2e-2


def check_topset(got, universe, scores, k, what=""):
    """got: ascending indices the library chose from `universe` (ascending),
    scores: oracle scores aligned with `universe`. Returns True if identical to
    the oracle's choice, False if it differs only by near-ties; raises otherwise."""
    got = np.asarray(got, np.int64)
    universe = np.asarray(universe, np.int64)
    scores = np.nan_to_num(np.asarray(scores, np.float64))
    assert got.shape == (k,), f"{what}: expected {k} items, got {got.shape}"
    assert np.all(np.diff(got) > 0), f"{what}: not strictly ascending"
    pos = {int(j): n for n, j in enumerate(universe)}
    assert all(int(j) in pos for j in got), f"{what}: item outside the universe"
    want = universe[O.topk_set(scores, k)] if k > 0 else np.zeros(0, np.int64)
    if np.array_equal(got, want):
        return True
    order = np.sort(scores)[::-1]
    boundary = order[k - 1]
    diff = set(map(int, got)) ^ set(map(int, want))
    bad = [j for j in diff if abs(scores[pos[j]] - boundary) > NEAR_TIE * max(boundary, 1e-300)]
    assert not bad, f"{what}: sets differ beyond near-ties at {bad[:5]} (boundary {boundary})"
    return False


def rel_l2(got_bits, want_bits):
    g = O.bf16_to_f64(got_bits)
    w = O.bf16_to_f64(want_bits)
    return float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-300))
