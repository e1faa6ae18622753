"""GPU parity of the recovery variant in which candidates screened in but not
kept enter the low-rank map with their exact activation (moe_select_forward_ex
with CFM_RECOVER_CANDIDATES_EXACT), on both forward passes.

Same bars as the default method: candidate and kept sets equal to the oracle's
up to near-ties, outputs within 2e-2 relative L2 of the oracle run with the same
variant. The variant's defining property is checked on the device too: with
every channel screened in and a full-rank map the layer equals the dense layer.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import cfm_oracle as O
from gpu_util import custom_workload, dev, down_bf16, log, oracle_map, up_bf16, upload
from parity import OUT_TOL, rel_l2
from test_gpu_parity import compare_forward, gpu_sketch, run_select

pytestmark = pytest.mark.gpu
EXACT = "candidates_exact"


@pytest.fixture(scope="module")
def cfm():
    import calibration_free_channel_amd as m
    return m


PATHS = {"per_pair": 1, "grouped": 2}

WORKLOADS = [
    synth.WORKLOADS["tiny"],
    custom_workload("rx_ragged", 6, 3, 101, 128, 5, 17, 33, 8, 5),
    custom_workload("rx_shared16", 8, 2, 128, 256, 16, 23, 46, 8, 20),
    custom_workload("rx_crowded", 2, 2, 96, 128, 70, 10, 20, 8, 21),
    custom_workload("rx_hmax", 2, 2, 24, 8192, 2, 3, 6, 8, 7),
]
# ranks that are not a multiple of 8 (the per-pair pass only; the grouped pass needs r % 8 == 0)
PER_PAIR_ONLY = [
    custom_workload("rx_ragged_r6", 6, 3, 101, 128, 5, 17, 33, 6, 5),
    custom_workload("rx_hmax_r2", 2, 2, 24, 8192, 2, 3, 6, 2, 7),
]
CASES = [(wl, p) for wl in WORKLOADS for p in PATHS] + [(wl, "per_pair") for wl in PER_PAIR_ONLY]


@pytest.mark.parametrize("wl,path", CASES, ids=lambda v: v if isinstance(v, str) else v.name)
def test_candidates_exact_parity(cfm, wl, path):
    log(f"candidates_exact {wl.name} {path}")
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, sorted(set(L.host.ids.reshape(-1).tolist())), E, I, H)
    with cfm.forward_path(PATHS[path]):
        got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r, recovery=EXACT)
    compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, what=f"{wl.name}/{path}", recovery=EXACT)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("kc", [(0, 20), (0, 0), (20, 20), (0, 64), (1, 64)])
def test_candidates_exact_budget_edges(cfm, kc, path):
    """k = 0 with candidates (the exact step runs only for the recovery), no candidates,
    k = c (nothing dropped), every channel a candidate."""
    k, c = kc
    wl = custom_workload(f"rx_edge_k{k}_c{c}", 4, 2, 64, 128, 9, k, c, 8, 31)
    log(f"candidates_exact {wl.name} {path}")
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, 8, range(4), 4, 64, 128)
    with cfm.forward_path(PATHS[path]):
        got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), k, c, 8, recovery=EXACT)
    compare_forward(L, A, Bt, got, cand, keep, k, c, what=f"{wl.name}/{path}", recovery=EXACT)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("k", [0, 9])
def test_all_screened_full_rank_equals_dense(cfm, k, path):
    """c = I and r = min(H, I): every channel enters with its exact activation, through its
    down row or through the map, so the layer equals the dense layer up to the BF16 map."""
    wl = custom_workload(f"rx_dense_k{k}", 4, 2, 64, 128, 12, k, 64, 64, 32)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, 64, range(4), 4, 64, 128)
    with cfm.forward_path(PATHS[path]):
        got, _, _ = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), k, 64, 64, recovery=EXACT)
        dense = down_bf16(cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd))
        base, _, _ = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), k, 64, 64)
    errs = [rel_l2(got[t], dense[t]) for t in range(got.shape[0])]
    base_errs = [rel_l2(base[t], dense[t]) for t in range(got.shape[0])]
    log(f"k={k} {path}: variant vs dense max rel L2 {max(errs):.3e}; default recovery {max(base_errs):.3e}")
    assert max(errs) <= OUT_TOL
    assert min(base_errs) > max(errs), "the default recovery should not reproduce the dense layer"


def test_candidates_exact_stats_bill_candidate_rows_at_k0(cfm):
    """With k = 0 the variant still computes the candidates' exact activations, and bills them."""
    wl = synth.WORKLOADS["tiny"]
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A = torch.zeros((8, 256, 8), dtype=torch.bfloat16, device=dev())
    Bt = torch.zeros((8, 128, 8), dtype=torch.bfloat16, device=dev())
    with cfm.forward_path(PATHS["per_pair"]):
        *_, st0 = run_select(cfm, L, sk, A, Bt, 0, 46, 8, stats=True)
        *_, st1 = run_select(cfm, L, sk, A, Bt, 0, 46, 8, stats=True, recovery=EXACT)
    tot = lambda st: sum(st[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery",
                                         "bytes_io"))
    assert tot(st0) == O.read_bytes(L.host.ids, 8, 128, 256, 0, 46, 8)
    assert tot(st1) == O.read_bytes(L.host.ids, 8, 128, 256, 0, 46, 8, recovery=EXACT)
    assert st1["bytes_candidates"] == 2 * 4 * 256 * 46 and st0["bytes_candidates"] == 0


def test_default_flags_match_plain_entry_point(cfm):
    """moe_select_forward_ex with flags 0 is moe_select_forward (bit for bit)."""
    import ctypes
    from calibration_free_channel_amd import _lib
    wl = custom_workload("rx_flags0", 8, 2, 128, 256, 3, 23, 46, 8, 33)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, 8, range(8), 8, 128, 256)
    A, Bt = up_bf16(A), up_bf16(Bt)
    a = down_bf16(cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, 23, 46, 8))
    T, H = L.x.shape
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev())
    ws = _lib.new_workspace(_lib.select_workspace(T, 2, 8, 128, 256, 23, 46, 8), dev())
    P = _lib._ptr
    rc = _lib._lib.moe_select_forward_ex(
        P(L.x), P(L.ids), P(L.w), T, 2, P(L.wg), P(L.wu), P(L.wd), 8, 128, 256, P(L.signs), *[P(t) for t in sk],
        P(A), P(Bt), 23, 46, 8, ctypes.c_uint(0), P(out), None, None, None, P(ws), ws.numel(),
        _lib._stream(dev()))
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(down_bf16(out), a)


def test_candidates_exact_every_channel_a_candidate_reads_no_sketch(cfm):
    """c = I with the variant: both passes skip the screen; their bytes leave out the sketch, and their
    outputs match each other and the oracle."""
    wl = custom_workload("rx_nosk", 4, 2, 64, 128, 6, 20, 64, 8, 34)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, 8, range(4), 4, 64, 128)
    A, Bt = up_bf16(A), up_bf16(Bt)
    with cfm.forward_path(PATHS["per_pair"]):
        got, cand, keep, st = run_select(cfm, L, sk, A, Bt, 20, 64, 8, stats=True, recovery=EXACT)
    assert st["bytes_sketch"] == 0
    # (the per-pair pass bills every pair on its own; compared on a token whose experts are distinct)
    L1 = upload(custom_workload("rx_nosk1", 4, 2, 64, 128, 1, 20, 64, 8, 35))
    with cfm.forward_path(PATHS["per_pair"]):
        *_, st1 = run_select(cfm, L1, gpu_sketch(cfm, L1), A, Bt, 20, 64, 8, stats=True, recovery=EXACT)
    tot = sum(st1[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery", "bytes_io"))
    assert tot == O.read_bytes(L1.host.ids, 4, 64, 128, 20, 64, 8, recovery=EXACT)
    with cfm.forward_path(PATHS["grouped"]):
        gg, gc, gk, gst = run_select(cfm, L, sk, A, Bt, 20, 64, 8, stats=True, recovery=EXACT)
    assert np.array_equal(cand, gc)
    # the grouped pass bills the union of each expert's pairs' sets
    T, K = L.host.ids.shape
    cs = {(t, q): gc[t * K + q] for t in range(T) for q in range(K)}
    ks = {(t, q): gk[t * K + q] for t in range(T) for q in range(K)}
    assert gst["bytes_sketch"] == 0
    gtot = sum(gst[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery", "bytes_io"))
    assert gtot == O.read_bytes(L.host.ids, 4, 64, 128, 20, 64, 8, cs, ks, recovery=EXACT)
    for t in range(wl.T):
        assert rel_l2(got[t], gg[t]) <= 1e-2
    Ah, Bh = oracle_map(L.host.w_down_t, 8, range(4), 4, 64, 128)
    compare_forward(L, Ah, Bh, got, cand, keep, 20, 64, what="rx_nosk", recovery=EXACT)
