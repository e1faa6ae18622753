"""GPU parity of the expert-grouped forward pass (pairs grouped by expert, each
weight row an expert needs read once for all of its tokens).

It must equal the per-pair result: the same candidate sets bit for bit (the
sketch activations are computed by the same integer arithmetic), kept sets
equal up to near-ties at the k-th score, and outputs within the tolerance.
Against the oracle it meets the same bars as the per-pair pass.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import cfm_oracle as O
from gpu_util import custom_workload, dev, down_bf16, log, oracle_map, up_bf16, upload
from parity import OUT_TOL, check_topset, rel_l2
from test_gpu_parity import compare_forward, gpu_sketch, run_select

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cfm():
    import calibration_free_channel_amd as m
    return m


def grouped(cfm):
    return cfm.forward_path(cfm.FORWARD_GROUPED)


def per_pair(cfm):
    return cfm.forward_path(cfm.FORWARD_PER_PAIR)


G_SMALL = [
    synth.WORKLOADS["tiny"],
    custom_workload("shared16", 8, 2, 128, 256, 16, 23, 46, 8, 20),
    custom_workload("crowded", 2, 2, 96, 128, 70, 10, 20, 8, 21),          # 70 tokens per expert
    custom_workload("ragged", 6, 3, 101, 128, 9, 17, 33, 8, 5),
    custom_workload("h64", 3, 2, 40, 64, 9, 4, 9, 8, 6),
    custom_workload("hmax", 2, 2, 24, 8192, 3, 3, 6, 8, 7),
    custom_workload("imax", 1, 1, 8192, 64, 2, 1474, 2948, 8, 9, rmsnorm=False),
]


@pytest.mark.parametrize("wl", G_SMALL, ids=lambda w: w.name)
def test_grouped_parity_small(cfm, wl):
    log(f"grouped select {wl.name}")
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, sorted(set(L.host.ids.reshape(-1).tolist())), E, I, H)
    with grouped(cfm):
        got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r)
    compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, what="grouped " + wl.name)


@pytest.mark.parametrize("kc", [(0, 0), (0, 40), (128, 128), (5, 128), (46, 46), (1, 1)])
@pytest.mark.parametrize("r", [0, 8])
def test_grouped_budget_edges(cfm, kc, r):
    k, c = kc
    wl = custom_workload(f"gedge_k{k}_c{c}_r{r}", 8, 2, 128, 256, 9, k, c, r, 11)
    log(f"grouped select {wl.name}")
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, r, range(E), E, I, H)
    with grouped(cfm):
        got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), k, c, r)
    compare_forward(L, A, Bt, got, cand, keep, k, c, what=wl.name)


def test_grouped_full_rank_recovery_only(cfm):
    """k = 0 and r = min(H, I): the whole layer comes through the map."""
    wl = custom_workload("gfullrank", 4, 2, 64, 128, 10, 0, 0, 64, 12)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, 64, range(4), 4, 64, 128)
    with grouped(cfm):
        got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), 0, 0, 64)
    compare_forward(L, A, Bt, got, cand, keep, 0, 0, what="gfullrank")


def test_grouped_all_kept_equals_grouped_dense(cfm):
    """k = c = I, r = 0: the grouped selected layer reads every row and equals the grouped dense layer bit for bit."""
    wl = custom_workload("gallkept", 8, 2, 128, 256, 12, 128, 128, 0, 14)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    with grouped(cfm):
        got, _, _ = run_select(cfm, L, sk, None, None, 128, 128, 0)
        dense = down_bf16(cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd))
    assert np.array_equal(got, dense)


@pytest.mark.parametrize("wl", [custom_workload("gd_tiny", 8, 2, 128, 256, 9, 1, 1, 0, 0),
                                custom_workload("gd_ragged", 6, 3, 101, 128, 11, 1, 1, 0, 5),
                                custom_workload("gd_crowded", 2, 2, 96, 128, 70, 1, 1, 0, 21),
                                custom_workload("gd_hmax", 2, 2, 24, 8192, 3, 1, 1, 0, 7)], ids=lambda w: w.name)
def test_grouped_dense_parity(cfm, wl):
    L = upload(wl)
    with grouped(cfm):
        got = down_bf16(cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd))
    h = L.host
    want = O.dense_forward(h.x, h.ids, h.w, h.w_gate, h.w_up, h.w_down_t)
    errs = [rel_l2(got[t], want[t]) for t in range(h.ids.shape[0])]
    log(f"grouped dense {wl.name}: max rel L2 {max(errs):.3e}")
    assert max(errs) <= OUT_TOL


def test_grouped_equals_per_pair(cfm):
    """Same inputs through both passes: identical candidate sets; kept sets equal up to
    near-ties of the exact scores; outputs agree within the tolerance."""
    wl = custom_workload("g_vs_p", 16, 4, 256, 512, 12, 46, 92, 16, 22)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, range(E), E, I, H)
    A, Bt = up_bf16(A), up_bf16(Bt)
    with per_pair(cfm):
        op, cp, kp = run_select(cfm, L, sk, A, Bt, wl.k, wl.c, wl.r)
    with grouped(cfm):
        og, cg, kg = run_select(cfm, L, sk, A, Bt, wl.k, wl.c, wl.r)
    assert np.array_equal(cp, cg), "candidate sets differ between the passes"
    same = np.all(kp == kg, axis=1)
    log(f"kept sets identical for {int(same.sum())}/{len(same)} pairs")
    assert same.mean() >= 0.9
    T, K = L.host.ids.shape
    for t in range(T):
        if np.all(same[t * K:(t + 1) * K]):
            assert rel_l2(og[t], op[t]) <= 1e-2


def test_grouped_determinism_and_batch_invariance(cfm):
    """Two grouped runs agree bit for bit; token 3 alone (per-pair pass) has the same candidate set."""
    wl = custom_workload("ginv", 8, 2, 128, 256, 12, 23, 46, 8, 15)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, 8, range(8), 8, 128, 256)
    A, Bt = up_bf16(A), up_bf16(Bt)
    with grouped(cfm):
        a = run_select(cfm, L, sk, A, Bt, 23, 46, 8)
        b = run_select(cfm, L, sk, A, Bt, 23, 46, 8)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    K = L.host.ids.shape[1]
    cand = torch.empty((K, 46), dtype=torch.int32, device=dev())
    one = cfm.moe_select_forward(L.x[3:4].contiguous(), L.ids[3:4].contiguous(), L.w[3:4].contiguous(),
                                 L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, 23, 46, 8, cand_out=cand)
    torch.cuda.synchronize()
    assert np.array_equal(cand.cpu().numpy(), a[1][3 * K:4 * K])
    assert rel_l2(down_bf16(one)[0], a[0][3]) <= 1e-2


def test_grouped_stats_counts_unions(cfm):
    """Byte accounting with sharing: per used expert, the union of its pairs' candidate and kept rows."""
    wl = custom_workload("gstats", 8, 2, 128, 256, 16, 23, 46, 8, 23)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A = torch.zeros((8, 256, 8), dtype=torch.bfloat16, device=dev())
    Bt = torch.zeros((8, 128, 8), dtype=torch.bfloat16, device=dev())
    with grouped(cfm):
        _, cand, keep, st = run_select(cfm, L, sk, A, Bt, 23, 46, 8, stats=True)
    T, K = L.host.ids.shape
    cs = {(t, q): cand[t * K + q] for t in range(T) for q in range(K)}
    ks = {(t, q): keep[t * K + q] for t in range(T) for q in range(K)}
    total = sum(st[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery", "bytes_io"))
    assert total == O.read_bytes(L.host.ids, 8, 128, 256, 23, 46, 8, cand_sets=cs, keep_sets=ks)
    assert st["bytes_dense_equiv"] == O.dense_bytes(L.host.ids, 8, 128, 256)
    assert st["experts_used"] == len(set(L.host.ids.reshape(-1).tolist()))
