"""GPU parity of the threshold keep rule (moe_select_forward_threshold): the
kept set is every candidate whose exact |h| reaches tau, in place of the top k.

Bars: candidate sets as for top-k (tests/parity.py); kept sets equal to the
oracle's threshold set over the library's candidates, up to near-ties (oracle
score within 1e-3 relative of tau); |S| reported per pair with the rest of
keep_out -1; outputs within 2e-2 relative L2 on the tokens whose sets are
identical; the byte statistics count the kept rows actually read. tau comes
from the oracle's offline calibration on the workload's own pairs, so it lies
inside the score distribution (for the output checks moved half-way to the next
lower score, so that no float32 score sits on it), and from the edges 0 and
+inf.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import cfm_oracle as O
from gpu_util import custom_workload, dev, down_bf16, log, oracle_map, up_bf16, upload
from parity import NEAR_TIE, OUT_TOL, check_topset, rel_l2
from test_gpu_parity import gpu_sketch, run_select

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cfm():
    import calibration_free_channel_amd as m
    return m


def run_threshold(cfm, L, sk, A, Bt, tau, c, r, stats=False, recovery="sketch"):
    T, K = L.host.ids.shape
    P = max(T * K, 1)
    cand = torch.empty((P, max(c, 1)), dtype=torch.int32, device=dev())
    keep = torch.full((P, max(c, 1)), -7, dtype=torch.int32, device=dev())
    cnt = torch.full((P,), -7, dtype=torch.int32, device=dev())
    st = torch.zeros(cfm.STATS_BYTES, dtype=torch.uint8, device=dev()) if stats else None
    out = cfm.moe_select_forward_threshold(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, tau, c, r,
                                           cand_out=cand if c > 0 else None, keep_out=keep if c > 0 else None,
                                           keep_count=cnt, stats=st, recovery=recovery)
    torch.cuda.synchronize()
    res = (down_bf16(out), cand.cpu().numpy()[:, :c], keep.cpu().numpy()[:, :c], cnt.cpu().numpy())
    return res + ((cfm.decode_stats(st),) if stats else ())


def oracle_sketch(L, tokens):
    h = L.host
    E = h.w_gate.shape[0]
    used = sorted(set(int(e) for t in tokens for e in h.ids[t]))
    parts = O.sketch_build(h.w_gate[used], h.w_up[used], h.signs)
    out = []
    for a in parts:
        z = np.zeros((E,) + a.shape[1:], a.dtype)
        z[used] = a
        out.append(z)
    return out


def calibrated_tau(L, A_bits, Bt_bits, k, c, tokens, between=False):
    """The oracle's offline calibration over the given tokens' pairs: k kept per pair on average.
    between: move tau half-way to the next lower pooled score (the same kept sets on the
    calibration pairs, but tau no longer equal to one of their scores, so that the library's
    float32 scores do not sit on it)."""
    h = L.host
    tg, tu, sg, su = oracle_sketch(L, tokens)
    _, pairs = O.select_forward(h.x, h.ids, h.w, h.w_gate, h.w_up, h.w_down_t, tg, tu, sg, su, h.signs,
                                A_bits, Bt_bits, 0, c, tokens=tokens)
    sets = [np.abs(d["h_all"][d["C"]]) for d in pairs.values()]
    tau = O.calibrate_threshold(sets, k)
    if between:
        below = np.concatenate(sets)
        below = below[below < tau]
        if below.size:
            tau = 0.5 * (tau + float(below.max()))
    return tau


def check_threshold_set(row, count, universe, scores, tau, what):
    """row: the library's keep_out row (S ascending, then -1); count: its |S|.
    True if identical to the oracle's threshold set over `universe`, False if it
    differs only by near-ties at tau; raises otherwise."""
    row = np.asarray(row, np.int64)
    universe = np.asarray(universe, np.int64)
    scores = np.nan_to_num(np.asarray(scores, np.float64))
    assert 0 <= count <= universe.size, f"{what}: count {count}"
    got = row[:count]
    assert np.all(row[count:] == -1), f"{what}: keep_out not -1 past |S|"
    assert np.all(np.diff(got) > 0), f"{what}: not strictly ascending"
    pos = {int(j): n for n, j in enumerate(universe)}
    assert all(int(j) in pos for j in got), f"{what}: item outside the candidates"
    want = universe[O.threshold_set(scores, tau)]
    if np.array_equal(got, want):
        return True
    diff = set(map(int, got)) ^ set(map(int, want))
    bad = [j for j in diff if not abs(scores[pos[j]] - tau) <= NEAR_TIE * max(tau, 1e-300)]
    assert not bad, f"{what}: sets differ beyond near-ties at {bad[:5]} (tau {tau})"
    return False


def compare_threshold(L, A_bits, Bt_bits, got, cand, keep, cnt, tau, c, tokens=None, what="",
                      recovery="sketch"):
    h = L.host
    T, K = h.ids.shape
    I = h.w_gate.shape[1]
    tokens = list(range(T)) if tokens is None else list(tokens)
    tg, tu, sg, su = oracle_sketch(L, tokens)
    out, pairs = O.select_forward(h.x, h.ids, h.w, h.w_gate, h.w_up, h.w_down_t, tg, tu, sg, su, h.signs,
                                  A_bits, Bt_bits, 0, c, tokens=tokens, recovery=recovery, tau=tau)
    same_tokens, errs = 0, []
    for n, t in enumerate(tokens):
        same = True
        for q in range(K):
            pr = pairs[(t, q)]
            p = t * K + q
            s1 = check_topset(cand[p], np.arange(I), np.abs(pr["hhat"]), c, f"{what} C(t={t},q={q})")
            s2 = check_threshold_set(keep[p], int(cnt[p]), cand[p], np.abs(pr["h_all"][cand[p]]), tau,
                                     f"{what} S(t={t},q={q})")
            same &= s1 and s2
        if same:
            same_tokens += 1
            want = out[n]
        else:
            # the library's sets differ from the oracle's by near-ties only: check
            # its output against the oracle's arithmetic on those same sets
            want = O.staged_forward(h.x, h.ids, h.w, h.w_gate, h.w_up, h.w_down_t, tg, tu, sg, su, h.signs,
                                    A_bits, Bt_bits, {(t, q): cand[t * K + q] for q in range(K)},
                                    {(t, q): keep[t * K + q][:int(cnt[t * K + q])] for q in range(K)}, [t],
                                    recovery=recovery)[0]
        err = rel_l2(got[t], want)
        errs.append(err)
        assert err <= OUT_TOL, f"{what}: token {t} relative L2 {err:.3e}" + ("" if same else " (staged)")
    log(f"{what}: {same_tokens}/{len(tokens)} tokens with identical sets, the rest checked staged; max rel L2 "
        f"{max(errs) if errs else float('nan'):.3e}; |S| {cnt[:T * K].min()}..{cnt[:T * K].max()}")


def _paths(cfm):
    return [("per_pair", cfm.FORWARD_PER_PAIR), ("grouped", cfm.FORWARD_GROUPED)]


SMALL = [
    synth.WORKLOADS["tiny"],
    custom_workload("shared16", 8, 2, 128, 256, 16, 23, 46, 8, 20),
    custom_workload("ragged", 6, 3, 101, 128, 9, 17, 33, 8, 5),
    custom_workload("h64", 3, 2, 40, 64, 9, 4, 9, 8, 6),
    custom_workload("hmax", 2, 2, 24, 8192, 3, 3, 6, 8, 7),
    custom_workload("imax", 1, 1, 8192, 64, 2, 1474, 2948, 8, 9, rmsnorm=False),
]


@pytest.mark.parametrize("recovery", ["sketch", "candidates_exact"])
@pytest.mark.parametrize("path", ["per_pair", "grouped"])
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_threshold_parity_small(cfm, wl, path, recovery):
    log(f"threshold {wl.name} {path} {recovery}")
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, range(E), E, I, H)
    tau = calibrated_tau(L, A, Bt, wl.k, wl.c, range(wl.T), between=True)
    with cfm.forward_path(dict(_paths(cfm))[path]):
        got, cand, keep, cnt = run_threshold(cfm, L, sk, up_bf16(A), up_bf16(Bt), tau, wl.c, wl.r,
                                             recovery=recovery)
    compare_threshold(L, A, Bt, got, cand, keep, cnt, tau, wl.c, what=f"{wl.name} {path} {recovery}",
                      recovery=recovery)


@pytest.mark.parametrize("path", ["per_pair", "grouped"])
def test_threshold_every_channel_a_candidate(cfm, path):
    """c = I with the recovery variant (no sketch activation enters, so both passes skip the screen):
    S = every channel whose exact |h| reaches tau, the rest through the map with their exact h."""
    wl = custom_workload("tall", 4, 2, 64, 128, 6, 20, 64, 8, 36)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, range(E), E, I, H)
    tau = calibrated_tau(L, A, Bt, wl.k, wl.c, range(wl.T), between=True)
    with cfm.forward_path(dict(_paths(cfm))[path]):
        got, cand, keep, cnt, st = run_threshold(cfm, L, sk, up_bf16(A), up_bf16(Bt), tau, wl.c, wl.r,
                                                 stats=True, recovery="candidates_exact")
    assert st["bytes_sketch"] == 0
    compare_threshold(L, A, Bt, got, cand, keep, cnt, tau, wl.c, what=f"tall {path}", recovery="candidates_exact")


def test_threshold_crowded_expert_grouped(cfm):
    """70 tokens on each of two experts through the grouped pass (several 16-token tiles per expert)."""
    wl = custom_workload("tcrowded", 2, 2, 96, 128, 70, 10, 20, 8, 21)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, range(E), E, I, H)
    tau = calibrated_tau(L, A, Bt, wl.k, wl.c, range(wl.T), between=True)
    with cfm.forward_path(cfm.FORWARD_GROUPED):
        got, cand, keep, cnt = run_threshold(cfm, L, sk, up_bf16(A), up_bf16(Bt), tau, wl.c, wl.r)
    compare_threshold(L, A, Bt, got, cand, keep, cnt, tau, wl.c, what="tcrowded grouped")


@pytest.mark.parametrize("r", [0, 8])
@pytest.mark.parametrize("path", ["per_pair", "grouped"])
def test_threshold_edges_match_topk(cfm, path, r):
    """tau = 0 keeps every candidate: the same bits as top-k with k = c. tau = +inf keeps none:
    the top-k result with k = 0 (to the tolerance: the passes differ in summation order).
    A tau between the k-th and (k+1)-th exact score of every pair is not possible in general, so
    the in-between case is covered by the calibrated parity tests."""
    wl = custom_workload(f"tedge_r{r}", 8, 2, 128, 256, 9, 11, 40, r, 12)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, r, range(E), E, I, H)
    A, Bt = up_bf16(A), up_bf16(Bt)
    with cfm.forward_path(dict(_paths(cfm))[path]):
        for rec in ("sketch", "candidates_exact"):
            g0, c0, k0, n0 = run_threshold(cfm, L, sk, A, Bt, 0.0, wl.c, r, recovery=rec)
            ga, ca, ka = run_select(cfm, L, sk, A, Bt, wl.c, wl.c, r, recovery=rec)
            assert np.all(n0 == wl.c) and np.array_equal(k0, ka) and np.array_equal(c0, ca)
            assert np.array_equal(g0, ga), f"tau 0 vs k = c ({rec})"
            gi, ci, ki, ni = run_threshold(cfm, L, sk, A, Bt, float("inf"), wl.c, r, recovery=rec)
            gz, cz, _ = run_select(cfm, L, sk, A, Bt, 0, wl.c, r, recovery=rec)
            assert np.all(ni == 0) and np.all(ki == -1) and np.array_equal(ci, cz)
            for t in range(wl.T):
                assert rel_l2(gi[t], gz[t]) <= 1e-2, f"tau inf vs k = 0 ({rec}) token {t}"


@pytest.mark.parametrize("path", ["per_pair", "grouped"])
def test_threshold_without_candidates(cfm, path):
    """c = 0: nothing can be kept; |S| = 0 for every pair and the result is the k = c = 0 result, bit for bit."""
    wl = custom_workload("tc0", 8, 2, 128, 256, 5, 0, 0, 8, 13)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, range(E), E, I, H)
    A, Bt = up_bf16(A), up_bf16(Bt)
    with cfm.forward_path(dict(_paths(cfm))[path]):
        g, _, _, n = run_threshold(cfm, L, sk, A, Bt, 0.5, 0, wl.r)
        gz, _, _ = run_select(cfm, L, sk, A, Bt, 0, 0, wl.r)
    assert np.all(n == 0)
    assert np.array_equal(g, gz)


@pytest.mark.parametrize("path", ["per_pair", "grouped"])
def test_threshold_determinism_and_batch_invariance(cfm, path):
    """Two calls agree bit for bit (outputs, sets, counts); on the per-pair pass a token alone gets the
    bits it gets inside the batch, and on the grouped pass its kept set is the same alone and in the batch
    (the grouped pass's exact activations are MFMA sums over the expert's tokens, so its output bits may
    differ with the batch)."""
    wl = custom_workload("tinv", 8, 2, 128, 256, 8, 23, 46, 8, 15)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, 8, range(E), E, I, H)
    tau = calibrated_tau(L, A, Bt, wl.k, wl.c, range(wl.T), between=True)
    A, Bt = up_bf16(A), up_bf16(Bt)
    with cfm.forward_path(dict(_paths(cfm))[path]):
        a = run_threshold(cfm, L, sk, A, Bt, tau, wl.c, wl.r)
        b = run_threshold(cfm, L, sk, A, Bt, tau, wl.c, wl.r)
        one = run_threshold(cfm, _token(L, 3), sk, A, Bt, tau, wl.c, wl.r)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    K = wl.shape.K
    assert np.array_equal(one[3], a[3][3 * K:4 * K])
    assert np.array_equal(one[2], a[2][3 * K:4 * K])
    assert np.array_equal(one[1], a[1][3 * K:4 * K])
    if path == "per_pair":
        assert np.array_equal(one[0][0], a[0][3])


@pytest.mark.parametrize("path", ["per_pair", "grouped"])
def test_threshold_stats_count_kept_rows(cfm, path):
    """One token with distinct experts: the bytes the call reports equal the oracle's count for the
    kept sets the call returned (the per-pair pass bills per pair, the grouped pass per expert union;
    with distinct experts the two agree)."""
    wl = custom_workload("tstats", 8, 4, 128, 256, 1, 23, 46, 8, 31)
    L = upload(wl)
    assert len(set(L.host.ids[0].tolist())) == 4
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, range(E), E, I, H)
    tau = calibrated_tau(L, A, Bt, wl.k, wl.c, [0])
    with cfm.forward_path(dict(_paths(cfm))[path]):
        _, cand, keep, cnt, st = run_threshold(cfm, L, sk, up_bf16(A), up_bf16(Bt), tau, wl.c, wl.r, stats=True)
    ks = {(0, q): keep[q][:cnt[q]] for q in range(4)}
    assert st["rows_down"] == int(cnt.sum())
    assert st["bytes_down"] == 2 * H * int(cnt.sum())
    total = sum(st[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery", "bytes_io"))
    assert total == O.read_bytes(L.host.ids, E, I, H, 0, wl.c, wl.r, keep_sets=ks, threshold=True)


@pytest.fixture(scope="module")
def q18_layer():
    wl = synth.WORKLOADS["q18_b1"]
    log("generating the Qwen3-30B-A3B-shaped layer")
    return upload(wl)


def test_threshold_q18_b1_full_size(cfm, q18_layer):
    """Qwen3-30B-A3B-shaped layer at batch 1 (H 2048, E 128, K 8, I 768, c 276, r 64), tau calibrated
    on the token's own pairs for k = 138 (18 %) and for k = 60, in the launch configuration the
    benchmark times."""
    L, wl = q18_layer, q18_layer.wl
    E, I, H = L.host.w_gate.shape
    used = sorted(set(L.host.ids.reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used, E, I, H)
    for k in (wl.k, 60):
        tau = calibrated_tau(L, A, Bt, k, wl.c, [0], between=True)
        got, cand, keep, cnt = run_threshold(cfm, L, sk, up_bf16(A), up_bf16(Bt), tau, wl.c, wl.r)
        compare_threshold(L, A, Bt, got, cand, keep, cnt, tau, wl.c, what=f"q18_b1 threshold k {k}")
        assert abs(int(cnt.sum()) - 8 * k) <= 4          # the calibration pairs keep k on average


def test_threshold_reads_vary_where_topk_is_constant(cfm):
    """The read-volume finding: a threshold calibrated offline for k kept channels per pair on some
    tokens keeps a different number on each pair of other tokens, so the bytes each token reads
    vary, while top-k reads the same for every token. Qwen3-30B-A3B-shaped layer at 16 tokens,
    calibrated on tokens 0-3 for k = 138, applied to tokens 4-15 one token per call."""
    wl = synth.WORKLOADS["q18_b16"]
    log("generating the 16-token Qwen3-30B-A3B-shaped layer")
    L = upload(wl)
    E, I, H = L.host.w_gate.shape
    sk = gpu_sketch(cfm, L)
    # the map does not enter the kept sets: zeros for the oracle's calibration, the library's own map here
    zA, zB = np.zeros((E, H, wl.r), np.uint16), np.zeros((E, I, wl.r), np.uint16)
    tau = calibrated_tau(L, zA, zB, wl.k, wl.c, range(4))
    A, Bt = cfm.lowrank_build(L.wd, wl.r)
    counts, thr_bytes, topk_bytes = [], [], []
    for t in range(4, 16):
        one = _token(L, t)
        _, _, _, cnt, st = run_threshold(cfm, one, sk, A, Bt, tau, wl.c, wl.r, stats=True)
        *_, st2 = run_select(cfm, one, sk, A, Bt, wl.k, wl.c, wl.r, stats=True)
        counts.extend(cnt.tolist())
        thr_bytes.append(st["bytes_down"])
        topk_bytes.append(st2["bytes_down"])
    log(f"threshold |S| over 96 pairs: min {min(counts)} mean {np.mean(counts):.1f} max {max(counts)}; "
        f"down bytes per token {min(thr_bytes)}..{max(thr_bytes)}; top-k {set(topk_bytes)}")
    assert len(set(topk_bytes)) == 1 and topk_bytes[0] == 2 * H * wl.k * 8
    assert max(counts) > min(counts)
    assert len(set(thr_bytes)) > 1


def _token(L, t):
    """Token t of a device layer as a batch of one (the weights are shared, not copied)."""
    h = dataclasses.replace(L.host, x=L.host.x[t:t + 1].copy(), ids=L.host.ids[t:t + 1].copy(),
                            w=L.host.w[t:t + 1].copy())
    return dataclasses.replace(L, host=h, x=L.x[t:t + 1].contiguous(), ids=L.ids[t:t + 1].contiguous(),
                               w=L.w[t:t + 1].contiguous())


def test_threshold_q18_b16_both_passes(cfm):
    """16 Qwen3-30B-A3B-shaped tokens (18 %: c 276) through both passes, each forced, tau calibrated on the
    sampled tokens' pairs; compared with the oracle on those tokens."""
    wl = synth.WORKLOADS["q18_b16"]
    log("generating the 16-token Qwen3-30B-A3B-shaped layer")
    L = upload(wl)
    E, I, H = L.host.w_gate.shape
    tokens = [0, wl.T // 2, wl.T - 1]
    used = sorted(set(L.host.ids[tokens].reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used, E, I, H)
    tau = calibrated_tau(L, A, Bt, wl.k, wl.c, tokens, between=True)
    for name, path in _paths(cfm):
        with cfm.forward_path(path):
            got, cand, keep, cnt = run_threshold(cfm, L, sk, up_bf16(A), up_bf16(Bt), tau, wl.c, wl.r)
        compare_threshold(L, A, Bt, got, cand, keep, cnt, tau, wl.c, tokens=tokens, what=f"q18_b16 {name}")
