"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bars (see tests/parity.py): packed sketches and scales bit-exact; candidate and
kept index sets equal to the oracle's up to near-ties at the boundary; BF16
outputs within 2e-2 relative L2 per token. The forward tests give the library
the oracle's low-rank map, so the forward kernels are checked in isolation;
the library's own map is checked by Eckart-Young optimality and end to end.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import cfm_oracle as O
from gpu_util import (custom_workload, dev, down_bf16, log, oracle_map, up, up_bf16, upload)
from parity import OUT_TOL, check_topset, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cfm():
    import calibration_free_channel_amd as m
    return m


def gpu_sketch(cfm, L):
    tg, tu, sg, su = cfm.sketch_build(L.wg, L.wu, L.signs)
    torch.cuda.synchronize()
    return tg, tu, sg, su


def run_select(cfm, L, sk, A, Bt, k, c, r, stats=False, recovery="sketch"):
    T, K = L.host.ids.shape
    cand = torch.empty((max(T * K, 1), max(c, 1)), dtype=torch.int32, device=dev())
    keep = torch.empty((max(T * K, 1), max(k, 1)), dtype=torch.int32, device=dev())
    st = torch.zeros(cfm.STATS_BYTES, dtype=torch.uint8, device=dev()) if stats else None
    out = cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, k, c, r,
                                 cand_out=cand if c > 0 else None, keep_out=keep if k > 0 else None,
                                 stats=st, recovery=recovery)
    torch.cuda.synchronize()
    res = (down_bf16(out), cand.cpu().numpy()[:, :c], keep.cpu().numpy()[:, :k])
    return res + ((cfm.decode_stats(st),) if stats else ())


def compare_forward(L, A_bits, Bt_bits, got, cand, keep, k, c, tokens=None, what="", recovery="sketch"):
    """Oracle run on the host inputs (its own sketch) vs the library's results.

    Candidate and kept sets must equal the oracle's up to near-ties (the kept
    set staged: the oracle's top-k over the library's candidates). Every
    token's output is then checked: against the oracle's output when its sets
    are the oracle's, else against the oracle's output on the library's own
    sets (staged), which isolates the arithmetic from the near-tie choice."""
    h = L.host
    T, K = h.ids.shape
    tokens = list(range(T)) if tokens is None else list(tokens)
    used = sorted(set(int(e) for t in tokens for e in h.ids[t]))
    E, I, H = h.w_gate.shape
    tg, tu, sg, su = O.sketch_build(h.w_gate[used], h.w_up[used], h.signs)
    # scatter back to full-E arrays (only the used experts are read)
    def full(a):
        z = np.zeros((E,) + a.shape[1:], a.dtype)
        z[used] = a
        return z
    tg, tu, sg, su = full(tg), full(tu), full(sg), full(su)
    out, pairs = O.select_forward(h.x, h.ids, h.w, h.w_gate, h.w_up, h.w_down_t, tg, tu, sg, su,
                                  h.signs, A_bits, Bt_bits, k, c, tokens=tokens, recovery=recovery)
    exact_tokens, staged_tokens, errs = 0, [], []
    for n, t in enumerate(tokens):
        same = True
        for q in range(K):
            pr = pairs[(t, q)]
            p = t * K + q
            s1 = check_topset(cand[p], np.arange(I), np.abs(pr["hhat"]), c, f"{what} C(t={t},q={q})")
            s2 = check_topset(keep[p], cand[p], np.abs(pr["h_all"][cand[p]]), k, f"{what} S(t={t},q={q})")
            same &= s1 and s2
        if same:
            exact_tokens += 1
            want = out[n]
        else:
            staged_tokens.append(t)
            want = O.staged_forward(h.x, h.ids, h.w, h.w_gate, h.w_up, h.w_down_t, tg, tu, sg, su, h.signs,
                                    A_bits, Bt_bits, {(t, q): cand[t * K + q] for q in range(K)},
                                    {(t, q): keep[t * K + q] for q in range(K)}, [t], recovery=recovery)[0]
        err = rel_l2(got[t], want)
        errs.append(err)
        assert err <= OUT_TOL, f"{what}: token {t} relative L2 {err:.3e}" + (" (staged)" if not same else "")
    log(f"{what}: {exact_tokens}/{len(tokens)} tokens with identical sets, {len(staged_tokens)} checked staged "
        f"on the library's near-tie sets; max rel L2 {max(errs) if errs else float('nan'):.3e}")
    return max(errs) if errs else 0.0


# ----------------------------------------------------------------------------- sketch

SKETCH_SHAPES = [
    custom_workload("tinyish", 8, 2, 128, 256, 1, 23, 46, 8, 0, chan_scale=False),
    custom_workload("ragged", 6, 3, 101, 128, 5, 17, 33, 6, 5),
    custom_workload("h64", 3, 2, 40, 64, 3, 4, 9, 3, 6),
    custom_workload("hmax", 2, 2, 24, 8192, 2, 3, 6, 2, 7),
]


@pytest.mark.parametrize("wl", SKETCH_SHAPES, ids=lambda w: w.name)
def test_sketch_bitwise(cfm, wl):
    log(f"sketch {wl.name}")
    L = upload(wl)
    tg, tu, sg, su = gpu_sketch(cfm, L)
    otg, otu, osg, osu = O.sketch_build(L.host.w_gate, L.host.w_up, L.host.signs)
    assert np.array_equal(tg.cpu().numpy(), otg)
    assert np.array_equal(tu.cpu().numpy(), otu)
    assert np.array_equal(sg.cpu().numpy().view(np.uint32), osg.view(np.uint32))
    assert np.array_equal(su.cpu().numpy().view(np.uint32), osu.view(np.uint32))


def test_sketch_round_trip_gpu(cfm):
    """Exactly ternary rotated rows: the library's sketch returns the ternary pattern, scale 1."""
    H, I = 256, 64
    r = np.random.default_rng(21)
    d = np.where(r.integers(0, 2, H) == 1, -1, 1).astype(np.int8)
    t = r.integers(-1, 2, size=(2, I, H)).astype(np.int8)
    hm = O.hadamard(H)
    w = d * (t.astype(np.float64) @ hm)          # integers |.| <= H: BF16-exact
    bits = O.f64_to_bf16(w)
    tg, tu, sg, su = cfm.sketch_build(up_bf16(bits[:1]), up_bf16(bits[1:]), up(d))
    torch.cuda.synchronize()
    assert np.array_equal(O.unpack_codes(tg.cpu().numpy()[0]), t[0])
    assert np.array_equal(O.unpack_codes(tu.cpu().numpy()[0]), t[1])
    assert np.all(sg.cpu().numpy() == 1.0) and np.all(su.cpu().numpy() == 1.0)


# ----------------------------------------------------------------------------- forward, small

SMALL = [
    synth.WORKLOADS["tiny"],
    custom_workload("ragged", 6, 3, 101, 128, 5, 17, 33, 6, 5),
    custom_workload("batch7", 8, 2, 128, 256, 7, 23, 46, 8, 8),
    custom_workload("h64", 3, 2, 40, 64, 3, 4, 9, 3, 6),
    custom_workload("hmax", 2, 2, 24, 8192, 2, 3, 6, 2, 7),
    custom_workload("imax", 1, 1, 8192, 64, 1, 1474, 2948, 8, 9, rmsnorm=False),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_select_parity_small(cfm, wl):
    log(f"select {wl.name}")
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, wl.r, sorted(set(L.host.ids.reshape(-1).tolist())), E, I, H)
    got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r)
    compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, what=wl.name)


@pytest.mark.parametrize("kc", [(0, 0), (0, 40), (128, 128), (5, 128), (46, 46), (1, 1)])
@pytest.mark.parametrize("r", [0, 8])
def test_select_budget_edges(cfm, kc, r):
    k, c = kc
    wl = custom_workload(f"edge_k{k}_c{c}_r{r}", 8, 2, 128, 256, 3, k, c, r, 11)
    log(f"select {wl.name}")
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    E, I, H = L.host.w_gate.shape
    A, Bt = oracle_map(L.host.w_down_t, r, range(E), E, I, H)
    got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), k, c, r)
    compare_forward(L, A, Bt, got, cand, keep, k, c, what=wl.name)


@pytest.mark.parametrize("T", [1, 2])
def test_select_candidates_concentrated(cfm, T):
    """Gate and up rows 0..c-1 of every expert scaled by 8 (exact in BF16, gate signs set so
    that token 0's gate is positive): the candidates crowd into the lowest channels, so the
    candidate list is far from evenly spread over the workgroups that screened it."""
    wl = custom_workload(f"conc_t{T}", 4, 1, 256, 256, T, 20, 40, 8, 24, chan_scale=False)
    h = synth.make_inputs(wl)
    x0 = O.bf16_to_f64(h.x[0])
    for wm in (h.w_gate, h.w_up):
        v = O.bf16_to_f64(wm[:, :40, :]) * 8.0
        if wm is h.w_gate:                     # positive gate for token 0, so SiLU keeps the scale
            v *= np.where(v @ x0 < 0, -1.0, 1.0)[:, :, None]
        wm[:, :40, :] = O.f64_to_bf16(v)
    L = upload(wl, h)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(h.w_down_t, 8, range(4), 4, 256, 256)
    got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), 20, 40, 8)
    assert np.sum(cand[0] < 40) >= 30, "the scaled rows should dominate the candidates"
    compare_forward(L, A, Bt, got, cand, keep, 20, 40, what=wl.name)


def test_select_full_rank_recovery_only(cfm):
    """k = 0 and r = min(H, I): every channel enters through the map (y = W_down hhat)."""
    wl = custom_workload("fullrank", 4, 2, 64, 128, 2, 0, 0, 64, 12)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, 64, range(4), 4, 64, 128)
    got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), 0, 0, 64)
    compare_forward(L, A, Bt, got, cand, keep, 0, 0, what="fullrank")


def test_empty_batch_is_noop(cfm):
    wl = custom_workload("empty", 4, 2, 64, 128, 0, 5, 10, 4, 13)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A = torch.zeros((4, 128, 4), dtype=torch.bfloat16, device=dev())
    Bt = torch.zeros((4, 64, 4), dtype=torch.bfloat16, device=dev())
    out = cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, 5, 10, 4)
    torch.cuda.synchronize()
    assert out.shape == (0, 128)


def test_all_kept_equals_dense_on_gpu(cfm):
    """k = c = I, r = 0: the selected layer reads every channel and must equal the dense kernel bit for bit."""
    wl = custom_workload("allkept", 8, 2, 128, 256, 4, 128, 128, 0, 14)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    got, _, _ = run_select(cfm, L, sk, None, None, 128, 128, 0)
    dense = down_bf16(cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd))
    assert np.array_equal(got, dense)


@pytest.mark.parametrize("wl", [synth.WORKLOADS["tiny"], custom_workload("ragged", 6, 3, 101, 128, 5, 17, 33, 6, 5),
                                custom_workload("hmax", 2, 2, 24, 8192, 2, 3, 6, 2, 7)], ids=lambda w: w.name)
def test_dense_parity(cfm, wl):
    L = upload(wl)
    got = down_bf16(cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd))
    h = L.host
    want = O.dense_forward(h.x, h.ids, h.w, h.w_gate, h.w_up, h.w_down_t)
    for t in range(h.ids.shape[0]):
        assert rel_l2(got[t], want[t]) <= OUT_TOL


def test_determinism_and_batch_invariance(cfm):
    """Per-pair pass: two runs agree bit for bit, and token 3 alone gives the bits it gets inside the batch."""
    wl = custom_workload("inv", 8, 2, 128, 256, 8, 23, 46, 8, 15)
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, 8, range(8), 8, 128, 256)
    A, Bt = up_bf16(A), up_bf16(Bt)
    with cfm.forward_path(cfm.FORWARD_PER_PAIR):
        a = run_select(cfm, L, sk, A, Bt, 23, 46, 8)
        b = run_select(cfm, L, sk, A, Bt, 23, 46, 8)
        one = cfm.moe_select_forward(L.x[3:4].contiguous(), L.ids[3:4].contiguous(), L.w[3:4].contiguous(),
                                     L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, 23, 46, 8)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    assert np.array_equal(down_bf16(one)[0], a[0][3])


def test_stats_counts(cfm):
    wl = synth.WORKLOADS["tiny"]
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A = torch.zeros((8, 256, 8), dtype=torch.bfloat16, device=dev())
    Bt = torch.zeros((8, 128, 8), dtype=torch.bfloat16, device=dev())
    *_, st = run_select(cfm, L, sk, A, Bt, 23, 46, 8, stats=True)
    total = sum(st[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery", "bytes_io"))
    assert total == O.read_bytes(L.host.ids, 8, 128, 256, 23, 46, 8)
    assert st["bytes_dense_equiv"] == O.dense_bytes(L.host.ids, 8, 128, 256)


# ----------------------------------------------------------------------------- low-rank map

def _check_lowrank(wd_bits, A_bits, Bt_bits, r, what=""):
    """The library's map against Eckart-Young: its residual ||W - A Bt^T||_F^2 may exceed the optimum
    sum_{i>r} s_i^2 by at most 1e-3 of the energy the optimum captures, sum_{i<=r} s_i^2 (BF16 storage of
    A and Bt alone costs about 1e-5 of it); at full rank (optimum 0), at most 1e-4 of ||W||_F^2. Bt has
    orthonormal columns to BF16 precision."""
    W = O.bf16_to_f64(wd_bits).T                      # H x I
    A, Bt = O.bf16_to_f64(A_bits), O.bf16_to_f64(Bt_bits)
    ev = np.sort(np.linalg.eigvalsh(W.T @ W))[::-1]
    opt = max(ev[r:].sum(), 0.0)
    captured = ev[:r].sum()
    resid = np.sum((W - A @ Bt.T) ** 2)
    if r >= min(W.shape):
        assert resid <= 1e-4 * ev.sum(), f"{what}: full-rank residual {resid / ev.sum():.2e} of ||W||^2"
    else:
        assert resid - opt <= 1e-3 * captured, \
            f"{what}: residual above the optimum by {(resid - opt) / captured:.2e} of the captured energy"
    assert np.allclose(Bt.T @ Bt, np.eye(r), atol=2e-2)
    return (resid - opt) / captured


@pytest.mark.parametrize("wl", [synth.WORKLOADS["tiny"], custom_workload("ragged", 6, 3, 101, 128, 5, 17, 33, 6, 5),
                                custom_workload("rfull", 3, 2, 64, 128, 1, 4, 8, 64, 16),
                                custom_workload("rfull_h", 2, 2, 256, 64, 1, 4, 8, 64, 17)], ids=lambda w: w.name)
def test_lowrank_optimality(cfm, wl):
    L = upload(wl)
    A, Bt = cfm.lowrank_build(L.wd, wl.r)
    torch.cuda.synchronize()
    A, Bt = down_bf16(A), down_bf16(Bt)
    worst = max(_check_lowrank(L.host.w_down_t[e], A[e], Bt[e], wl.r, f"{wl.name} expert {e}")
                for e in range(wl.shape.E))
    log(f"{wl.name}: worst excess over the optimum {worst:.2e} of the captured energy")


@pytest.mark.parametrize("IH", [(64, 128), (256, 64)], ids=["tall", "wide"])
def test_lowrank_rank_deficient(cfm, IH):
    """An expert of rank 3 (its channels repeat three BF16 rows scaled by powers of two, so the rank is
    exact after rounding) and an all-zero expert, at r = 8: the map reproduces W_down to BF16 storage
    precision, every value is finite, and each column of Bt is a unit vector or zero."""
    I, H = IH
    r, rank = 8, 3
    rng = np.random.default_rng(31)
    base = O.f64_to_bf16(rng.standard_normal((rank, H)) * 0.02)
    pick = rng.integers(0, rank, I)
    scale = 2.0 ** rng.integers(-2, 3, I)
    wd = np.zeros((2, I, H), np.uint16)
    wd[0] = O.f64_to_bf16(O.bf16_to_f64(base)[pick] * scale[:, None])
    A, Bt = cfm.lowrank_build(up_bf16(wd), r)
    torch.cuda.synchronize()
    A, Bt = O.bf16_to_f64(down_bf16(A)), O.bf16_to_f64(down_bf16(Bt))
    assert np.isfinite(A).all() and np.isfinite(Bt).all()
    W = O.bf16_to_f64(wd[0]).T
    assert np.sum((W - A[0] @ Bt[0].T) ** 2) <= 1e-4 * np.sum(W ** 2)
    assert not A[1].any()
    for e in range(2):
        n = np.linalg.norm(Bt[e], axis=0)
        assert np.all((np.abs(n - 1) <= 1e-2) | (n == 0)), f"expert {e}: column norms {n}"


def test_lowrank_end_to_end_tiny(cfm):
    """The library's own map in the forward pass, against the oracle with the oracle's map (full size:
    test_q18_b1_full_size)."""
    wl = synth.WORKLOADS["tiny"]
    L = upload(wl)
    sk = gpu_sketch(cfm, L)
    A, Bt = cfm.lowrank_build(L.wd, wl.r)
    got, cand, keep = run_select(cfm, L, sk, A, Bt, wl.k, wl.c, wl.r)
    Ao, Bo = oracle_map(L.host.w_down_t, wl.r, range(8), 8, 128, 256)
    compare_forward(L, Ao, Bo, got, cand, keep, wl.k, wl.c, what="tiny/own-map")


# ----------------------------------------------------------------------------- full-size configurations

@pytest.fixture(scope="module")
def q18_layer():
    wl = synth.WORKLOADS["q18_b1"]
    log("generating the Qwen3-30B-A3B-shaped layer")
    return upload(wl)


def test_q18_b1_full_size(cfm, q18_layer):
    """Qwen3-30B-A3B-shaped layer (H 2048, E 128, K 8, I 768), batch 1, k 138, c 276, r 64."""
    L, wl = q18_layer, q18_layer.wl
    E, I, H = L.host.w_gate.shape
    used = sorted(set(L.host.ids.reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    # sketch of the routed experts: bit-exact
    otg, otu, osg, osu = O.sketch_build(L.host.w_gate[used], L.host.w_up[used], L.host.signs)
    assert np.array_equal(sk[0].cpu().numpy()[used], otg)
    assert np.array_equal(sk[1].cpu().numpy()[used], otu)
    assert np.array_equal(sk[2].cpu().numpy()[used].view(np.uint32), osg.view(np.uint32))
    assert np.array_equal(sk[3].cpu().numpy()[used].view(np.uint32), osu.view(np.uint32))
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used, E, I, H)
    got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r)
    compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, what="q18_b1")
    # the library's own map on the routed experts: near-optimal
    Ag, Bg = cfm.lowrank_build(L.wd, wl.r)
    torch.cuda.synchronize()
    Ag, Bg = down_bf16(Ag), down_bf16(Bg)
    for e in used[:3]:
        _check_lowrank(L.host.w_down_t[e], Ag[e], Bg[e], wl.r, f"q18 expert {e}")
    # ... and end to end: the forward pass with the library's own map against the oracle with its map
    # (the map enters only the recovery term, so the sets are the same)
    got2, cand2, keep2 = run_select(cfm, L, sk, up_bf16(Ag), up_bf16(Bg), wl.k, wl.c, wl.r)
    assert np.array_equal(cand2, cand) and np.array_equal(keep2, keep)
    compare_forward(L, A, Bt, got2, cand2, keep2, wl.k, wl.c, what="q18_b1 with the library's own map")


def test_q18_b1_full_size_general_instance(cfm, q18_layer):
    """The batch-1 call through the general per-pair instance (the batch-1 instance switched off)."""
    L, wl = q18_layer, q18_layer.wl
    E, I, H = L.host.w_gate.shape
    used = sorted(set(L.host.ids.reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used, E, I, H)
    with cfm.forward_path(cfm.FORWARD_PER_PAIR_GENERAL):
        got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r)
    compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, what="q18_b1 general instance")


@pytest.mark.parametrize("kc", [(1, 2), (23, 46), (138, 276), (160, 768), (100, 700), (140, 141)],
                         ids=lambda kc: f"k{kc[0]}_c{kc[1]}")
def test_batch1_instance_against_general_and_oracle(cfm, kc):
    """The batch-1 instance (H 2048, r 64, 8 pairs) against the general instance on the same inputs (the
    same candidate and kept sets, bit for bit: both select from identical activations with the same tie
    rule; outputs within float rounding) and against the oracle, over budgets from 1 to 160 kept
    channels and up to every channel a candidate."""
    k, c = kc
    wl = custom_workload(f"lean_k{k}_c{c}", 8, 8, 768, 2048, 1, k, c, 64, 60 + k)
    log(f"batch-1 instance {wl.name}")
    L = upload(wl)
    E, I, H = L.host.w_gate.shape
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, sorted(set(L.host.ids.reshape(-1).tolist())), E, I, H)
    with cfm.forward_path(cfm.FORWARD_PER_PAIR):
        got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), k, c, wl.r)
    with cfm.forward_path(cfm.FORWARD_PER_PAIR_GENERAL):
        got_g, cand_g, keep_g = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), k, c, wl.r)
    assert np.array_equal(cand, cand_g) and np.array_equal(keep, keep_g)
    assert rel_l2(got[0], got_g[0]) <= 1e-2
    compare_forward(L, A, Bt, got, cand, keep, k, c, what=wl.name)


def test_q18_b1_full_size_candidates_exact(cfm, q18_layer):
    """The recovery variant (dropped candidates recovered with their exact activation) at full size."""
    L, wl = q18_layer, q18_layer.wl
    E, I, H = L.host.w_gate.shape
    used = sorted(set(L.host.ids.reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used, E, I, H)
    got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r, recovery="candidates_exact")
    compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, what="q18_b1 candidates_exact", recovery="candidates_exact")


@pytest.mark.parametrize("name", ["q13_b8", "q13_b16", "q18_b8", "q18_b16"])
def test_batched_full_size(cfm, name):
    """Batches of 8 and 16 tokens through both passes (each forced)."""
    wl = synth.WORKLOADS[name]
    log(f"generating {name}")
    L = upload(wl)
    E, I, H = L.host.w_gate.shape
    tokens = [0, wl.T // 2, wl.T - 1]
    used = sorted(set(L.host.ids[tokens].reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used, E, I, H)
    for path in (cfm.FORWARD_GROUPED, cfm.FORWARD_PER_PAIR):
        with cfm.forward_path(path):
            got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r)
        compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, tokens=tokens, what=f"{name} path {path}")


@pytest.mark.parametrize("spec", [("ms_q18_b4", (128, 8, 768, 2048, 4, 138, 276, 64, 37)),
                                  ("ms_q18_b3", (128, 8, 768, 2048, 3, 138, 276, 64, 38)),
                                  ("ms_ragged", (6, 3, 300, 128, 12, 54, 108, 8, 39)),
                                  ("ms_rank6", (6, 3, 300, 128, 12, 54, 108, 6, 40)),
                                  ("ms_h512", (16, 4, 640, 512, 8, 115, 230, 16, 44)),
                                  ("ms_rank0", (16, 4, 640, 512, 8, 115, 230, 0, 45))],
                         ids=lambda s: s[0])
def test_multi_subchunk_instance(cfm, spec):
    """Three or more 32-channel sub-chunks per workgroup below the grouped screen's 40 pairs: the instance that
    keeps the next sub-chunk's sketch rows in flight (path 1) against the general instance (path 3) on the
    same inputs (the same candidate and kept sets bit for bit; outputs within float rounding: the partial
    recovery sums are added in another order), and against the oracle on sampled tokens."""
    name, shape = spec
    wl = custom_workload(name, *shape)
    log(f"multi-sub-chunk instance {name}")
    L = upload(wl)
    E, I, H = L.host.w_gate.shape
    T, K = L.host.ids.shape
    tokens = sorted({0, T // 2, T - 1})
    used_s = sorted(set(L.host.ids[tokens].reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used_s, E, I, H)
    Ag, Btg = (up_bf16(A), up_bf16(Bt)) if wl.r > 0 else (None, None)
    res = {}
    for path in (cfm.FORWARD_PER_PAIR, cfm.FORWARD_PER_PAIR_GENERAL):
        with cfm.forward_path(path):
            res[path] = run_select(cfm, L, sk, Ag, Btg, wl.k, wl.c, wl.r)
    (g1, c1, k1), (g3, c3, k3) = res[cfm.FORWARD_PER_PAIR], res[cfm.FORWARD_PER_PAIR_GENERAL]
    assert np.array_equal(c1, c3) and np.array_equal(k1, k3)
    err = max(rel_l2(g1[t], g3[t]) for t in range(T))
    assert err <= 2e-3, f"{name}: the two instances differ by rel L2 {err:.2e}"
    compare_forward(L, A, Bt, g1, c1, k1, wl.k, wl.c, tokens=tokens, what=f"{name} multi-sub-chunk instance")


@pytest.mark.parametrize("spec", [("q18_b8", None), ("q13_b16", None),
                                  ("ps_small", (16, 4, 256, 512, 16, 46, 92, 8, 33)),
                                  ("ps_ragged", (6, 3, 101, 128, 40, 17, 33, 8, 34)),
                                  ("ps_rank0", (16, 4, 256, 512, 16, 46, 92, 0, 35)),
                                  ("ps_k0_fullrank", (4, 2, 64, 128, 80, 0, 0, 64, 36))],
                         ids=lambda s: s[0])
def test_per_pair_screens_agree(cfm, spec):
    """The per-pair pass with several tokens, its screen run by the expert-grouped screen kernels before
    the single launch (path 1) against the screen inside the launch (path 4), on the same inputs: the same
    candidate and kept sets bit for bit (both select from bit-identical sketch activations and the same
    exact activations), outputs within float rounding (the partial recovery sums are added in another
    order), and the screen's reads requested once per used expert instead of once per pair. Path 1 is
    also checked against the oracle on sampled tokens."""
    name, shape = spec
    wl = synth.WORKLOADS[name] if shape is None else custom_workload(name, *shape)
    log(f"per-pair screens {name}")
    L = upload(wl)
    E, I, H = L.host.w_gate.shape
    T, K = L.host.ids.shape
    tokens = [0, T // 2, T - 1]
    used_s = sorted(set(L.host.ids[tokens].reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used_s, E, I, H)
    Ag, Btg = (up_bf16(A), up_bf16(Bt)) if wl.r > 0 else (None, None)
    res = {}
    for path in (cfm.FORWARD_PER_PAIR, cfm.FORWARD_PER_PAIR_SINGLE):
        with cfm.forward_path(path):
            res[path] = run_select(cfm, L, sk, Ag, Btg, wl.k, wl.c, wl.r, stats=True)
    (g1, c1, k1, s1), (g4, c4, k4, s4) = res[cfm.FORWARD_PER_PAIR], res[cfm.FORWARD_PER_PAIR_SINGLE]
    assert np.array_equal(c1, c4) and np.array_equal(k1, k4)
    err = max(rel_l2(g1[t], g4[t]) for t in range(T))
    assert err <= 2e-3, f"{name}: paths 1 and 4 differ by rel L2 {err:.2e}"
    used = len(set(L.host.ids.reshape(-1).tolist()))
    screen = 2 * I * (H // 4) + 8 * I + 2 * I * wl.r
    assert s4["bytes_requested"] - s1["bytes_requested"] == (T * K - used) * screen, (s1, s4)
    log(f"{name}: paths 1 and 4 agree (max rel L2 {err:.2e}); screen reads {used} experts instead of {T * K} pairs")
    compare_forward(L, A, Bt, g1, c1, k1, wl.k, wl.c, tokens=tokens, what=f"{name} path 1")


@pytest.mark.parametrize("T", [1, 8])
def test_qwen_all_candidates_full_size(cfm, T):
    """Qwen3-30B-A3B-shaped layer with every channel a candidate (c = I = 768) and a 53 % budget
    (k = 407): the screen's top-c is the whole width and the exact pass covers it; both passes."""
    wl = custom_workload(f"q53_all_b{T}", 128, 8, 768, 2048, T, 407, 768, 64, 11)
    log(f"generating {wl.name}")
    L = upload(wl)
    E, I, H = L.host.w_gate.shape
    tokens = sorted({0, T - 1})
    used = sorted(set(L.host.ids[tokens].reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used, E, I, H)
    for path in (cfm.FORWARD_GROUPED, cfm.FORWARD_PER_PAIR):
        with cfm.forward_path(path):
            got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r)
        compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, tokens=tokens, what=f"{wl.name} path {path}")


def test_olmoe_b64_full_size(cfm):
    """OLMoE-shaped layer, 64 tokens with Zipf-skewed experts (hot experts serve most tokens): both passes
    (the automatic choice here is the grouped pass)."""
    wl = synth.WORKLOADS["olmoe_b64"]
    log("generating the OLMoE-shaped layer")
    L = upload(wl)
    E, I, H = L.host.w_gate.shape
    tokens = [0, 31, 63]
    used = sorted(set(L.host.ids[tokens].reshape(-1).tolist()))
    sk = gpu_sketch(cfm, L)
    A, Bt = oracle_map(L.host.w_down_t, wl.r, used, E, I, H)
    for path in (cfm.FORWARD_AUTO, cfm.FORWARD_PER_PAIR):
        with cfm.forward_path(path):
            got, cand, keep = run_select(cfm, L, sk, up_bf16(A), up_bf16(Bt), wl.k, wl.c, wl.r)
        compare_forward(L, A, Bt, got, cand, keep, wl.k, wl.c, tokens=tokens, what=f"olmoe_b64 path {path}")
