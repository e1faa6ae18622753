"""GPU checks of the boundary itself: the seeded rotation signs, the seeded
sketch build, workspace reuse across shapes and passes, and the failure channel
of the single-launch pass (forced from the host through the wait limit, so that
every workgroup still runs to its end)."""
import numpy as np
import pytest
import torch

import synth
from oracle import cfm_oracle as O
from gpu_util import custom_workload, dev, down_bf16, log, oracle_map, upload

pytestmark = pytest.mark.gpu
ETIMEOUT = -5


@pytest.fixture(scope="module")
def cfm():
    import calibration_free_channel_amd as m
    return m


@pytest.mark.parametrize("seed", [0, 1, 1234567, (1 << 63) + 5, (1 << 64) - 1])
@pytest.mark.parametrize("H", [1, 64, 1000, 2048, 8192])
def test_rotation_signs_bitwise(cfm, seed, H):
    log(f"rotation_signs seed={seed} H={H}")
    got = cfm.rotation_signs(seed, H, device=dev())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.rotation_signs(seed, H))


@pytest.mark.parametrize("wl", [synth.WORKLOADS["tiny"], custom_workload("ragged", 6, 3, 101, 128, 5, 17, 33, 6, 5)],
                         ids=lambda w: w.name)
def test_sketch_build_seeded_bitwise(cfm, wl):
    log(f"sketch_build_seeded {wl.name}")
    L = upload(wl)
    seed = 77 + wl.shape.H
    signs, tg, tu, sg, su = cfm.sketch_build_seeded(L.wg, L.wu, seed)
    torch.cuda.synchronize()
    osigns = O.rotation_signs(seed, wl.shape.H)
    assert np.array_equal(signs.cpu().numpy(), osigns)
    otg, otu, osg, osu = O.sketch_build(L.host.w_gate, L.host.w_up, osigns)
    assert np.array_equal(tg.cpu().numpy(), otg) and np.array_equal(tu.cpu().numpy(), otu)
    assert np.array_equal(sg.cpu().numpy().view(np.uint32), osg.view(np.uint32))
    assert np.array_equal(su.cpu().numpy().view(np.uint32), osu.view(np.uint32))
    assert cfm.sketch_bytes(*L.wg.shape) == 2 * tg.numel() + 4 * 2 * sg.numel() + signs.numel()


def _layer_and_map(wl):
    L = upload(wl)
    h = L.host
    E, I, H = h.w_gate.shape
    used = sorted(set(int(e) for e in h.ids.reshape(-1)))
    A, Bt = oracle_map(h.w_down_t, wl.r, used, E, I, H)
    from gpu_util import up_bf16
    return L, up_bf16(A), up_bf16(Bt)


@pytest.mark.parametrize("path", ["per_pair", "grouped", "per_pair_screened"])
def test_workspace_reuse_across_shapes(cfm, path):
    """T = 1, then T = 8 (16 with the per-pair pass's grouped screen in front), then T = 1 again, then
    the dense layer, on one workspace: each result equals the same call on a fresh workspace, bit for
    bit (the calls are deterministic)."""
    log(f"workspace reuse {path}")
    big = 16 if path == "per_pair_screened" else 8          # 64 routed pairs: the grouped screen runs first
    wl8 = custom_workload(f"reuse{big}", 16, 4, 256, 512, big, 46, 92, 8, 31)
    L, A, Bt = _layer_and_map(wl8)
    sk = cfm.sketch_build(L.wg, L.wu, L.signs)
    E, I, H = L.host.w_gate.shape
    K = L.host.ids.shape[1]
    k, c, r = wl8.k, wl8.c, wl8.r
    sizes = [cfm.select_workspace(T, K, E, I, H, k, c, r) for T in (1, big)] + [cfm.dense_workspace(big, K, E, I, H)]
    shared = cfm.new_workspace(max(sizes), dev())
    mode = cfm.FORWARD_GROUPED if path == "grouped" else cfm.FORWARD_PER_PAIR

    def sel(T, ws):
        return down_bf16(cfm.moe_select_forward(L.x[:T].contiguous(), L.ids[:T].contiguous(), L.w[:T].contiguous(),
                                                L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, k, c, r, ws=ws))

    def dense(T, ws):
        return down_bf16(cfm.moe_dense_forward(L.x[:T].contiguous(), L.ids[:T].contiguous(), L.w[:T].contiguous(),
                                               L.wg, L.wu, L.wd, ws=ws))
    with cfm.forward_path(mode):
        for step, (fn, T) in enumerate([(sel, 1), (sel, big), (sel, 1), (dense, big), (sel, big)]):
            got = fn(T, shared)
            want = fn(T, None)
            torch.cuda.synchronize()
            assert np.array_equal(got, want), f"step {step}: {fn.__name__} T={T} differs on a reused workspace"
            assert cfm.workspace_status(shared) == 0


def test_failure_channel_forced_from_host(cfm):
    """With the wait limit at 0 every exchange wait gives up at once: the call's outputs are NaN and
    workspace_status reports the expiry once; with the limit restored the next call is correct."""
    log("failure channel")
    wl = synth.WORKLOADS["tiny"]
    L, A, Bt = _layer_and_map(wl)
    sk = cfm.sketch_build(L.wg, L.wu, L.signs)
    E, I, H = L.host.w_gate.shape
    K = L.host.ids.shape[1]
    ws = cfm.new_workspace(cfm.select_workspace(1, K, E, I, H, wl.k, wl.c, wl.r), dev())
    with cfm.forward_path(cfm.FORWARD_PER_PAIR):
        good = down_bf16(cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt,
                                                wl.k, wl.c, wl.r, ws=ws))
        assert cfm.workspace_status(ws) == 0
        prev = cfm.set_wait_limit(0)
        try:
            bad = down_bf16(cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt,
                                                   wl.k, wl.c, wl.r, ws=ws))
            dbad = down_bf16(cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, ws=ws))
        finally:
            cfm.set_wait_limit(prev)
        assert cfm.workspace_status(ws) == ETIMEOUT
        assert "bounded wait expired" in cfm.last_error()
        assert cfm.workspace_status(ws) == 0             # read and cleared
        nan = lambda b: (b & 0x7FFF) > 0x7F80
        assert nan(bad).all() and nan(dbad).all()
        again = down_bf16(cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt,
                                                 wl.k, wl.c, wl.r, ws=ws))
        assert np.array_equal(again, good)
        assert cfm.workspace_status(ws) == 0


def test_resident_limit_rounds_and_refusal(cfm):
    """A device that holds fewer workgroups than the grid wants: the single launch runs the routed pairs
    in rounds and gives the same result; one that holds none is refused before anything is launched."""
    log("resident limit")
    wl = custom_workload("resident", 8, 8, 768, 2048, 2, 138, 276, 64, 53)
    L, A, Bt = _layer_and_map(wl)
    sk = cfm.sketch_build(L.wg, L.wu, L.signs)
    with cfm.forward_path(cfm.FORWARD_PER_PAIR):
        want = down_bf16(cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt,
                                                wl.k, wl.c, wl.r))
        dwant = down_bf16(cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd))
        prev = cfm.set_resident_limit(5)
        try:
            got = down_bf16(cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt,
                                                   wl.k, wl.c, wl.r))
            dgot = down_bf16(cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd))
            cfm.set_resident_limit(0)
            with pytest.raises(cfm.CfmError, match="cannot hold one workgroup"):
                cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, wl.k, wl.c, wl.r)
            with pytest.raises(cfm.CfmError, match="cannot hold one workgroup"):
                cfm.moe_dense_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd)
        finally:
            cfm.set_resident_limit(prev)
        torch.cuda.synchronize()
    # the same sets and arithmetic per pair; only the order of the partial sums over slices differs
    for a, b in ((got, want), (dgot, dwant)):
        fa, fb = O.bf16_to_f64(a), O.bf16_to_f64(b)
        assert np.linalg.norm(fa - fb) <= 1e-2 * np.linalg.norm(fb)


@pytest.mark.parametrize("which", ["lean", "general"])
def test_bytes_requested(cfm, which):
    """bytes_requested equals the kept-row count where only kept rows are read (the lean batch-1
    instance: 8 pairs, H 2048, I 768, r 64) and adds the candidates' down rows where they are
    prefetched (the general instance, here at H 256)."""
    log(f"bytes_requested {which}")
    if which == "lean":
        wl = custom_workload("req_lean", 8, 8, 768, 2048, 1, 138, 276, 64, 51)
    else:
        wl = custom_workload("req_gen", 8, 2, 128, 256, 1, 23, 46, 8, 52, chan_scale=False)
    L, A, Bt = _layer_and_map(wl)
    sk = cfm.sketch_build(L.wg, L.wu, L.signs)
    st = torch.zeros(cfm.STATS_BYTES, dtype=torch.uint8, device=dev())
    with cfm.forward_path(cfm.FORWARD_PER_PAIR):
        cfm.moe_select_forward(L.x, L.ids, L.w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, wl.k, wl.c, wl.r, stats=st)
    torch.cuda.synchronize()
    d = cfm.decode_stats(st)
    algo = sum(d[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery", "bytes_io"))
    P = L.host.ids.size
    H = L.host.w_gate.shape[2]
    if which == "lean":
        assert d["bytes_requested"] == algo
    else:
        assert d["bytes_requested"] == algo - d["bytes_down"] + P * 2 * H * wl.c
    assert cfm.workspace_status(cfm.new_workspace(2048, dev())) == 0
