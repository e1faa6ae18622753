"""The no-allocation entry point (moe_select_forward_noalloc) against
moe_select_forward with a workspace of its own, on two calls in a row, the
second with fewer tokens: outputs, candidate and kept sets equal bit for bit
(both passes are deterministic). Runs last in the GPU suite."""
import numpy as np
import pytest
import torch

from gpu_util import custom_workload, dev, down_bf16, log, oracle_map, up_bf16, upload

pytestmark = pytest.mark.gpu
EWORKSPACE = -3


@pytest.fixture(scope="module")
def cfm():
    import calibration_free_channel_amd as m
    return m


def _run(cfm, L, A, Bt, sk, T, k, c, r, noalloc):
    x, ids, w = L.x[:T].contiguous(), L.ids[:T].contiguous(), L.w[:T].contiguous()
    K = ids.shape[1]
    cand = torch.full((T * K, c), -7, dtype=torch.int32, device=dev())
    keep = torch.full((T * K, k), -7, dtype=torch.int32, device=dev())
    out = torch.empty((T, x.shape[1]), dtype=torch.bfloat16, device=dev())
    fn = cfm.moe_select_forward_noalloc if noalloc else cfm.moe_select_forward
    fn(x, ids, w, L.wg, L.wu, L.wd, L.signs, *sk, A, Bt, k, c, r, out=out, cand_out=cand, keep_out=keep)
    torch.cuda.synchronize()
    return down_bf16(out), cand.cpu().numpy(), keep.cpu().numpy()


@pytest.mark.parametrize("shape", ["qwen_like", "small", "screened"])
def test_noalloc_matches_workspace_entry(cfm, shape):
    if shape == "qwen_like":   # H 2048, I 768, 18 %: 4 tokens (16 pairs), then 2 tokens (8 pairs, the lean kernel)
        wl = custom_workload("noalloc_q", 16, 4, 768, 2048, 4, 138, 276, 64, 41)
        sizes = (4, 2)
    elif shape == "screened":  # 16 tokens (64 pairs), then 10 (40): the grouped screen runs before the launch
        wl = custom_workload("noalloc_g", 16, 4, 768, 2048, 16, 138, 276, 64, 43)
        sizes = (16, 10)
    else:
        wl = custom_workload("noalloc_s", 12, 3, 200, 256, 9, 36, 72, 8, 42)
        sizes = (9, 3)
    log(f"noalloc {shape}")
    L = upload(wl)
    h = L.host
    E, I, H = h.w_gate.shape
    used = sorted(set(int(e) for e in h.ids.reshape(-1)))
    A, Bt = (up_bf16(a) for a in oracle_map(h.w_down_t, wl.r, used, E, I, H))
    sk = cfm.sketch_build(L.wg, L.wu, L.signs)
    for T in sizes:
        got = _run(cfm, L, A, Bt, sk, T, wl.k, wl.c, wl.r, True)
        want = _run(cfm, L, A, Bt, sk, T, wl.k, wl.c, wl.r, False)
        for g, w_, what in zip(got, want, ("out", "cand", "keep")):
            assert np.array_equal(g, w_), f"{shape} T={T}: {what} differs from moe_select_forward"


def test_noalloc_rejects_oversized_call(cfm):
    log("noalloc oversized")
    T, K, E, I, H, k, c, r = 128, 8, 128, 768, 2048, 138, 276, 64
    assert cfm.select_workspace(T, K, E, I, H, k, c, r) > 32 << 20
    fake = torch.zeros(1, dtype=torch.bfloat16, device=dev())
    lib = cfm._lib._lib
    import ctypes
    P = ctypes.c_void_p(fake.data_ptr())
    rc = lib.moe_select_forward_noalloc(P, P, P, T, K, P, P, P, E, I, H, P, P, P, P, P, P, P, k, c, r, P,
                                        None, None, None, None)
    assert rc == EWORKSPACE and "32 MiB" in cfm.last_error()
