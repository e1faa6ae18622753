"""Device helpers for the GPU tests: upload synthetic inputs, read results back.

Inputs always come from the host generator (synth) and are uploaded; nothing the
oracle consumes is produced by the HIP library.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import synth
from oracle import cfm_oracle as O


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


def up_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def down_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


@dataclasses.dataclass
class DevLayer:
    wl: synth.Workload
    host: synth.LayerInputs
    wg: torch.Tensor
    wu: torch.Tensor
    wd: torch.Tensor
    signs: torch.Tensor
    x: torch.Tensor
    ids: torch.Tensor
    w: torch.Tensor


def upload(wl: synth.Workload, host: synth.LayerInputs | None = None) -> DevLayer:
    h = host if host is not None else synth.make_inputs(wl)
    return DevLayer(wl, h, up_bf16(h.w_gate), up_bf16(h.w_up), up_bf16(h.w_down_t), up(h.signs),
                    up_bf16(h.x), up(h.ids.astype(np.int32)), up(h.w.astype(np.float32)))


_MAP_CACHE: dict = {}


def _expert_map(w_rows: np.ndarray, r: int):
    """The oracle's map of one expert (BF16 bits), memoised on the expert's bytes within a session."""
    import hashlib
    key = (hashlib.sha1(np.ascontiguousarray(w_rows).tobytes()).hexdigest(), w_rows.shape, r)
    if key not in _MAP_CACHE:
        a, b = O.lowrank(w_rows, r)
        _MAP_CACHE[key] = (O.f64_to_bf16(a), O.f64_to_bf16(b))
    return _MAP_CACHE[key]


def oracle_map(w_down_t: np.ndarray, r: int, experts, E: int, I: int, H: int):
    """Oracle low-rank maps (BF16 bits) for `experts`; zeros elsewhere (never read)."""
    A = np.zeros((E, H, r), np.uint16)
    Bt = np.zeros((E, I, r), np.uint16)
    for e in experts:
        A[e], Bt[e] = _expert_map(w_down_t[e], r)
    return A, Bt


def custom_workload(name, E, K, I, H, T, k, c, r, seed, chan_scale=True, zipf=None, rmsnorm=True):
    shape = synth.LayerShape(E=E, K=K, I=I, H=H, chan_scale=chan_scale)
    return synth.Workload(name, shape, T=T, k=k, c=c, r=r, seed=seed, rmsnorm_x=rmsnorm, zipf=zipf)
