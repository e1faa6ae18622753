"""ctypes binding of libcfm.so (include/cfm.h).

Argument marshalling only: every step of the computation runs in the HIP
library. PyTorch supplies device memory and the current stream. BF16 arrays
are torch.bfloat16 (or raw torch.int16 / torch.uint16) tensors.

There is no fallback: if libcfm.so is missing the import raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CFM_PHASE_TRACE=1 selects the instrumented build (phase timestamps compiled in)
LIB_PATH = os.path.join(_HERE, "libcfm_trace.so" if os.environ.get("CFM_PHASE_TRACE") == "1" else "libcfm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python calibration_free_channel_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_z = ctypes.c_size_t

_SIGS = {
    "cfm_last_error": (ctypes.c_char_p, []),
    "cfm_version": (ctypes.c_char_p, []),
    "sketch_build": (_i, [_p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _p]),
    "rotation_signs": (_i, [ctypes.c_uint64, _i, _p, _p]),
    "sketch_bytes": (_z, [_i, _i, _i]),
    "sketch_build_seeded": (_i, [_p, _p, _i, _i, _i, ctypes.c_uint64, _p, _p, _p, _p, _p, _p]),
    "lowrank_workspace": (_z, [_i, _i, _i, _i]),
    "lowrank_build": (_i, [_p, _i, _i, _i, _i, _p, _p, _p, _z, _p]),
    "select_workspace": (_z, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "moe_select_forward": (_i, [_p, _p, _p, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p,
                                _p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _z, _p]),
    "moe_select_forward_noalloc": (_i, [_p, _p, _p, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p,
                                        _p, _p, _i, _i, _i, _p, _p, _p, _p, _p]),
    "moe_select_forward_ex": (_i, [_p, _p, _p, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p,
                                   _p, _p, _i, _i, _i, ctypes.c_uint, _p, _p, _p, _p, _p, _z, _p]),
    "moe_select_forward_threshold": (_i, [_p, _p, _p, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p,
                                          _p, _p, ctypes.c_float, _i, _i, ctypes.c_uint, _p, _p, _p, _p, _p,
                                          _p, _z, _p]),
    "moe_layer_forward": (_i, [_p, _p, ctypes.c_float, _p, _i, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p,
                               _p, _p, _i, _i, _i, ctypes.c_uint, _p, _p, _p, _p, _p, _z, _p]),
    "moe_layer_dense_forward": (_i, [_p, _p, ctypes.c_float, _p, _i, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p,
                                     _p, _p, _z, _p]),
    "dense_workspace": (_z, [_i, _i, _i, _i, _i]),
    "moe_dense_forward": (_i, [_p, _p, _p, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _z, _p]),
    "cfm_set_forward_path": (_i, [_i]),
    "cfm_timing_enable": (_i, [_i]),
    "cfm_timing_report": (_i, [ctypes.c_char_p, _z]),
    "cfm_phase_trace": (_i, [_p]),
    "cfm_workspace_status": (_i, [_p, _z, _p]),
    "cfm_set_wait_limit": (_i, [ctypes.c_uint]),
    "cfm_set_resident_limit": (_i, [ctypes.c_int]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)

STATS_FIELDS = ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery", "bytes_io",
                "bytes_dense_equiv", "experts_used", "rows_candidates", "rows_down", "bytes_requested")
STATS_BYTES = 6 * 8 + 4 * 4 + 8


class CfmError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib.cfm_last_error().decode()
        super().__init__(f"{where} failed ({code}): {msg}")
        self.code = code


def _check(code: int, where: str):
    if code != 0:
        raise CfmError(code, where)


def version() -> str:
    return _lib.cfm_version().decode()


def last_error() -> str:
    return _lib.cfm_last_error().decode()


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libcfm must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _bf16(t, name):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold BF16 values (torch.bfloat16), got {t.dtype}")
    return t


# ----------------------------------------------------------------------------- entry points

def sketch_build(w_gate, w_up, signs, out=None):
    """Sketch of every expert's gate and up rows. Returns (tg, tu, sg, su)."""
    _bf16(w_gate, "w_gate"), _bf16(w_up, "w_up")
    E, I, H = w_gate.shape
    if w_up.shape != w_gate.shape or signs.shape != (H,) or signs.dtype != torch.int8:
        raise ValueError("shape/dtype mismatch")
    dev = w_gate.device
    if out is None:
        out = (torch.empty((E, I, H // 4), dtype=torch.uint8, device=dev),
               torch.empty((E, I, H // 4), dtype=torch.uint8, device=dev),
               torch.empty((E, I), dtype=torch.float32, device=dev),
               torch.empty((E, I), dtype=torch.float32, device=dev))
    tg, tu, sg, su = out
    _check(_lib.sketch_build(_ptr(w_gate), _ptr(w_up), E, I, H, _ptr(signs), _ptr(tg), _ptr(tu),
                             _ptr(sg), _ptr(su), _stream(dev)), "sketch_build")
    return tg, tu, sg, su


def rotation_signs(seed: int, H: int, device="cuda", out=None):
    """The layer's rotation signs (int8 [H], +-1) from a 64-bit seed (SplitMix64, bit 63)."""
    if out is None:
        out = torch.empty(H, dtype=torch.int8, device=device)
    if out.dtype != torch.int8 or out.numel() != H:
        raise ValueError("signs: int8 tensor of H entries")
    _check(_lib.rotation_signs(ctypes.c_uint64(seed & (2**64 - 1)), H, _ptr(out), _stream(out.device)),
           "rotation_signs")
    return out


def sketch_bytes(E: int, I: int, H: int) -> int:
    """Device bytes of one layer's sketch (codes, scales and signs)."""
    return int(_lib.sketch_bytes(E, I, H))


def sketch_build_seeded(w_gate, w_up, seed: int, out=None):
    """Signs from `seed`, then the sketch. Returns (signs, tg, tu, sg, su)."""
    _bf16(w_gate, "w_gate"), _bf16(w_up, "w_up")
    E, I, H = w_gate.shape
    if w_up.shape != w_gate.shape:
        raise ValueError("shape mismatch")
    dev = w_gate.device
    if out is None:
        out = (torch.empty(H, dtype=torch.int8, device=dev),
               torch.empty((E, I, H // 4), dtype=torch.uint8, device=dev),
               torch.empty((E, I, H // 4), dtype=torch.uint8, device=dev),
               torch.empty((E, I), dtype=torch.float32, device=dev),
               torch.empty((E, I), dtype=torch.float32, device=dev))
    signs, tg, tu, sg, su = out
    _check(_lib.sketch_build_seeded(_ptr(w_gate), _ptr(w_up), E, I, H, ctypes.c_uint64(seed & (2**64 - 1)),
                                    _ptr(signs), _ptr(tg), _ptr(tu), _ptr(sg), _ptr(su), _stream(dev)),
           "sketch_build_seeded")
    return signs, tg, tu, sg, su


def lowrank_workspace(E, I, H, r) -> int:
    return int(_lib.lowrank_workspace(E, I, H, r))


def lowrank_build(w_down_t, r, ws=None, out=None):
    """Rank-r map of every expert's down projection. Returns (A [E][H][r], Bt [E][I][r]) BF16."""
    _bf16(w_down_t, "w_down_t")
    E, I, H = w_down_t.shape
    dev = w_down_t.device
    if out is None:
        out = (torch.empty((E, H, r), dtype=torch.bfloat16, device=dev),
               torch.empty((E, I, r), dtype=torch.bfloat16, device=dev))
    A, Bt = out
    if r == 0:
        return A, Bt
    need = lowrank_workspace(E, I, H, r)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(_lib.lowrank_build(_ptr(w_down_t), E, I, H, r, _ptr(A), _ptr(Bt), _ptr(ws), ws.numel(),
                              _stream(dev)), "lowrank_build")
    return A, Bt


def select_workspace(T, K, E, I, H, k, c, r) -> int:
    return int(_lib.select_workspace(T, K, E, I, H, k, c, r))


def dense_workspace(T, K, E, I, H) -> int:
    return int(_lib.dense_workspace(T, K, E, I, H))


def new_workspace(nbytes, device):
    """A zero-filled workspace (the forward calls require zeroed memory on first use)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


RECOVER_SKETCH = "sketch"                       # every skipped channel enters the map with hhat
RECOVER_CANDIDATES_EXACT = "candidates_exact"   # dropped candidates enter with their exact h
_RECOVER_FLAGS = {RECOVER_SKETCH: 0, RECOVER_CANDIDATES_EXACT: 1}   # CFM_RECOVER_CANDIDATES_EXACT


def moe_select_forward(x, topk_ids, topk_w, w_gate, w_up, w_down_t, signs, tg, tu, sg, su, A, Bt,
                       k, c, r, out=None, ws=None, cand_out=None, keep_out=None, stats=None,
                       recovery=RECOVER_SKETCH):
    """Selected-channel MoE layer. Returns out [T][H] BF16.

    recovery: RECOVER_SKETCH (moe_select_forward) or RECOVER_CANDIDATES_EXACT
    (moe_select_forward_ex with CFM_RECOVER_CANDIDATES_EXACT)."""
    if recovery not in _RECOVER_FLAGS:
        raise ValueError(f"unknown recovery variant {recovery!r}")
    T, H = x.shape
    K = topk_ids.shape[1]
    E, I, _ = w_gate.shape
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = new_workspace(select_workspace(T, K, E, I, H, k, c, r), dev)
    head = (_ptr(x), _ptr(topk_ids), _ptr(topk_w), T, K, _ptr(w_gate), _ptr(w_up), _ptr(w_down_t),
            E, I, H, _ptr(signs), _ptr(tg), _ptr(tu), _ptr(sg), _ptr(su),
            _ptr(A) if r > 0 else None, _ptr(Bt) if r > 0 else None, k, c, r)
    tail = (_ptr(out), _ptr(cand_out), _ptr(keep_out), _ptr(stats), _ptr(ws), ws.numel(), _stream(dev))
    flags = _RECOVER_FLAGS[recovery]
    if flags:
        _check(_lib.moe_select_forward_ex(*head, flags, *tail), "moe_select_forward_ex")
    else:
        _check(_lib.moe_select_forward(*head, *tail), "moe_select_forward")
    return out


def moe_select_forward_noalloc(x, topk_ids, topk_w, w_gate, w_up, w_down_t, signs, tg, tu, sg, su, A, Bt,
                               k, c, r, out=None, cand_out=None, keep_out=None, stats=None):
    """moe_select_forward on the library's own per-GPU scratch (no workspace argument; the call
    allocates no device memory when `out` is given). Returns out [T][H] BF16."""
    T, H = x.shape
    K = topk_ids.shape[1]
    E, I, _ = w_gate.shape
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(_lib.moe_select_forward_noalloc(
        _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, K, _ptr(w_gate), _ptr(w_up), _ptr(w_down_t), E, I, H,
        _ptr(signs), _ptr(tg), _ptr(tu), _ptr(sg), _ptr(su), _ptr(A) if r > 0 else None,
        _ptr(Bt) if r > 0 else None, k, c, r, _ptr(out), _ptr(cand_out), _ptr(keep_out), _ptr(stats),
        _stream(dev)), "moe_select_forward_noalloc")
    return out


def moe_select_forward_threshold(x, topk_ids, topk_w, w_gate, w_up, w_down_t, signs, tg, tu, sg, su, A, Bt,
                                 tau, c, r, out=None, ws=None, cand_out=None, keep_out=None, keep_count=None,
                                 stats=None, recovery=RECOVER_SKETCH):
    """Selected-channel MoE layer with the threshold keep rule S = {j in C : |h_j| >= tau}.

    keep_out: optional [T*K][c] int32 (S ascending, then -1); keep_count:
    optional [T*K] int32. Returns out [T][H] BF16."""
    if recovery not in _RECOVER_FLAGS:
        raise ValueError(f"unknown recovery variant {recovery!r}")
    T, H = x.shape
    K = topk_ids.shape[1]
    E, I, _ = w_gate.shape
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = new_workspace(select_workspace(T, K, E, I, H, c, c, r), dev)
    _check(_lib.moe_select_forward_threshold(
        _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, K, _ptr(w_gate), _ptr(w_up), _ptr(w_down_t),
        E, I, H, _ptr(signs), _ptr(tg), _ptr(tu), _ptr(sg), _ptr(su),
        _ptr(A) if r > 0 else None, _ptr(Bt) if r > 0 else None, float(tau), c, r, _RECOVER_FLAGS[recovery],
        _ptr(out), _ptr(cand_out), _ptr(keep_out), _ptr(keep_count), _ptr(stats), _ptr(ws), ws.numel(),
        _stream(dev)), "moe_select_forward_threshold")
    return out


def moe_dense_forward(x, topk_ids, topk_w, w_gate, w_up, w_down_t, out=None, ws=None):
    """Dense routed-expert SwiGLU layer (every channel). Returns out [T][H] BF16."""
    T, H = x.shape
    K = topk_ids.shape[1]
    E, I, _ = w_gate.shape
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = new_workspace(dense_workspace(T, K, E, I, H), dev)
    _check(_lib.moe_dense_forward(
        _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, K, _ptr(w_gate), _ptr(w_up), _ptr(w_down_t),
        E, I, H, _ptr(out), _ptr(ws), ws.numel(), _stream(dev)), "moe_dense_forward")
    return out


def moe_layer_forward(h, norm_w, eps, w_router, K, w_gate, w_up, w_down_t, signs, tg, tu, sg, su, A, Bt,
                      k, c, r, renorm=False, out=None, ws=None, ids_out=None, w_out=None, x_out=None,
                      recovery=RECOVER_SKETCH):
    """The routed-expert block of a decode layer with its envelope (RMSNorm, router, residual add) in one
    launch. Returns out [T][H] BF16 (h + block output); out may be h."""
    if recovery not in _RECOVER_FLAGS:
        raise ValueError(f"unknown recovery variant {recovery!r}")
    T, H = h.shape
    E, I, _ = w_gate.shape
    dev = h.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = new_workspace(select_workspace(T, K, E, I, H, k, c, r), dev)
    _check(_lib.moe_layer_forward(
        _ptr(h), _ptr(norm_w), float(eps), _ptr(w_router), 1 if renorm else 0, T, K, _ptr(w_gate), _ptr(w_up),
        _ptr(w_down_t), E, I, H, _ptr(signs), _ptr(tg), _ptr(tu), _ptr(sg), _ptr(su),
        _ptr(A) if r > 0 else None, _ptr(Bt) if r > 0 else None, k, c, r, _RECOVER_FLAGS[recovery], _ptr(out),
        _ptr(ids_out), _ptr(w_out), _ptr(x_out), _ptr(ws), ws.numel(), _stream(dev)), "moe_layer_forward")
    return out


def moe_layer_dense_forward(h, norm_w, eps, w_router, K, w_gate, w_up, w_down_t, renorm=False, out=None, ws=None,
                            ids_out=None, w_out=None, x_out=None):
    """The same envelope around the dense block. Returns out [T][H] BF16."""
    T, H = h.shape
    E, I, _ = w_gate.shape
    dev = h.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = new_workspace(dense_workspace(T, K, E, I, H), dev)
    _check(_lib.moe_layer_dense_forward(
        _ptr(h), _ptr(norm_w), float(eps), _ptr(w_router), 1 if renorm else 0, T, K, _ptr(w_gate), _ptr(w_up),
        _ptr(w_down_t), E, I, H, _ptr(out), _ptr(ids_out), _ptr(w_out), _ptr(x_out), _ptr(ws), ws.numel(),
        _stream(dev)), "moe_layer_dense_forward")
    return out


FORWARD_AUTO, FORWARD_PER_PAIR, FORWARD_GROUPED, FORWARD_PER_PAIR_GENERAL, FORWARD_PER_PAIR_SINGLE = 0, 1, 2, 3, 4


def set_forward_path(path: int) -> int:
    """Select the forward kernels (0 automatic, 1 per-pair, 2 expert-grouped, 3 per-pair on the general instance
    only, 4 per-pair with the screen always inside the single launch); returns the previous setting."""
    prev = _lib.cfm_set_forward_path(int(path))
    if prev < 0:
        raise CfmError(prev, "cfm_set_forward_path")
    return prev


class forward_path:
    """Context manager: run the enclosed forward calls on the given path."""

    def __init__(self, path: int):
        self.path = path

    def __enter__(self):
        self.prev = set_forward_path(self.path)
        return self

    def __exit__(self, *exc):
        set_forward_path(self.prev)
        return False


def timing_enable(on: bool = True):
    """Bracket every library kernel launch with HIP events (instrumentation)."""
    _lib.cfm_timing_enable(1 if on else 0)


def timing_report() -> dict:
    """{kernel name: (launches, total_ms)} since the last report; synchronises the events."""
    buf = ctypes.create_string_buffer(1 << 16)
    n = _lib.cfm_timing_report(buf, len(buf))
    if n < 0:
        raise CfmError(n, "cfm_timing_report")
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


def workspace_status(ws) -> int:
    """Synchronise the current stream, read and clear the workspace's failure word: 0 if no bounded
    wait of a forward call on it expired since the last check, else CFM_ETIMEOUT (-5)."""
    return int(_lib.cfm_workspace_status(_ptr(ws), ws.numel(), _stream(ws.device)))


def set_wait_limit(polls: int) -> int:
    """Polls of one exchanged value before a single-launch forward call gives up (default 2^20;
    0: every wait gives up at once, for testing the failure path). Returns the previous value."""
    return int(_lib.cfm_set_wait_limit(int(polls)))


def set_resident_limit(workgroups: int) -> int:
    """Cap on the workgroups a single-launch forward call assumes resident (-1: the device's own count;
    0: none, so the call is refused). Returns the previous value."""
    return int(_lib.cfm_set_resident_limit(int(workgroups)))


def phase_trace(buf):
    """Phase timestamps of every later per-pair launch into buf (int64 device tensor of at least
    256 * 32 entries; None stops). Needs the trace build (CFM_PHASE_TRACE=1)."""
    if buf is not None and (buf.dtype != torch.int64 or buf.numel() < 256 * 32):
        raise ValueError("phase-trace buffer: int64 tensor of at least 256 * 32 entries")
    _check(_lib.cfm_phase_trace(_ptr(buf)), "cfm_phase_trace")


def decode_stats(buf) -> dict:
    """cfm_stats bytes (a uint8 tensor of STATS_BYTES) -> dict."""
    import numpy as np
    raw = buf.detach().cpu().numpy().tobytes()
    u64 = np.frombuffer(raw[:48], dtype="<u8")
    u32 = np.frombuffer(raw[48:64], dtype="<u4")
    req = np.frombuffer(raw[64:72], dtype="<u8")
    vals = list(map(int, u64)) + list(map(int, u32[:3])) + [int(req[0])]
    return dict(zip(STATS_FIELDS, vals))
