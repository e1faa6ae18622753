"""Seeded synthetic inputs for the selected-channel MoE FFN.

This module only draws inputs: BF16 expert weights, hidden states, router
outputs and the rotation sign vector. It holds none of the method's
arithmetic (no transform, no sketch, no selection, no projection), so both the
CPU oracle (``oracle/``) and the HIP path (through its Python binding) can be
fed from it without sharing any of the computation under test.

The workloads stand in for the decode traffic of the models named on the
pages (Qwen3-30B-A3B-shaped and OLMoE-1B-7B-shaped MoE layers, arXiv:2610.37386,
"Numbers and limits"); no model weights or evaluation data are used.

Every tensor comes from its own counter-derived stream,
``SeedSequence([seed, layer, tensor_id, expert])``, so any single expert of any
layer can be regenerated on its own (the oracle checks a few experts of a
full-size layer without regenerating the rest).

BF16 values are produced by rounding float32 samples to the nearest BF16
(ties to even) and are returned as raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import numpy as np

# tensor ids for the per-tensor streams
_T_GATE, _T_UP, _T_DOWN = 1, 2, 3
_T_SCALE_GATE, _T_SCALE_UP, _T_SCALE_DOWN = 4, 5, 6
_T_X, _T_LOGITS, _T_SIGNS, _T_ZIPF_PERM, _T_ZIPF_DRAW = 7, 8, 9, 10, 11
_T_ROUTER, _T_NORM, _T_RESID = 12, 13, 14


def _rng(seed: int, layer: int, tensor: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, tensor, sub])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest BF16 (ties to even); return raw bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw BF16 bits to float64."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    E: int          # routed experts
    K: int          # experts per token
    I: int          # SwiGLU intermediate width per expert
    H: int          # hidden width
    sigma: float = 0.02          # weight std
    chan_scale: bool = False     # per-channel LogNormal(0, 0.5) factor


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    T: int                 # tokens in the decode batch
    k: int                 # kept channels per (token, expert) pair
    c: int                 # screened candidates per pair
    r: int                 # recovery rank
    seed: int
    rmsnorm_x: bool = False
    zipf: float | None = None   # expert-popularity exponent (None: softmax routing)
    layers: int = 1


QWEN3_30B_A3B = LayerShape(E=128, K=8, I=768, H=2048, chan_scale=True)
OLMOE_1B_7B = LayerShape(E=64, K=8, I=1024, H=2048, chan_scale=False)
TINY = LayerShape(E=8, K=2, I=128, H=256, chan_scale=False)


def budget_to_kc(frac: float, I: int) -> tuple[int, int]:
    """Read budget f (fraction of the intermediate width) -> (k, c=min(2k, I))."""
    k = int(round(frac * I))
    return k, min(2 * k, I)


WORKLOADS: dict[str, Workload] = {
    # tiny layer that the oracle checks in seconds
    "tiny": Workload("tiny", TINY, T=1, k=23, c=46, r=8, seed=0),
    # Qwen3-30B-A3B-shaped layer, batch-1 decode, 18 % budget
    "q18_b1": Workload("q18_b1", QWEN3_30B_A3B, T=1, k=138, c=276, r=64, seed=1, rmsnorm_x=True),
    # same layer, 13 % budget, decode batches of 8 and 16 tokens
    "q13_b8": Workload("q13_b8", QWEN3_30B_A3B, T=8, k=100, c=200, r=64, seed=2, rmsnorm_x=True),
    "q13_b16": Workload("q13_b16", QWEN3_30B_A3B, T=16, k=100, c=200, r=64, seed=2, rmsnorm_x=True),
    # the 18 % budget at batches 8 and 16 as well
    "q18_b8": Workload("q18_b8", QWEN3_30B_A3B, T=8, k=138, c=276, r=64, seed=2, rmsnorm_x=True),
    "q18_b16": Workload("q18_b16", QWEN3_30B_A3B, T=16, k=138, c=276, r=64, seed=2, rmsnorm_x=True),
    # OLMoE-1B-7B-shaped layer, 64 tokens, Zipf(1.1) expert popularity
    "olmoe_b64": Workload("olmoe_b64", OLMOE_1B_7B, T=64, k=184, c=368, r=64, seed=3, zipf=1.1),
}


def stack_workload(T: int, frac: float, layers: int = 48) -> Workload:
    """48-layer stack of Qwen3-30B-A3B-shaped layers at batch T and budget frac."""
    k, c = budget_to_kc(frac, QWEN3_30B_A3B.I)
    return Workload(f"stack{layers}_b{T}_f{int(round(frac * 100))}", QWEN3_30B_A3B, T=T, k=k, c=c,
                    r=64, seed=4, rmsnorm_x=True, layers=layers)


# ----------------------------------------------------------------------------- weights

def expert_matrix(shape: LayerShape, seed: int, layer: int, which: str, e: int) -> np.ndarray:
    """One expert's [I][H] BF16 matrix (raw bits). which in {'gate','up','down'}.

    'down' is returned channel-major: row j is column j of W_down, so each
    row is the H-vector that intermediate channel j writes to the output.
    """
    tid = {"gate": _T_GATE, "up": _T_UP, "down": _T_DOWN}[which]
    sid = {"gate": _T_SCALE_GATE, "up": _T_SCALE_UP, "down": _T_SCALE_DOWN}[which]
    z = _rng(seed, layer, tid, e).standard_normal((shape.I, shape.H), dtype=np.float32)
    z *= np.float32(shape.sigma)
    if shape.chan_scale:
        s = _rng(seed, layer, sid, e).lognormal(0.0, 0.5, size=shape.I).astype(np.float32)
        z *= s[:, None]
    return f32_to_bf16_bits(z)


def layer_weights(shape: LayerShape, seed: int, layer: int = 0, experts=None):
    """(w_gate, w_up, w_down_t), each [E][I][H] uint16; experts=None -> all."""
    ids = range(shape.E) if experts is None else experts
    out = []
    for which in ("gate", "up", "down"):
        out.append(np.stack([expert_matrix(shape, seed, layer, which, e) for e in ids]))
    return tuple(out)


def rotation_signs(H: int, seed: int, layer: int = 0) -> np.ndarray:
    """The layer's random +-1 vector for the rotation (int8 [H])."""
    bits = _rng(seed, layer, _T_SIGNS).integers(0, 2, size=H)
    return np.where(bits == 1, -1, 1).astype(np.int8)


# ----------------------------------------------------------------------------- tokens

def hidden_states(T: int, H: int, seed: int, layer: int = 0, rmsnorm: bool = False) -> np.ndarray:
    """[T][H] BF16 bits; N(0,1), optionally RMS-normalised (eps 1e-6, unit gain)."""
    z = _rng(seed, layer, _T_X).standard_normal((T, H))
    if rmsnorm and T > 0:
        z = z / np.sqrt(np.mean(z * z, axis=1, keepdims=True) + 1e-6)
    return f32_to_bf16_bits(z.astype(np.float32))


# ----------------------------------------------------------------------------- decode-layer envelope inputs

def router_weights(E: int, H: int, seed: int, layer: int = 0, sigma: float = 0.02) -> np.ndarray:
    """Router rows W_r [E][H] BF16 bits, N(0, sigma)."""
    return f32_to_bf16_bits((_rng(seed, layer, _T_ROUTER).standard_normal((E, H)) * sigma).astype(np.float32))


def norm_weight(H: int, seed: int, layer: int = 0) -> np.ndarray:
    """RMSNorm weight [H] BF16 bits, 1 + 0.1 N(0, 1)."""
    return f32_to_bf16_bits((1.0 + 0.1 * _rng(seed, layer, _T_NORM).standard_normal(H)).astype(np.float32))


def residual_states(T: int, H: int, seed: int, layer: int = 0, scale: float = 1.0) -> np.ndarray:
    """The residual stream entering a decode layer's MoE block, [T][H] BF16 bits, N(0, scale^2)."""
    return f32_to_bf16_bits((scale * _rng(seed, layer, _T_RESID).standard_normal((T, H))).astype(np.float32))


def routing(T: int, E: int, K: int, seed: int, layer: int = 0, zipf: float | None = None):
    """Router output: (topk_ids int32 [T][K], topk_w float32 [T][K]).

    Softmax routing: logits ~ N(0,1) per (token, expert), softmax over E, the
    K largest probabilities (lower id first on ties), weights not renormalised.

    Zipf routing: expert popularity p(rank) ~ rank^-zipf over a seeded
    permutation of ids; each token draws K distinct experts sequentially
    without replacement; its weights are the softmax of K N(0,1) logits.
    """
    if T == 0:
        return np.zeros((0, K), np.int32), np.zeros((0, K), np.float32)
    if zipf is None:
        logits = _rng(seed, layer, _T_LOGITS).standard_normal((T, E))
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -p), axis=1)[:, :K]
        ids = order.astype(np.int32)
        w = np.take_along_axis(p, order, axis=1).astype(np.float32)
        return ids, w
    perm = _rng(seed, layer, _T_ZIPF_PERM).permutation(E)
    pop = np.arange(1, E + 1, dtype=np.float64) ** (-zipf)
    rng = _rng(seed, layer, _T_ZIPF_DRAW)
    ids = np.zeros((T, K), np.int32)
    for t in range(T):
        avail = np.ones(E, bool)
        for q in range(K):
            pr = np.where(avail, pop, 0.0)
            rank = rng.choice(E, p=pr / pr.sum())
            avail[rank] = False
            ids[t, q] = perm[rank]
    lg = _rng(seed, layer, _T_LOGITS).standard_normal((T, K))
    w = np.exp(lg - lg.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


@dataclasses.dataclass
class LayerInputs:
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down_t: np.ndarray
    signs: np.ndarray
    x: np.ndarray
    ids: np.ndarray
    w: np.ndarray


def make_inputs(wl: Workload, layer: int = 0, experts=None) -> LayerInputs:
    s = wl.shape
    wg, wu, wd = layer_weights(s, wl.seed, layer, experts)
    ids, w = routing(wl.T, s.E, s.K, wl.seed, layer, wl.zipf)
    return LayerInputs(wg, wu, wd, rotation_signs(s.H, wl.seed, layer),
                       hidden_states(wl.T, s.H, wl.seed, layer, wl.rmsnorm_x), ids, w)
