"""CPU oracle for the channel-selected routed-expert SwiGLU FFN.

TEST INFRASTRUCTURE ONLY. The oracle is the plain C++17 library built from
oracle/cfm_oracle.cpp (standard library only, float64 throughout); this module
is its ctypes binding: argument marshalling, the per-token bookkeeping of a
batch, and the byte count. Only the tests, the smoke check and the CPU
baseline leg of the benchmark import it; the product path never does. It
shares no code with the HIP path.

The method (arXiv:2610.37386, "Channel Selection for Mixture-of-Experts
Decoding Needs No Calibration Data"; abstract, and the aimodeling.com article
on it, sections "Swapping the threshold for top-k" and "A reader that needs no
data at all"): each routed (token, expert) pair screens its expert's channels
with a rotated ternary sketch of W_gate / W_up, keeps the top-k channels by
exact BF16 activations (top-k, no calibrated threshold), runs the down
projection over those channels only and adds back the skipped channels through
a low-rank map of W_down built from the weights alone. Each function below
names the step it computes; the readings taken where the pages are silent are
stated in oracle/cfm_oracle.cpp at the step.

Notation: E experts, K experts per token, T tokens, H hidden, I intermediate,
k kept channels, c candidates, r recovery rank. Weights are [E][I][H] raw BF16
bits (uint16); the down projection is channel-major (row j = column j of
W_down).

Parity pins: every function is pinned by tests in tests/test_oracle_*.py
against closed forms, independent constructions, library routines or brute
force (none is left unpinned). set_mutation() plants a named mistake in the
C++ oracle so that a test can check that a pin catches it.
"""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cfm_oracle.cpp")
LIB_PATH = os.path.join(_HERE, "libcfm_oracle.so")
CXXFLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = False) -> str:
    """Compile the oracle with g++ into oracle/libcfm_oracle.so (when missing, stale, or forced)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        tmp = LIB_PATH + ".tmp"
        r = subprocess.run(["g++", *CXXFLAGS, _SRC, "-o", tmp], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"g++ failed on {_SRC}:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = ctypes.CDLL(build())

_l, _i, _d, _u64 = ctypes.c_long, ctypes.c_int, ctypes.c_double, ctypes.c_uint64
_P = ctypes.c_void_p
for _name, _res, _args in [
    ("cfo_set_mutation", _i, [ctypes.c_char_p]),
    ("cfo_bf16_to_f64", None, [_l, _P, _P]),
    ("cfo_f64_to_bf16", None, [_l, _P, _P]),
    ("cfo_silu", None, [_l, _P, _P]),
    ("cfo_splitmix64", None, [_u64, _l, _P]),
    ("cfo_rotation_signs", None, [_u64, _l, _P]),
    ("cfo_hadamard", _i, [_l, _P]),
    ("cfo_rotate", _i, [_l, _l, _P, _P, _P]),
    ("cfo_ternarize", None, [_l, _l, _P, _P, _P]),
    ("cfo_sketch_rows", _i, [_l, _l, _P, _P, _P, _P]),
    ("cfo_pack_codes", _i, [_l, _l, _P, _P]),
    ("cfo_unpack_codes", _i, [_l, _l, _P, _P]),
    ("cfo_sketch_build", _i, [_l, _l, _l, _P, _P, _P, _P, _P, _P, _P, _i]),
    ("cfo_lowrank", _i, [_l, _l, _P, _l, _P, _P, _i]),
    ("cfo_topk_set", None, [_l, _P, _l, _P]),
    ("cfo_threshold_set", _l, [_l, _P, _d, _P]),
    ("cfo_calibrate_threshold", _d, [_l, _P, _l, _l]),
    ("cfo_screen_scores", _i, [_l, _l, _P, _P, _P, _P, _P, _P, _P]),
    ("cfo_exact_activations", None, [_l, _l, _P, _P, _P, _P]),
    ("cfo_select_pair", _i, [_l, _l, _l, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _l, _l, _i, _i, _d,
                             _P, _P, _P, _P, _P, _P]),
    ("cfo_combine", None, [_l, _l, _P, _P, _P, _P]),
    ("cfo_select_forward", _i, [_l, _l, _l, _l, _l, _l, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _l, _l, _i, _i, _d, _P, _P, _l, _i, _P, _P, _P, _P, _P, _P, _P]),
    ("cfo_staged_forward", _i, [_l, _l, _l, _l, _l, _l, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P, _l, _P, _l, _P, _i, _P, _P, _l, _i, _P]),
    ("cfo_dense_forward", _i, [_l, _l, _l, _l, _l, _P, _P, _P, _P, _P, _P, _P, _P, _l, _i, _P]),
    ("cfo_rmsnorm", None, [_l, _l, _P, _P, _d, _P]),
    ("cfo_router", None, [_l, _l, _l, _P, _P, _l, _i, _P, _P, _P]),
]:
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _c(a, dtype):
    """A C-contiguous array of the given dtype (a copy only when needed)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    """A pointer argument that keeps its array alive for as long as the pointer object lives (the
    argument tuple of the call), so a converted temporary is not freed before the C code reads it."""
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _ok(rc, what):
    if rc != 0:
        raise ValueError(f"oracle: {what} rejected its arguments")


def set_mutation(name: str = "") -> None:
    """Plant the named mistake in the C++ oracle ('' removes it). Tests only."""
    _lib.cfo_set_mutation(name.encode())


# Default CPU threads of the batch calls (the oracle's arithmetic does not
# depend on it: each pair is computed by one thread, in a fixed order).
THREADS = max(1, min(16, os.cpu_count() or 1))

# ----------------------------------------------------------------------------- numerics helpers


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Raw BF16 bit patterns -> float64 (exact)."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    _lib.cfo_bf16_to_f64(b.size, _p(b), _p(out))
    return out


def as_f64(a: np.ndarray) -> np.ndarray:
    """uint16 arrays are read as raw BF16 bits; anything else as numbers."""
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> raw BF16 bits, rounded once to nearest, ties to even."""
    x = _c(v, np.float64)
    out = np.empty(x.shape, np.uint16)
    _lib.cfo_f64_to_bf16(x.size, _p(x), _p(out))
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^-z), the gate nonlinearity of a SwiGLU expert."""
    x = _c(z, np.float64)
    out = np.empty(x.shape, np.float64)
    _lib.cfo_silu(x.size, _p(x), _p(out))
    return out


# ----------------------------------------------------------------------------- rotation


@functools.lru_cache(maxsize=4)
def hadamard(H: int) -> np.ndarray:
    """Unnormalised Sylvester-Hadamard matrix in natural order, float64 (read-only):
    entry (i, j) is (-1)**popcount(i & j)."""
    out = np.empty((H, H), np.float64)
    _ok(_lib.cfo_hadamard(H, _p(out)), "hadamard (H must be a power of two)")
    out.setflags(write=False)
    return out


def splitmix64(seed: int, n: int) -> list:
    """The first n outputs of SplitMix64 started at `seed`."""
    out = np.empty(n, np.uint64)
    _lib.cfo_splitmix64(seed & (2**64 - 1), n, _p(out))
    return [int(v) for v in out]


def rotation_signs(seed: int, H: int) -> np.ndarray:
    """The layer's rotation signs from a seed: d_i = -1 if bit 63 of SplitMix64's
    i-th output is set, else +1 (int8 [H])."""
    out = np.empty(H, np.int8)
    _lib.cfo_rotation_signs(seed & (2**64 - 1), H, _p(out))
    return out


def rotate(v: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """T(v) = Hadamard (d . v) along the last axis, float64 (fast Walsh-Hadamard)."""
    x = _c(v, np.float64)
    H = x.shape[-1]
    d = _c(signs, np.int8)
    out = np.empty(x.shape, np.float64)
    _ok(_lib.cfo_rotate(x.size // H, H, _p(x), _p(d), _p(out)), "rotate")
    return out


# ----------------------------------------------------------------------------- ternary sketch

TWN_DELTA = 0.7   # threshold factor of Ternary Weight Networks (Li & Liu, 2016), as in the C++ oracle


def ternarize(wt: np.ndarray):
    """Per-row Ternary Weight Networks code and scale of already-rotated rows
    wt [n][H]: (codes int8 [n][H] in {-1, 0, 1}, alpha float64 [n])."""
    x = _c(wt, np.float64)
    H = x.shape[-1]
    codes = np.empty(x.shape, np.int8)
    alpha = np.empty(x.shape[:-1], np.float64)
    _lib.cfo_ternarize(x.size // H, H, _p(x), _p(codes), _p(alpha))
    return codes, alpha


def sketch_rows(w_bits: np.ndarray, signs: np.ndarray):
    """Sketch of BF16 rows w_bits [n][H]: (codes int8 [n][H], scale float32 [n]),
    scale = float32(alpha / H)."""
    w = _c(w_bits, np.uint16)
    H = w.shape[-1]
    codes = np.empty(w.shape, np.int8)
    scale = np.empty(w.shape[:-1], np.float32)
    _ok(_lib.cfo_sketch_rows(w.size // H, H, _p(w), _p(_c(signs, np.int8)), _p(codes), _p(scale)), "sketch_rows")
    return codes, scale


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Ternary codes [n][H] -> 2 bits per value, uint8 [n][H/4] (layout in cfm_oracle.cpp)."""
    c = _c(codes, np.int8)
    n, H = c.shape
    out = np.empty((n, H // 4), np.uint8)
    _ok(_lib.cfo_pack_codes(n, H, _p(c), _p(out)), "pack_codes (H must be a multiple of 16)")
    return out


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_codes: uint8 [n][H/4] -> int8 [n][H]."""
    pk = _c(packed, np.uint8)
    n, hb = pk.shape
    out = np.empty((n, 4 * hb), np.int8)
    _ok(_lib.cfo_unpack_codes(n, 4 * hb, _p(pk), _p(out)), "unpack_codes")
    return out


def sketch_build(w_gate: np.ndarray, w_up: np.ndarray, signs: np.ndarray):
    """Sketch of every expert's gate and up rows ([E][I][H] BF16 bits each):
    (tg, tu uint8 [E][I][H/4], sg, su float32 [E][I])."""
    wg, wu = _c(w_gate, np.uint16), _c(w_up, np.uint16)
    E, I, H = wg.shape
    tg, tu = np.empty((E, I, H // 4), np.uint8), np.empty((E, I, H // 4), np.uint8)
    sg, su = np.empty((E, I), np.float32), np.empty((E, I), np.float32)
    _ok(_lib.cfo_sketch_build(E, I, H, _p(wg), _p(wu), _p(_c(signs, np.int8)), _p(tg), _p(tu), _p(sg), _p(su),
                              THREADS), "sketch_build")
    return tg, tu, sg, su


# ----------------------------------------------------------------------------- low-rank map


def lowrank(w_down_t_bits: np.ndarray, r: int):
    """Rank-r map of one expert's down projection (BF16 bits or floats [I][H]),
    float64: A = U_r diag(s_r) [H][r], Bt = V_r [I][r] of W_down's SVD (one-sided
    Jacobi), each column of V_r signed so its largest-magnitude entry is positive."""
    wdt = _c(as_f64(w_down_t_bits), np.float64)
    I, H = wdt.shape
    if not 0 <= r <= min(H, I):
        raise ValueError("rank out of range")
    A, Bt = np.zeros((H, r)), np.zeros((I, r))
    _ok(_lib.cfo_lowrank(I, H, _p(wdt), r, _p(A), _p(Bt), THREADS), "lowrank")
    return A, Bt


def lowrank_build(w_down_t: np.ndarray, r: int):
    """Every expert's map, stored as BF16 bits: (A [E][H][r], Bt [E][I][r])."""
    As, Bs = [], []
    for e in range(w_down_t.shape[0]):
        A, Bt = lowrank(w_down_t[e], r)
        As.append(f64_to_bf16(A))
        Bs.append(f64_to_bf16(Bt))
    return np.stack(As), np.stack(Bs)


# ----------------------------------------------------------------------------- selection


def topk_set(scores: np.ndarray, k: int) -> np.ndarray:
    """The k largest scores by (score desc, index asc), NaN as 0; ascending indices."""
    s = _c(scores, np.float64).reshape(-1)
    k = max(0, min(int(k), s.size))
    out = np.empty(k, np.int64)
    _lib.cfo_topk_set(s.size, _p(s), k, _p(out))
    return out


def threshold_set(scores: np.ndarray, tau: float) -> np.ndarray:
    """{j : s_j >= tau}, ascending (NaN as 0): the keep rule that top-k replaces."""
    s = _c(scores, np.float64).reshape(-1)
    out = np.empty(s.size, np.int64)
    n = _lib.cfo_threshold_set(s.size, _p(s), float(tau), _p(out))
    return out[:n].copy()


def calibrate_threshold(score_sets, k: int) -> float:
    """One threshold per layer for a mean budget of k over n calibration pairs:
    the (k n)-th largest pooled score (+inf when k n = 0)."""
    pooled = np.concatenate([_c(s, np.float64).reshape(-1) for s in score_sets]) if len(score_sets) else np.zeros(0)
    pooled = _c(pooled, np.float64)
    v = _lib.cfo_calibrate_threshold(pooled.size, _p(pooled), len(score_sets), int(k))
    if np.isnan(v):
        raise ValueError("budget above the number of calibration scores")
    return float(v)


def screen_scores(x_bits, tg_rows, tu_rows, sg_rows, su_rows, signs):
    """Sketch activations hhat [I] of one expert's channels for one token."""
    tg, tu = _c(tg_rows, np.uint8), _c(tu_rows, np.uint8)
    I, hb = tg.shape
    out = np.empty(I, np.float64)
    _ok(_lib.cfo_screen_scores(I, 4 * hb, _p(_c(x_bits, np.uint16)), _p(tg), _p(tu), _p(_c(sg_rows, np.float32)),
                               _p(_c(su_rows, np.float32)), _p(_c(signs, np.int8)), _p(out)), "screen_scores")
    return out


def exact_activations(x_bits, wg_rows_bits, wu_rows_bits):
    """h_j = SiLU(Wg_j . x) (Wu_j . x) from the native BF16 rows, float64."""
    wg, wu = _c(wg_rows_bits, np.uint16), _c(wu_rows_bits, np.uint16)
    I, H = wg.shape
    out = np.empty(I, np.float64)
    _lib.cfo_exact_activations(I, H, _p(_c(x_bits, np.uint16)), _p(wg), _p(wu), _p(out))
    return out


RECOVERY_SKETCH = "sketch"
RECOVERY_CANDIDATES_EXACT = "candidates_exact"
_RECOVERY = {RECOVERY_SKETCH: 0, RECOVERY_CANDIDATES_EXACT: 1}


def _map_values(A, Bt, r):
    if r == 0:
        return None, None
    return _c(as_f64(A), np.float64), _c(as_f64(Bt), np.float64)


def select_pair(x_bits, e, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c,
                recovery=RECOVERY_SKETCH, tau=None):
    """The method for one routed (token, expert) pair: screen, C = top-c by
    |hhat|, exact h on C, S = top-k of C by |h| (or, with tau, the threshold
    rule on the same score), y = sum_{j in S} h_j Wd_t[j] + A z with
    z = sum_{j not in S} a_j Bt[j] (a_j = hhat_j; with recovery=
    "candidates_exact", h_j for the candidates screened in but not kept).

    A [E][H][r], Bt [E][I][r]: the stored map (BF16 bits, or floats).
    Returns a dict with hhat [I], C, h_all [I] (exact, every channel), S, y [H]."""
    if recovery not in _RECOVERY:
        raise ValueError(f"unknown recovery variant {recovery!r}")
    E, I, H = np.shape(w_gate)
    r = np.shape(A)[-1]
    Ae, Bte = _map_values(np.asarray(A)[e], np.asarray(Bt)[e], r)
    hhat, h_all, y = np.empty(I), np.empty(I), np.empty(H)
    C, S = np.empty(max(c, 1), np.int64), np.empty(max(c, 1), np.int64)
    nS = ctypes.c_long(0)
    rc = _lib.cfo_select_pair(
        I, H, r, _p(_c(x_bits, np.uint16)), _p(_c(w_gate[e], np.uint16)), _p(_c(w_up[e], np.uint16)),
        _p(_c(w_down_t[e], np.uint16)), _p(_c(tg[e], np.uint8)), _p(_c(tu[e], np.uint8)), _p(_c(sg[e], np.float32)),
        _p(_c(su[e], np.float32)), _p(_c(signs, np.int8)), _p(Ae), _p(Bte), int(k), int(c), _RECOVERY[recovery],
        0 if tau is None else 1, 0.0 if tau is None else float(tau), _p(hhat), _p(C), _p(h_all), _p(S),
        ctypes.byref(nS), _p(y))
    _ok(rc, "select_pair")
    return {"hhat": hhat, "C": C[:c].copy(), "h_all": h_all, "S": S[:nS.value].copy(), "y": y}


def combine(ys: np.ndarray, w: np.ndarray, resid=None) -> np.ndarray:
    """out = BF16( resid + sum_q w_q y_q ) over a token's K experts, one rounding
    (router weights used as given)."""
    ys = _c(ys, np.float64)
    K, H = ys.shape
    out = np.empty(H, np.uint16)
    _lib.cfo_combine(K, H, _p(ys), _p(_c(w, np.float64)), _p(None if resid is None else _c(resid, np.uint16)),
                     _p(out))
    return out


def select_forward(x, ids, w, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c,
                   tokens=None, recovery=RECOVERY_SKETCH, resid=None, tau=None, threads=None, details=True):
    """Selected-channel MoE layer over a decode batch (selection per (token,
    expert) pair, independent of the batch). x [T][H] BF16 bits, ids [T][K],
    w [T][K]; tokens: optional subset to evaluate; resid: optional BF16 bits
    [T][H] added before each token's single rounding.

    Returns (out BF16 bits [len(tokens)][H], {(t, q): select_pair dict}); the
    dict is empty with details=False."""
    if recovery not in _RECOVERY:
        raise ValueError(f"unknown recovery variant {recovery!r}")
    ids = _c(ids, np.int32)
    T, K = ids.shape
    E, I, H = np.shape(w_gate)
    r = np.shape(A)[-1]
    tok = np.arange(T, dtype=np.int64) if tokens is None else _c(list(tokens), np.int64)
    n, P = tok.size, tok.size * K
    out = np.empty((n, H), np.uint16)
    Af, Btf = _map_values(A, Bt, r)
    cc = max(c, 1)
    hhat = np.empty((P, I)) if details else None
    h_all = np.empty((P, I)) if details else None
    C = np.empty((P, cc), np.int64) if details else None
    S = np.empty((P, cc), np.int64) if details else None
    nS = np.empty(P, np.int64) if details else None
    y = np.empty((P, H)) if details else None
    rc = _lib.cfo_select_forward(
        T, K, E, I, H, r, _p(_c(x, np.uint16)), _p(ids), _p(_c(w, np.float64)), _p(_c(w_gate, np.uint16)),
        _p(_c(w_up, np.uint16)), _p(_c(w_down_t, np.uint16)), _p(_c(tg, np.uint8)), _p(_c(tu, np.uint8)),
        _p(_c(sg, np.float32)), _p(_c(su, np.float32)), _p(_c(signs, np.int8)), _p(Af), _p(Btf), int(k), int(c),
        _RECOVERY[recovery], 0 if tau is None else 1, 0.0 if tau is None else float(tau),
        _p(None if resid is None else _c(resid, np.uint16)), _p(tok), n, THREADS if threads is None else int(threads),
        _p(out), _p(hhat), _p(C), _p(h_all), _p(S), _p(nS), _p(y))
    _ok(rc, "select_forward")
    pairs = {}
    if details:
        for m, t in enumerate(tok):
            for q in range(K):
                pn = m * K + q
                pairs[(int(t), q)] = {"hhat": hhat[pn], "C": C[pn, :c].copy(), "h_all": h_all[pn],
                                      "S": S[pn, :nS[pn]].copy(), "y": y[pn]}
    return out, pairs


def staged_forward(x, ids, w, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, cand_sets, keep_sets, tokens,
                   recovery=RECOVERY_SKETCH, resid=None, threads=None):
    """The layer's outputs for `tokens` with the candidate and kept sets given
    ({(t, q): ascending index array}) instead of selected: the oracle's own
    activations, down projection and recovery applied to another selection
    (one that differs from the oracle's by near-ties). BF16 bits [len][H]."""
    if recovery not in _RECOVERY:
        raise ValueError(f"unknown recovery variant {recovery!r}")
    ids = _c(ids, np.int32)
    T, K = ids.shape
    E, I, H = np.shape(w_gate)
    r = np.shape(A)[-1]
    tok = _c(list(tokens), np.int64)
    P = tok.size * K
    c = max(len(cand_sets[(int(tok[0]), 0)]), 1) if P else 1
    smax = max([len(keep_sets[(int(t), q)]) for t in tok for q in range(K)] + [1])
    C = np.zeros((P, c), np.int64)
    S = np.zeros((P, smax), np.int64)
    nS = np.zeros(P, np.int64)
    for m, t in enumerate(tok):
        for q in range(K):
            cs, ks = np.asarray(cand_sets[(int(t), q)]), np.asarray(keep_sets[(int(t), q)])
            C[m * K + q, :cs.size] = cs
            S[m * K + q, :ks.size] = ks
            nS[m * K + q] = ks.size
    Af, Btf = _map_values(A, Bt, r)
    out = np.empty((tok.size, H), np.uint16)
    rc = _lib.cfo_staged_forward(
        T, K, E, I, H, r, _p(_c(x, np.uint16)), _p(ids), _p(_c(w, np.float64)), _p(_c(w_gate, np.uint16)),
        _p(_c(w_up, np.uint16)), _p(_c(w_down_t, np.uint16)), _p(_c(tg, np.uint8)), _p(_c(tu, np.uint8)),
        _p(_c(sg, np.float32)), _p(_c(su, np.float32)), _p(_c(signs, np.int8)), _p(Af), _p(Btf), _p(C), c, _p(S),
        smax, _p(nS), _RECOVERY[recovery], _p(None if resid is None else _c(resid, np.uint16)), _p(tok), tok.size,
        THREADS if threads is None else int(threads), _p(out))
    _ok(rc, "staged_forward")
    return out


def dense_forward(x, ids, w, w_gate, w_up, w_down_t, tokens=None, resid=None, threads=None):
    """The same layer with every channel read: y = sum_j h_j Wd_t[j] (ascending j)."""
    ids = _c(ids, np.int32)
    T, K = ids.shape
    E, I, H = np.shape(w_gate)
    tok = np.arange(T, dtype=np.int64) if tokens is None else _c(list(tokens), np.int64)
    out = np.empty((tok.size, H), np.uint16)
    rc = _lib.cfo_dense_forward(
        T, K, E, I, H, _p(_c(x, np.uint16)), _p(ids), _p(_c(w, np.float64)), _p(_c(w_gate, np.uint16)),
        _p(_c(w_up, np.uint16)), _p(_c(w_down_t, np.uint16)), _p(None if resid is None else _c(resid, np.uint16)),
        _p(tok), tok.size, THREADS if threads is None else int(threads), _p(out))
    _ok(rc, "dense_forward")
    return out


# ----------------------------------------------------------------------------- decode-layer envelope


def rmsnorm(h_bits, gamma_bits, eps: float):
    """x = BF16( h / sqrt(mean(h^2) + eps) * gamma ), per token, one rounding."""
    h = _c(h_bits, np.uint16)
    H = h.shape[-1]
    out = np.empty(h.shape, np.uint16)
    _lib.cfo_rmsnorm(h.size // H, H, _p(h), _p(_c(gamma_bits, np.uint16)), float(eps), _p(out))
    return out


def router(x_bits, w_router_bits, K: int, renorm: bool):
    """Top-K softmax routing of BF16 states x [T][H] with router rows W_r [E][H]:
    (ids int32 [T][K] in descending probability, lower id first on ties;
    weights float64 [T][K]; logits float64 [T][E])."""
    x = _c(x_bits, np.uint16)
    x2 = x.reshape(-1, x.shape[-1])
    wr = _c(as_f64(w_router_bits), np.float64)
    E, H = wr.shape
    T = x2.shape[0]
    ids, w, logits = np.empty((T, K), np.int32), np.empty((T, K)), np.empty((T, E))
    _lib.cfo_router(T, H, E, _p(x2), _p(wr), int(K), 1 if renorm else 0, _p(ids), _p(w), _p(logits))
    return ids, w, logits


def layer_forward(h, gamma, eps, w_router, K, renorm, w_gate, w_up, w_down_t, tg=None, tu=None, sg=None,
                  su=None, signs=None, A=None, Bt=None, k=0, c=0, recovery=RECOVERY_SKETCH, dense=False,
                  x=None, ids=None, w=None, tokens=None):
    """One decode layer's routed-expert block with its envelope:
    out = BF16(h + sum_q w_q y_(t,q)) with x = rmsnorm(h), (ids, w) = router(x).

    dense=True runs the dense block. x, ids, w: optional overrides (e.g. the
    values a device computed), so that later steps can be checked on the same
    selections. Returns (out BF16 bits, x, ids, w, per-pair details or None)."""
    xs = rmsnorm(h, gamma, eps) if x is None else x
    if ids is None or w is None:
        ids_r, w_r, _ = router(xs, w_router, K, renorm)
        ids = ids_r if ids is None else ids
        w = w_r if w is None else w
    if dense:
        out = dense_forward(xs, ids, w, w_gate, w_up, w_down_t, tokens=tokens, resid=h)
        return out, xs, ids, w, None
    out, pairs = select_forward(xs, ids, w, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c,
                                tokens=tokens, recovery=recovery, resid=h)
    return out, xs, ids, w, pairs


# ----------------------------------------------------------------------------- byte accounting


def read_bytes(ids, E, I, H, k, c, r, cand_sets=None, keep_sets=None, recovery=RECOVERY_SKETCH,
               threshold=False):
    """Bytes the method must read for one layer call (algorithmic count).

    Reads are counted the way hardware bills them: a touched segment is paid
    in full (article section "Calibrated thresholds do not pin down how much
    you read"). Every row below is a whole number of 128-byte segments, so the
    count is the byte size of: per routed expert, its sketch (I·H/4 per
    matrix) and scales (4·I per matrix), its map (2·H·r + 2·I·r), the BF16
    gate and up rows of the union of its pairs' candidates (2·2·H per row) and
    the down rows of the union of kept channels (2·H per row); plus the hidden
    states (2·T·H) and router output (8·T·K) and the BF16 result (2·T·H).

    cand_sets/keep_sets: {(t, q): index array}; when absent the sets are taken
    as disjoint per pair (c and k rows each). The candidates' gate and up rows
    are read only when their exact activations are used: to rank them for the
    kept set (k > 0) or, in the candidates_exact recovery variant, as the
    dropped candidates' recovery coefficients. With the variant and c = I
    every channel is a candidate, so no sketch activation enters the result
    and the sketch is not read. threshold: the kept sets come from the
    threshold keep rule (keep_sets must be given; k is not used).
    """
    if threshold and keep_sets is None:
        raise ValueError("the threshold keep rule needs the kept sets")
    exact_step = k > 0 or threshold or recovery == RECOVERY_CANDIDATES_EXACT
    sketch_read = not (recovery == RECOVERY_CANDIDATES_EXACT and c >= I)
    T, K = ids.shape
    total = 0
    for e in sorted(set(int(v) for v in ids.reshape(-1))):
        pairs = [(t, q) for t in range(T) for q in range(K) if ids[t, q] == e]
        nc = c * len(pairs) if cand_sets is None else \
            len(set().union(*[set(map(int, cand_sets[p])) for p in pairs]))
        nk = k * len(pairs) if keep_sets is None else \
            len(set().union(*[set(map(int, keep_sets[p])) for p in pairs]))
        if not exact_step:
            nc = 0
        sketch = 2 * (I * H // 4) + 2 * 4 * I if sketch_read else 0
        total += sketch + 2 * H * r + 2 * I * r + 4 * H * nc + 2 * H * nk
    return total + 2 * T * H + 8 * T * K + 2 * T * H


def dense_bytes(ids, E, I, H):
    T, K = ids.shape
    used = len(set(int(v) for v in ids.reshape(-1)))
    return used * 6 * I * H + 2 * T * H + 8 * T * K + 2 * T * H
