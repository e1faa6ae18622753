"""CPU oracle for the channel-selected routed-expert SwiGLU FFN (float64).

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference that the
HIP library is checked against. Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path never does. It
shares no code with the HIP path: it has its own transform, sketch, packing,
selection, low-rank map and combine, written from the method's description.

The method (arXiv:2610.37386, "Channel Selection for Mixture-of-Experts
Decoding Needs No Calibration Data"; abstract, and the aimodeling.com article
on it, section "A reader that needs no data at all"):
  * small-batch MoE decoding is bound by loading routed-expert weights, and
    most intermediate channels of a routed expert contribute little to a
    given token, so a selector predicts the channels that matter and reads
    only their weights (abstract);
  * the keep rule is top-k per token, with no calibrated threshold
    (abstract; article section "Swapping the threshold for top-k");
  * each expert keeps a rotated ternary sketch of its gate and up projections,
    resident on the GPU, used to screen candidate channels; the kept top-k is
    then computed exactly from the native BF16 weights; the skipped channels
    are recovered through a low-rank map of the down projection; nothing uses
    calibration data (article section "A reader that needs no data at all").

The pages give no formulas. Every step below states the plain reading taken
where they are silent; the readings are listed together in the design notes.

Notation: E experts, K experts per token, T tokens, H hidden, I intermediate,
k kept channels, c candidates, r recovery rank. Weights are [E][I][H]; the
down projection is passed channel-major (row j = column j of W_down).

Parity pins: every function here is pinned by tests in tests/test_oracle_*.py
against closed forms, independent constructions, library routines or brute
force (no function is left unpinned).
"""
from __future__ import annotations

import functools

import numpy as np

# ----------------------------------------------------------------------------- numerics helpers


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Raw BF16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    """uint16 arrays are read as raw BF16 bits; anything else as numbers."""
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> raw BF16 bits, rounded once to nearest, ties to even.

    Written from the format: 8 significant bits, 8 exponent bits, subnormal
    spacing 2**-133 below 2**-126, overflow to infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x8000, 0).astype(np.uint32)
    a = np.abs(v)
    _, e = np.frexp(a)                         # a = m * 2**e with 0.5 <= m < 1
    e = np.maximum(e, -125)                    # below 2**-126 the spacing stays 2**-133
    q = np.rint(np.ldexp(a, 8 - e))            # significand in units of the BF16 spacing, ties even
    val = np.ldexp(q, e - 8)                   # a BF16 value (or 2**128 on overflow)
    with np.errstate(over="ignore"):
        bits32 = val.astype(np.float32).view(np.uint32)
    out = ((bits32 >> 16) | sign).astype(np.uint16)
    out[np.isnan(v)] = 0x7FC0
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^-z), the gate nonlinearity of a SwiGLU expert."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------- rotation


@functools.lru_cache(maxsize=4)
def hadamard(H: int) -> np.ndarray:
    """Unnormalised Sylvester-Hadamard matrix in natural order, float64 (read-only).

    Entry (i, j) is (-1)**popcount(i & j). It is symmetric and H·H = H·Id.
    """
    if H <= 0 or H & (H - 1):
        raise ValueError("H must be a power of two")
    i = np.arange(H, dtype=np.int64)
    par = np.bitwise_count(np.bitwise_and.outer(i, i)) & 1
    m = np.where(par == 0, 1.0, -1.0)
    m.setflags(write=False)
    return m


_M64 = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> list:
    """The first n outputs of SplitMix64 started at `seed` (Steele, Lea and Flood,
    "Fast splittable pseudorandom number generators", OOPSLA 2014): the state
    advances by the 64-bit golden-ratio increment, and each output is the new
    state passed through two xor-shift-multiply rounds and a final xor-shift
    (all arithmetic mod 2^64)."""
    out, state = [], seed & _M64
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        out.append(z ^ (z >> 31))
    return out


def rotation_signs(seed: int, H: int) -> np.ndarray:
    """The layer's random signs d of the rotation, from a seed (article section
    "A reader that needs no data at all": the sketch is rotated; the pages do
    not say how the rotation is drawn). Reading: d_i = -1 if bit 63 of
    SplitMix64's i-th output is set, else +1. int8 [H]."""
    return np.array([-1 if (z >> 63) & 1 else 1 for z in splitmix64(seed, H)], dtype=np.int8)


def rotate(v: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """T(v) = Hadamard · (d ⊙ v) along the last axis, float64.

    The sketch is "rotated" (article section "A reader that needs no data at
    all"); the reading taken is a random-sign Walsh-Hadamard rotation, one
    sign vector d per layer shared by the gate rows, the up rows and the
    hidden state. The orthonormal rotation would carry a factor 1/sqrt(H) on
    each side; here both are folded into the sketch scale, so that
    w·x = T(w)·T(x) / H exactly.
    """
    v = np.asarray(v, dtype=np.float64)
    d = np.asarray(signs, dtype=np.float64)
    return (v * d) @ hadamard(v.shape[-1])


# ----------------------------------------------------------------------------- ternary sketch

TWN_DELTA = 0.7   # threshold factor of Ternary Weight Networks (Li & Liu, 2016)


def ternarize(wt: np.ndarray):
    """Per-row ternary code and scale of already-rotated rows wt [n][H].

    Reading of "ternary sketch" (article section "A reader that needs no data
    at all"): the Ternary Weight Networks rule. Threshold
    delta = 0.7 * mean_i |wt_i|; t_i = +1 if wt_i > delta, -1 if
    wt_i < -delta, else 0 (a value exactly at the threshold gives 0); scale
    alpha = mean of |wt_i| over the nonzero t_i (alpha = 0 if none), the
    least-squares scale for that pattern.

    Returns (codes int8 [n][H] in {-1,0,1}, alpha float64 [n]).
    """
    wt = np.asarray(wt, dtype=np.float64)
    H = wt.shape[-1]
    a = np.abs(wt)
    mean_abs = np.sum(a, axis=-1) / H
    delta = TWN_DELTA * mean_abs
    codes = np.zeros(wt.shape, np.int8)
    codes[wt > delta[..., None]] = 1
    codes[wt < -delta[..., None]] = -1
    nz = codes != 0
    n = np.sum(nz, axis=-1)
    s2 = np.sum(np.where(nz, a, 0.0), axis=-1)
    alpha = np.where(n > 0, s2 / np.maximum(n, 1), 0.0)
    return codes, alpha


def sketch_rows(w_bits: np.ndarray, signs: np.ndarray):
    """Sketch of BF16 rows w_bits [n][H] (raw bits).

    Returns (codes int8 [n][H], scale float32 [n]) where the stored scale is
    alpha / H rounded to float32 (nearest, ties even): the 1/H undoes the
    unnormalised transform, so scale * (t · T(x)) estimates w · x.
    """
    codes, alpha = ternarize(rotate(bf16_to_f64(w_bits), signs))
    H = codes.shape[-1]
    return codes, (alpha / H).astype(np.float32)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack ternary codes [n][H] into 2 bits per value -> uint8 [n][H/4].

    Format (a reading: the pages say only that the sketch is ternary). Each
    value has two flag bits, nz = (t != 0) and neg = (t < 0). A row is cut
    into 16-value groups; group b becomes one little-endian 32-bit word
    (bytes 4b..4b+3 of the row). Value 16b+q (q < 8) and value 16b+8+q share
    nibble q of that word:
        bit 4q+0 = nz(t[16b+8+q])   bit 4q+1 = nz(t[16b+q])
        bit 4q+2 = neg(t[16b+8+q])  bit 4q+3 = neg(t[16b+q])
    """
    codes = np.asarray(codes)
    n, H = codes.shape
    if H % 16:
        raise ValueError("H must be a multiple of 16")
    g = codes.reshape(n, H // 16, 16)
    nz = (g != 0).astype(np.uint32)
    neg = (g < 0).astype(np.uint32)
    word = np.zeros((n, H // 16), np.uint32)
    for q in range(8):
        word |= nz[:, :, 8 + q] << np.uint32(4 * q + 0)
        word |= nz[:, :, q] << np.uint32(4 * q + 1)
        word |= neg[:, :, 8 + q] << np.uint32(4 * q + 2)
        word |= neg[:, :, q] << np.uint32(4 * q + 3)
    return word.astype("<u4").view(np.uint8).reshape(n, H // 4)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_codes: uint8 [n][H/4] -> int8 [n][H]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n, hb = packed.shape
    word = packed.reshape(n, hb // 4, 4).copy().view("<u4").reshape(n, hb // 4).astype(np.uint32)
    out = np.zeros((n, hb // 4, 16), np.int8)
    for q in range(8):
        for half, (bnz, bneg) in ((0, (4 * q + 1, 4 * q + 3)), (8, (4 * q + 0, 4 * q + 2))):
            nzb = (word >> np.uint32(bnz)) & 1
            ngb = (word >> np.uint32(bneg)) & 1
            out[:, :, half + q] = np.where(nzb == 1, np.where(ngb == 1, -1, 1), 0)
    return out.reshape(n, hb * 4)


def sketch_build(w_gate: np.ndarray, w_up: np.ndarray, signs: np.ndarray):
    """Sketch of every expert's gate and up rows ([E][I][H] BF16 bits each).

    Returns (tg, tu uint8 [E][I][H/4], sg, su float32 [E][I]).
    """
    E, I, H = w_gate.shape
    out = []
    for w in (w_gate, w_up):
        codes, scale = sketch_rows(w.reshape(E * I, H), signs)
        out.append((pack_codes(codes).reshape(E, I, H // 4), scale.reshape(E, I)))
    (tg, sg), (tu, su) = out
    return tg, tu, sg, su


# ----------------------------------------------------------------------------- low-rank map


def lowrank(w_down_t_bits: np.ndarray, r: int):
    """Rank-r map of one expert's down projection (BF16 bits or floats), float64.

    "The skipped channels are recovered through a low-rank map of the down
    projections", built from weights only (article section "A reader that
    needs no data at all"). Reading: the truncated SVD of W_down (H x I),
    W_down ~ A·B with A = U_r·diag(s_r) [H][r] and B = V_r^T; B is returned
    transposed as Bt = V_r [I][r]. Each column of V_r gets the sign that makes
    its largest-magnitude entry positive (lowest index on ties); A·B does not
    depend on this choice.
    """
    wd = as_f64(w_down_t_bits).T                 # W_down, H x I
    H, I = wd.shape
    if not 0 <= r <= min(H, I):
        raise ValueError("rank out of range")
    U, s, Vt = np.linalg.svd(wd, full_matrices=False)
    A = U[:, :r] * s[:r]
    Bt = Vt[:r].T.copy()
    for l in range(r):
        j = int(np.argmax(np.abs(Bt[:, l])))
        if Bt[j, l] < 0:
            Bt[:, l] = -Bt[:, l]
            A[:, l] = -A[:, l]
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
    """The k largest scores by (score descending, index ascending).

    Top-k keeps each token's k highest-scoring channels (abstract). Ties go to
    the lower index; NaN counts as 0. Returned as ascending indices.
    """
    s = np.nan_to_num(np.asarray(scores, dtype=np.float64), nan=0.0)
    order = np.lexsort((np.arange(s.size), -s))
    return np.sort(order[:k])


def threshold_set(scores: np.ndarray, tau: float) -> np.ndarray:
    """The indices whose score reaches tau, {j : s_j >= tau}, ascending.

    The keep rule that top-k replaces: a selector keeps the channels whose
    score passes a threshold fixed offline, so how many it keeps, and reads,
    depends on the input (abstract; article section "Calibrated thresholds do
    not pin down how much you read"). NaN counts as 0, as in topk_set.
    """
    s = np.nan_to_num(np.asarray(scores, dtype=np.float64), nan=0.0)
    return np.flatnonzero(s >= tau)


def calibrate_threshold(score_sets, k: int) -> float:
    """The threshold that keeps k channels per pair on average over calibration pairs.

    The offline step a threshold selector needs (abstract: thresholds
    calibrated for a read budget). Plain reading: one threshold per layer,
    matched to the budget's mean, i.e. the (k n)-th largest of the pooled
    scores of the n calibration pairs, so that exactly k n of them reach it
    when they are distinct (more on ties). k = 0 gives +inf (nothing passes).
    """
    pooled = np.concatenate([np.nan_to_num(np.asarray(s, np.float64), nan=0.0) for s in score_sets]) \
        if len(score_sets) else np.zeros(0)
    m = k * len(score_sets)
    if m <= 0:
        return float("inf")
    if m > pooled.size:
        raise ValueError("budget above the number of calibration scores")
    return float(np.sort(pooled)[::-1][m - 1])


def screen_scores(x_bits, tg_rows, tu_rows, sg_rows, su_rows, signs):
    """Sketch activations of every channel of one expert for one token.

    ghat_j = sg_j * (t^g_j · T(x)), uhat_j likewise, hhat_j = SiLU(ghat_j)·uhat_j
    (the SwiGLU coefficient the sketch predicts for channel j). The screen
    score of channel j is |hhat_j|.
    """
    xt = rotate(bf16_to_f64(x_bits), signs)
    tg = unpack_codes(tg_rows).astype(np.float64)
    tu = unpack_codes(tu_rows).astype(np.float64)
    ghat = sg_rows.astype(np.float64) * (tg @ xt)
    uhat = su_rows.astype(np.float64) * (tu @ xt)
    return silu(ghat) * uhat


def exact_activations(x_bits, wg_rows_bits, wu_rows_bits):
    """h_j = SiLU(Wg_j · x) * (Wu_j · x) from the native BF16 rows, float64."""
    x = bf16_to_f64(x_bits)
    g = bf16_to_f64(wg_rows_bits) @ x
    u = bf16_to_f64(wu_rows_bits) @ x
    return silu(g) * u


RECOVERY_SKETCH = "sketch"
RECOVERY_CANDIDATES_EXACT = "candidates_exact"


def select_pair(x_bits, e, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c,
                recovery=RECOVERY_SKETCH, tau=None):
    """The method for one routed (token, expert) pair.

    1. screen: hhat for all channels from the sketch; C = top-c by |hhat|
       (candidate screen, article section "A reader that needs no data at all");
    2. exact: h_j for j in C from the BF16 gate/up rows; S = top-k of C by |h_j|
       ("the top-k is computed exactly from the native BF16 weights");
    3. down over kept: y = sum_{j in S} h_j · Wd_t[j] (read only the kept
       channels' weights, abstract);
    4. recovery: z = sum_{j not in S} a_j · Bt[j]; y += A · z ("skipped
       channels are recovered through a low-rank map"). The coefficient a_j of
       a skipped channel is its sketch activation hhat_j (the default reading:
       every skipped channel, including candidates screened in but not kept).
       recovery="candidates_exact" is the variant that gives the candidates
       screened in but not kept their exact h_j instead (they were computed
       for the top-k anyway); channels never screened in keep hhat_j.

    tau: when given, step 2 uses the threshold keep rule on the same score in
    place of top-k, S = {j in C : |h_j| >= tau} (threshold_set), and k is not
    used; |S| then varies with the input.

    A [E][H][r], Bt [E][I][r] are the stored map (BF16 bits, or floats).
    Returns a dict with hhat [I], C, h_all [I] (exact, every channel), S, y [H].
    """
    if recovery not in (RECOVERY_SKETCH, RECOVERY_CANDIDATES_EXACT):
        raise ValueError(f"unknown recovery variant {recovery!r}")
    I = w_gate.shape[1]
    hhat = screen_scores(x_bits, tg[e], tu[e], sg[e], su[e], signs)
    C = topk_set(np.abs(hhat), c)
    h_all = exact_activations(x_bits, w_gate[e], w_up[e])   # the scores the kernel needs only on C
    if tau is None:
        S = C[topk_set(np.abs(h_all[C]), k)] if k > 0 else np.zeros(0, np.int64)
    else:
        S = C[threshold_set(np.abs(h_all[C]), tau)]
    wd = bf16_to_f64(w_down_t[e])
    y = h_all[S] @ wd[S] if len(S) > 0 else np.zeros(wd.shape[1])
    r = A.shape[-1]
    if r > 0:
        coef = hhat.copy()
        if recovery == RECOVERY_CANDIDATES_EXACT:
            coef[C] = h_all[C]
        skip = np.ones(I, bool)
        skip[S] = False
        z = as_f64(Bt[e])[skip].T @ coef[skip]
        y = y + as_f64(A[e]) @ z
    return {"hhat": hhat, "C": C, "h_all": h_all, "S": S, "y": y}


def combine(ys: np.ndarray, w: np.ndarray, resid=None) -> np.ndarray:
    """out = resid + sum_q w_q · y_q over a token's K routed experts, as BF16 bits.

    Router weights are used as given (never renormalised); the sum is in
    float64 and rounded once to BF16. resid: optional BF16 bits [H] (the
    residual stream the decode layer adds the block's output to).
    """
    acc = np.tensordot(np.asarray(w, np.float64), ys, axes=(0, 0))
    if resid is not None:
        acc = acc + bf16_to_f64(resid)
    return f64_to_bf16(acc)


def select_forward(x, ids, w, w_gate, w_up, w_down_t, tg, tu, sg, su, signs, A, Bt, k, c,
                   tokens=None, recovery=RECOVERY_SKETCH, resid=None, tau=None):
    """Selected-channel MoE layer over a decode batch.

    x [T][H] BF16 bits, ids [T][K], w [T][K]. Selection is per (token, expert)
    pair and does not depend on the rest of the batch ("each token's k
    highest-scoring channels", abstract). tokens: optional subset of token
    indices to evaluate (the others are skipped). recovery, tau: as in
    select_pair.
    resid: optional BF16 bits [T][H] added to each token's output before its
    single rounding (see combine).

    Returns (out BF16 bits [len(tokens)][H], per-pair details
    {(t, q): select_pair dict}).
    """
    T, K = ids.shape
    H = w_gate.shape[2]
    tok = range(T) if tokens is None else tokens
    outs, pairs = [], {}
    for t in tok:
        ys = np.zeros((K, H))
        for q in range(K):
            d = select_pair(x[t], int(ids[t, q]), w_gate, w_up, w_down_t, tg, tu, sg, su, signs,
                            A, Bt, k, c, recovery=recovery, tau=tau)
            pairs[(t, q)] = d
            ys[q] = d["y"]
        outs.append(combine(ys, w[t], None if resid is None else resid[t]))
    return (np.stack(outs) if outs else np.zeros((0, H), np.uint16)), pairs


def dense_forward(x, ids, w, w_gate, w_up, w_down_t, tokens=None, resid=None):
    """The same layer with every channel read: y = sum_j h_j · Wd_t[j]."""
    T, K = ids.shape
    H = w_gate.shape[2]
    tok = range(T) if tokens is None else tokens
    outs = []
    for t in tok:
        ys = np.zeros((K, H))
        for q in range(K):
            e = int(ids[t, q])
            h = exact_activations(x[t], w_gate[e], w_up[e])
            ys[q] = h @ bf16_to_f64(w_down_t[e])
        outs.append(combine(ys, w[t], None if resid is None else resid[t]))
    return np.stack(outs) if outs else np.zeros((0, H), np.uint16)


# ----------------------------------------------------------------------------- decode-layer envelope
#
# The steps on either side of the routed-expert block in a decode layer: the
# block's input is the RMS-normalised hidden state, the router picks each
# token's K experts from it, and the block's output is added to the residual
# stream (abstract: MoE blocks and whole-model decoding; the block speedups
# are measured with routing in place). Readings: RMSNorm with a learned
# per-feature weight, rounded once to BF16; router logits W_r x from the BF16
# normalised state; softmax over all experts; the K most probable experts in
# descending probability, lower id first on ties; their probabilities as
# weights, optionally renormalised to sum to 1; output = BF16(h + block).


def rmsnorm(h_bits, gamma_bits, eps: float):
    """x = BF16( h / sqrt(mean(h^2) + eps) * gamma ), per token, float64, one rounding."""
    h = bf16_to_f64(h_bits)
    inv = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + float(eps))
    return f64_to_bf16(h * inv * bf16_to_f64(gamma_bits))


def router(x_bits, w_router_bits, K: int, renorm: bool):
    """Top-K softmax routing of BF16 states x [T][H] with router rows W_r [E][H].

    Returns (ids int32 [T][K] in descending probability, lower id first on
    ties; weights float64 [T][K]; logits float64 [T][E])."""
    x = bf16_to_f64(x_bits)
    logits = x @ bf16_to_f64(w_router_bits).T
    p = np.exp(logits - logits.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    T, E = p.shape
    ids = np.zeros((T, K), np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-p[t, e], e))
        ids[t] = order[:K]
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=-1, keepdims=True)
    return ids, w, logits


def layer_forward(h, gamma, eps, w_router, K, renorm, w_gate, w_up, w_down_t, tg=None, tu=None, sg=None,
                  su=None, signs=None, A=None, Bt=None, k=0, c=0, recovery=RECOVERY_SKETCH, dense=False,
                  x=None, ids=None, w=None, tokens=None):
    """One decode layer's routed-expert block with its envelope:
    out = BF16(h + sum_q w_q y_(t,q)) with x = rmsnorm(h), (ids, w) = router(x).

    dense=True runs the dense block (every channel) instead of the selected
    one. x, ids, w: optional overrides (e.g. the values a device computed), so
    that later steps can be checked on the same selections.
    Returns (out BF16 bits, x, ids, w, per-pair details or None)."""
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
    are read only when their exact activations are used: to rank them for
    the kept set (k > 0) or, in the candidates_exact recovery variant, as the
    dropped candidates' recovery coefficients. With k = 0 and the default
    recovery nothing reads them. With the variant and c = I every channel is
    a candidate, so no sketch activation enters the result and the sketch is
    not read. threshold: the kept sets come from the threshold keep rule, so
    the candidates' exact activations are always used and keep_sets must be
    given (k is not used).
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
