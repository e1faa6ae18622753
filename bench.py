"""Benchmark of the selected-channel routed-expert SwiGLU layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--no-cpu]

Workload: a Qwen3-30B-A3B-shaped MoE layer (H 2048, 128 experts, top-8,
SwiGLU intermediate 768, BF16 weights ~N(0, 0.02) times a per-channel
LogNormal(0, 0.5) factor), decode batch 1, read budget k = 138 (18 % of I),
c = 276 candidates, rank r = 64. One step is one call of moe_select_forward
(the whole hot path: screen, exact top-k, down over kept channels, low-rank
recovery, combine) for one fresh token. Steps cycle over a ring of L
independently drawn layers, so every step streams weights that are not
resident in the 256 MiB last-level cache, as in a real decode step through a
48-layer model. Inputs are resident in HBM before the timed region; the K
timed steps are one replay of a HIP graph holding K distinct calls.

Prints one JSON line on stdout (logs go to stderr).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer µs/token + achieved HBM GB/s at 18% read budget, batch 1/8/16"
PEAK_HBM_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="ring of independently drawn layers")
    ap.add_argument("--batches", default="1,8,16")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--stack", action="store_true",
                    help="instead of the default line: a 48-layer stack of independently drawn layers, "
                         "batches 1/4/8/16/32, budgets 10.8/13/18/53/67 %%")
    ap.add_argument("--olmoe", action="store_true",
                    help="instead of the default line: the OLMoE-1B-7B-shaped layer, 64 tokens, Zipf(1.1) experts")
    ap.add_argument("--layer-stack", action="store_true",
                    help="instead of the default line: the 48-layer stack run as a chained decode step with the "
                         "envelope (RMSNorm, router, residual add) fused into each layer's launch, batches 1-32, "
                         "18 %% budget, against the fused dense layer and an unfused torch envelope")
    ap.add_argument("--recovery", action="store_true",
                    help="instead of the default line: recovery rank sweep (r 0..128) of both recovery variants "
                         "at batch 1 and 16, 18 %% budget, with each output's deviation from the dense layer")
    ap.add_argument("--threshold", action="store_true",
                    help="instead of the default line: the threshold keep rule against top-k at batch 1, "
                         "tau calibrated offline for 18 %% and 13 %% budgets: kept channels, bytes read and "
                         "time per token on evaluation tokens, same-distribution and RMS-shifted")
    ap.add_argument("--cold", action="store_true",
                    help="instead of the default line: batch 1, each call timed on its own after a 1 GiB "
                         "cache flush, median / p10 / p90 of the selected and the dense layer")
    ap.add_argument("--general", action="store_true",
                    help="with --phase-trace: the general per-pair instance instead of the batch-1 one")
    ap.add_argument("--trace-batch", type=int, default=1,
                    help="with --phase-trace: tokens per call (8 and 16 run the general per-pair instance)")
    ap.add_argument("--phase-trace", action="store_true",
                    help="instead of the default line: per-phase timeline of the batch-1 selected and dense "
                         "kernels from in-kernel clock stamps (needs the trace build, CFM_PHASE_TRACE=1)")
    ap.add_argument("--cold-reps", type=int, default=40, help="cold calls timed for the default line")
    ap.add_argument("--summarize-pmc", default="", metavar="F,W,CF,CW,MIB",
                    help="only print the per-launch traffic record from rocprofv3 --pmc result folders (bench "
                         "FETCH_SIZE, bench WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE) and the copy size")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device (calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- inputs on the device

def make_layer(torch, seed, layer, E, I, H, sigma=0.02, chan_scale=True):
    """Synthetic BF16 expert weights drawn on the device (same recipe as synth/), and the layer's
    rotation signs from its 64-bit seed through the library's own generator."""
    import calibration_free_channel_amd as cfm
    g = torch.Generator(device="cuda")
    g.manual_seed(seed * 100003 + layer)
    mats = []
    for _ in range(3):
        w = torch.randn((E, I, H), generator=g, device="cuda", dtype=torch.float32).mul_(sigma)
        if chan_scale:
            s = torch.randn((E, I, 1), generator=g, device="cuda", dtype=torch.float32).mul_(0.5).exp_()
            w.mul_(s)
        mats.append(w.to(torch.bfloat16))
        del w
    signs = cfm.rotation_signs(seed * 100003 + layer, H)
    return mats[0], mats[1], mats[2], signs


def make_tokens(torch, seed, n, T, E, K, H):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed * 7919 + 17)
    z = torch.randn((n, T, H), generator=g, device="cuda", dtype=torch.float32)
    z = z * torch.rsqrt(z.pow(2).mean(-1, keepdim=True) + 1e-6)
    x = z.to(torch.bfloat16)
    logits = torch.randn((n, T, E), generator=g, device="cuda", dtype=torch.float32)
    p = torch.softmax(logits, dim=-1)
    w, ids = torch.topk(p, K, dim=-1)
    return x.contiguous(), ids.to(torch.int32).contiguous(), w.contiguous()


# ----------------------------------------------------------------------------- GPU measurement

def timed_graph(torch, fn, n_steps):
    """Capture fn(i) for i < n_steps in one graph; return (ms for one replay, wall ms)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_steps):
            fn(i)
    g.replay()                      # first replay: untimed (graph upload)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return e0.elapsed_time(e1), wall


def kernel_times(torch, cfm, fn, n_steps):
    """Average duration of each library kernel (HIP events around every launch,
    host kept ahead of the GPU so the events bracket only device work)."""
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    cfm.timing_enable(True)
    for i in range(n_steps):
        fn(i)
    cfm.timing_enable(False)
    rep = cfm.timing_report()
    return {k: v[1] / v[0] for k, v in rep.items()}, {k: v[0] / n_steps for k, v in rep.items()}


def stream_gbps(torch, nbytes=2 << 30, reps=10):
    """Context for the roofline: what plain streaming kernels achieve on this GPU, as (read GB/s of
    torch's sum over a 2 GiB float32 buffer, read + write GB/s of torch's copy of 1 GiB)."""
    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3
    t = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    rd = nbytes / timed(lambda: t.sum()) / 1e9
    del t
    a = torch.ones(nbytes // 2, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    cp = nbytes / timed(lambda: b.copy_(a)) / 1e9
    del a, b
    return rd, cp


def measured_traffic():
    """HBM bytes per launch of k_select_fused from the committed rocprofv3 --pmc
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or
    None when the kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "k_select_fused_q18_b1_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec["source_files"] != kernel_sources() or rec["source_sha256"] != sources_sha256(rec["source_files"]):
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


def kernel_sources():
    """The files the single-launch kernels are built from (every header of the library and the
    fused translation units), relative to the repository root."""
    import glob
    csrc = os.path.join(ROOT, "calibration_free_channel_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.h")) + glob.glob(os.path.join(csrc, "fused*.hip")))
    return [os.path.relpath(f, ROOT) for f in files]


def sources_sha256(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def summarize_pmc(spec):
    """Per-launch HBM bytes of the batch-1 kernels from four rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE of the bench, then of a plain copy of known size), scaled by what the counters read for
    the copy; prints the record that bench.py reads back as `traffic`. spec: comma-separated
    fetch_dir,write_dir,copy_fetch_dir,copy_write_dir,copy_mib."""
    import glob
    import sqlite3
    import statistics
    fdir, wdir, cfdir, cwdir, mib = spec.split(",")
    mib = int(mib)

    def per_kernel(d, counter):
        """{kernel name: median over dispatches of the counter (KiB)} from rocprofv3's result database."""
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True):
            con = sqlite3.connect(f)
            for name, disp, v in con.execute(
                    "select kernel_name, dispatch_id, sum(value) from counters_collection "
                    "where counter_name = ? group by dispatch_id", (counter,)):
                vals.setdefault(name, []).append(float(v))
            con.close()
        return {k: statistics.median(v) for k, v in vals.items()}

    def find(d, name):
        hits = {k: v for k, v in d.items() if name + "<" in k}
        if not hits:
            raise SystemExit(f"no {name} dispatches in the counter output")
        return max(hits.items(), key=lambda kv: kv[1])

    copy_kib = mib * 1024.0
    cf = max(per_kernel(cfdir, "FETCH_SIZE").values())
    cw = max(per_kernel(cwdir, "WRITE_SIZE").values())
    fscale, wscale = copy_kib / cf, copy_kib / cw
    fetch, write = per_kernel(fdir, "FETCH_SIZE"), per_kernel(wdir, "WRITE_SIZE")
    rec = {"kernel": "k_select_fused", "workload": "q18_b1"}
    for key, name in (("", "k_select_fused"), ("dense_", "k_dense_fused")):
        kn, fk = find(fetch, name)
        _, wk = find(write, name)
        rec[key + "kernel_name"] = kn
        rec[key + "fetch_kib_raw"] = round(fk, 2)
        rec[key + "write_kib_raw"] = round(wk, 2)
        rec[key + "fetch_bytes"] = int(round(fk * fscale * 1024))
        rec[key + "write_bytes"] = int(round(wk * wscale * 1024))
    rec.update({"fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
                "copy_probe_mib": mib, "source_files": kernel_sources()})
    rec["source_sha256"] = sources_sha256(rec["source_files"])
    print(json.dumps(rec, indent=1))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl_name="q18_b1", target_s=8.0):
    """The CPU oracle (plain C++, float64) on a bounded sample of the same workload: the selected forward
    (screen, exact top-k, down, recovery, combine) of whole tokens, routed pairs spread over the threads,
    timed on 1 thread and on all of the host's threads (at most 16)."""
    import numpy as np

    import synth
    from oracle import cfm_oracle as O

    wl = synth.WORKLOADS[wl_name]
    s = wl.shape
    n_tok = 2
    ids, w = synth.routing(n_tok, s.E, s.K, wl.seed + 101, 0)
    x = synth.hidden_states(n_tok, s.H, wl.seed + 101, 0, rmsnorm=True)
    used = sorted(set(int(e) for e in ids.reshape(-1)))
    local = {e: n for n, e in enumerate(used)}
    ids_l = np.vectorize(local.get)(ids).astype(np.int32)
    wg, wu, wd = synth.layer_weights(s, wl.seed, 0, experts=used)
    signs = synth.rotation_signs(s.H, wl.seed, 0)
    tg, tu, sg, su = O.sketch_build(wg, wu, signs)          # offline steps: not timed
    A, Bt = O.lowrank_build(wd, wl.r)
    all_threads = max(1, min(16, os.cpu_count() or 1))
    res = {}
    for th in sorted({1, all_threads}):
        done, t0 = 0, time.perf_counter()
        while True:
            O.select_forward(x, ids_l, w, wg, wu, wd, tg, tu, sg, su, signs, A, Bt, wl.k, wl.c, threads=th,
                             details=False)
            done += n_tok
            el = time.perf_counter() - t0
            if el >= target_s / 2:
                break
        t0 = time.perf_counter()
        O.dense_forward(x, ids_l, w, wg, wu, wd, threads=th)
        res[th] = (el / done * 1e6, (time.perf_counter() - t0) / n_tok * 1e6, done)
    us_all, dense_all, done_all = res[all_threads]
    return {"value": round(us_all, 1), "unit": "us/token", "cores": all_threads, "kind": "oracle",
            "sample": f"{wl_name}: {n_tok} tokens (their {len(used)} routed experts) through the plain-C++ float64 "
                      f"oracle's selected forward, repeated to {done_all} tokens on {all_threads} threads and "
                      f"{res[1][2]} on 1 thread; sketch and low-rank map prepared untimed",
            "us_per_token_1_thread": round(res[1][0], 1), "cpu_model": cpu_model(),
            "dense_us_per_token": round(dense_all, 1), "dense_us_per_token_1_thread": round(res[1][1], 1)}


SELECT_PHASES = {
    0: "start", 1: "first loads issued (x, signs, router id, sketch rows, scales, Bt)", 2: "x rotated",
    3: "screen done", 4: "recovery partial sums published", 5: "sketch activations + partial sums in",
    6: "top-c done", 7: "exact rows done (h published)", 8: "candidate-row prefetch issued (general instance)",
    9: "exact activations in", 10: "top-k done",
    11: "kept down and Bt row loads issued (batch-1 instance) / candidate rows landed (general, one token) / "
        "z formed (general, several tokens)",
    12: "kept Bt rows in, z formed / A z formed (general, several tokens)", 13: "pair output slice stored",
    14: "combine done",
    15: "wave 0 sketch activations in", 16: "wave 1 sketch activations in", 17: "wave 2 sketch activations in",
    18: "wave 3 sketch activations in", 19: "wave 0 exact activations in", 20: "wave 1 exact activations in",
    21: "wave 2 exact activations in", 22: "wave 3 exact activations in", 23: "top-c range known",
    24: "top-c pass 1", 25: "top-c last pass", 26: "top-c ranks known", 27: "top-k range known",
    28: "top-k pass 1", 29: "top-k last pass", 30: "top-k ranks known"}
DENSE_PHASES = {0: "start", 20: "exact rows done", 21: "activations in", 22: "down + combine done"}


def phase_trace(torch, cfm, args):
    """Per-phase timeline of the per-pair kernels from in-kernel clock stamps (100 MHz device clock),
    taken from the last launch of a ring of back-to-back launches; medians over repetitions. Batch 1 by
    default; --trace-batch 8 or 16 traces the general instance at that batch (one pair slot per workgroup)."""
    import numpy as np
    E, K, I, H = 128, 8, 768, 2048
    k, c, r = 138, 276, 64
    L = args.layers
    layers = []
    lr_ws = torch.empty(cfm.lowrank_workspace(E, I, H, r), dtype=torch.uint8, device="cuda")
    for l in range(L):
        wg, wu, wd, signs = make_layer(torch, args.seed, l, E, I, H)
        sk = cfm.sketch_build(wg, wu, signs)
        A, Bt = cfm.lowrank_build(wd, r, ws=lr_ws)
        layers.append((wg, wu, wd, signs, sk, A, Bt))
    del lr_ws
    ring, reps = 16, 60
    T = args.trace_batch
    if T not in (1, 8, 16):
        raise SystemExit("--trace-batch: 1, 8 or 16 (one pair slot per workgroup of the 256-workgroup grid)")
    x, ids, w = make_tokens(torch, args.seed + 1, ring, T, E, K, H)
    ws_s = cfm.new_workspace(cfm.select_workspace(T, K, E, I, H, k, c, r), "cuda")
    ws_d = cfm.new_workspace(cfm.dense_workspace(T, K, E, I, H), "cuda")
    out = torch.empty((ring, T, H), dtype=torch.bfloat16, device="cuda")
    buf = torch.zeros(256 * 32, dtype=torch.int64, device="cuda")
    cfm.phase_trace(buf)

    def sel(i):
        wg, wu, wd, signs, sk, A, Bt = layers[i % L]
        cfm.moe_select_forward(x[i], ids[i], w[i], wg, wu, wd, signs, *sk, A, Bt, k, c, r, out=out[i], ws=ws_s)

    def dense(i):
        wg, wu, wd, *_ = layers[i % L]
        cfm.moe_dense_forward(x[i], ids[i], w[i], wg, wu, wd, out=out[i], ws=ws_d)

    res = {}
    prev_path = cfm.set_forward_path(cfm.FORWARD_PER_PAIR_GENERAL if args.general else cfm.FORWARD_PER_PAIR)
    for name, fn, phases in (("selected", sel, SELECT_PHASES), ("dense", dense, DENSE_PHASES)):
        for i in range(ring):
            fn(i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(ring):
                fn(i)
        rows = []
        for _ in range(reps):
            buf.zero_()
            g.replay()
            torch.cuda.synchronize()
            rows.append(buf.view(256, 32).cpu().numpy().copy())
        st = np.stack(rows)                                    # [reps][G][32]
        passes = {}
        if name == "selected":                                 # (clock << 4 | passes) in the last-pass slots
            for slot, what in ((25, "top-c"), (29, "top-k")):
                v = st[:, :, slot]
                passes[what] = np.bincount(np.where(v > 0, v & 15, 1).ravel()).tolist()
                st[:, :, slot] = v >> 4
        t0 = st[:, :, 0].min(axis=1, keepdims=True)
        rel = np.where(st > 0, (st - t0[:, :, None]) * 0.01, np.nan)   # us (100 MHz clock); 0 = not stamped
        table = {}
        for n, what in phases.items():
            v = rel[:, :, n]
            if np.isnan(v).all():
                continue
            table[f"{n:02d} {what}"] = {"median_wg_us": round(float(np.nanmedian(np.nanmedian(v, axis=1))), 2),
                                        "max_wg_us": round(float(np.nanmedian(np.nanmax(v, axis=1))), 2)}
        xcd = st[:, :, 31]
        starts = [round(float(np.median([(st[q, xcd[q] == d, 0].min() - t0[q, 0]) * 0.01 for q in range(reps)])), 2)
                  for d in range(8)]
        res[name] = {"phases": table, "xcd_start_us": starts, "select_pass_histogram": passes}
        if os.environ.get("CFM_TRACE_DUMP"):
            np.save(os.environ["CFM_TRACE_DUMP"] + f"_{name}.npy", st)
        log(f"{name}: " + "; ".join(f"{kk}: {vv['median_wg_us']}/{vv['max_wg_us']}" for kk, vv in table.items()))
        log(f"{name}: XCD start offsets (us) {starts}; passes per select (count of workgroups by passes) {passes}")
    cfm.phase_trace(None)
    cfm.set_forward_path(prev_path)
    print(json.dumps({"phase_trace": res, "workload": f"q18_b{T}",
                      "instance": "general" if (args.general or T > 1) else "batch-1",
                      "ring": ring, "reps": reps}), flush=True)


def stack(torch, cfm, args):
    """A decode step's routed-expert work through 48 independently drawn Qwen3-30B-A3B-shaped
    layers (58 GB of BF16 weights, resident in HBM), one call per layer in one HIP graph."""
    E, K, I, H, r = 128, 8, 768, 2048, 64
    NL = 48
    layers = []
    lr_ws = torch.empty(cfm.lowrank_workspace(E, I, H, r), dtype=torch.uint8, device="cuda")
    t0 = time.perf_counter()
    for l in range(NL):
        wg, wu, wd, signs = make_layer(torch, args.seed + 1000, l, E, I, H)
        sk = cfm.sketch_build(wg, wu, signs)
        A, Bt = cfm.lowrank_build(wd, r, ws=lr_ws)
        layers.append((wg, wu, wd, signs, sk, A, Bt))
        if l % 8 == 7:
            log(f"  {l + 1} layers built ({time.perf_counter() - t0:.0f} s)")
    del lr_ws
    torch.cuda.synchronize()
    fracs = [0.108, 0.13, 0.18, 0.53, 0.67]
    rows = []
    for T in (1, 4, 8, 16, 32):
        x, ids, w = make_tokens(torch, args.seed + 77 + T, NL, T, E, K, H)
        out = torch.empty((NL, T, H), dtype=torch.bfloat16, device="cuda")
        wsd = cfm.new_workspace(cfm.dense_workspace(T, K, E, I, H), "cuda")

        def dense(i):
            wg, wu, wd, *_ = layers[i % NL]
            cfm.moe_dense_forward(x[i % NL], ids[i % NL], w[i % NL], wg, wu, wd, out=out[i % NL], ws=wsd)

        for i in range(NL):
            dense(i)
        ms_d, _ = timed_graph(torch, dense, NL)
        for f in fracs:
            k = int(round(f * I))
            c = min(2 * k, I)
            wss = cfm.new_workspace(cfm.select_workspace(T, K, E, I, H, k, c, r), "cuda")

            def sel(i):
                wg, wu, wd, signs, sk, A, Bt = layers[i % NL]
                cfm.moe_select_forward(x[i % NL], ids[i % NL], w[i % NL], wg, wu, wd, signs, *sk, A, Bt, k, c, r,
                                       out=out[i % NL], ws=wss)

            for i in range(NL):
                sel(i)
            ms_s, _ = timed_graph(torch, sel, NL)
            st = torch.zeros(cfm.STATS_BYTES, dtype=torch.uint8, device="cuda")
            wg, wu, wd, signs, sk, A, Bt = layers[0]
            cfm.moe_select_forward(x[0], ids[0], w[0], wg, wu, wd, signs, *sk, A, Bt, k, c, r, out=out[0], ws=wss,
                                   stats=st)
            torch.cuda.synchronize()
            sd = cfm.decode_stats(st)
            nbytes = sum(sd[q] for q in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery",
                                          "bytes_io"))
            row = {"T": T, "budget": f, "k": k, "c": c,
                   "us_per_token_per_layer": round(ms_s * 1e3 / (NL * T), 3),
                   "dense_us_per_token_per_layer": round(ms_d * 1e3 / (NL * T), 3),
                   "speedup_vs_dense": round(ms_d / ms_s, 3),
                   "read_fraction_of_dense": round(nbytes / sd["bytes_dense_equiv"], 3)}
            rows.append(row)
            log(f"T={T} f={f}: {row}")
            del wss
        del wsd, out, x, ids, w
    print(json.dumps({"workload": "48-layer stack of Qwen3-30B-A3B-shaped MoE layers (H 2048, E 128, top-8, "
                                  "I 768), r 64, one decode step per graph replay", "data": "synthetic",
                      "rows": rows}), flush=True)


def layer_stack(torch, cfm, args):
    """One decode step through 48 independently drawn Qwen3-30B-A3B-shaped MoE blocks with their envelope:
    h_(l+1) = h_l + block_l(RMSNorm_l(h_l)) with the router's top-8 routing, each layer one launch reading
    the previous layer's output (a real chain, captured as one HIP graph). Compared with the same chain on
    the dense block, and with an unfused envelope (torch RMSNorm, router matmul, softmax, top-k and add
    around the plain selected entry point)."""
    E, K, I, H, r = 128, 8, 768, 2048, 64
    k, c = 138, 276
    NL = 48
    eps = 1e-6
    layers = []
    lr_ws = torch.empty(cfm.lowrank_workspace(E, I, H, r), dtype=torch.uint8, device="cuda")
    t0 = time.perf_counter()
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed * 131 + 7)
    for l in range(NL):
        wg, wu, wd, signs = make_layer(torch, args.seed + 3000, l, E, I, H)
        sk = cfm.sketch_build(wg, wu, signs)
        A, Bt = cfm.lowrank_build(wd, r, ws=lr_ws)
        wr = torch.randn((E, H), generator=g, device="cuda").mul_(0.02).to(torch.bfloat16)
        gam = (1.0 + 0.1 * torch.randn((H,), generator=g, device="cuda")).to(torch.bfloat16)
        layers.append((wg, wu, wd, signs, sk, A, Bt, wr, gam))
        if l % 8 == 7:
            log(f"  {l + 1} layers built ({time.perf_counter() - t0:.0f} s)")
    del lr_ws
    torch.cuda.synchronize()
    rows = []
    for T in (1, 4, 8, 16, 32):
        hs = torch.empty((NL + 1, T, H), dtype=torch.bfloat16, device="cuda")
        hs[0] = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
        wss = cfm.new_workspace(cfm.select_workspace(T, K, E, I, H, k, c, r), "cuda")
        wsd = cfm.new_workspace(cfm.dense_workspace(T, K, E, I, H), "cuda")

        def fused_sel(i):
            wg, wu, wd, signs, sk, A, Bt, wr, gam = layers[i]
            cfm.moe_layer_forward(hs[i], gam, eps, wr, K, wg, wu, wd, signs, *sk, A, Bt, k, c, r, out=hs[i + 1], ws=wss)

        def fused_dense(i):
            wg, wu, wd, signs, sk, A, Bt, wr, gam = layers[i]
            cfm.moe_layer_dense_forward(hs[i], gam, eps, wr, K, wg, wu, wd, out=hs[i + 1], ws=wsd)

        def unfused_sel(i):
            wg, wu, wd, signs, sk, A, Bt, wr, gam = layers[i]
            x = torch.nn.functional.rms_norm(hs[i].float(), (H,), weight=gam.float(), eps=eps).to(torch.bfloat16)
            p = torch.softmax((x @ wr.t()).float(), dim=-1)
            w, ids = torch.topk(p, K, dim=-1)
            y = cfm.moe_select_forward(x, ids.to(torch.int32), w.contiguous(), wg, wu, wd, signs, *sk, A, Bt, k, c,
                                       r, ws=wss)
            hs[i + 1].copy_(hs[i] + y)

        res = {}
        for name, fn in (("selected_fused", fused_sel), ("dense_fused", fused_dense), ("selected_unfused", unfused_sel)):
            with cfm.forward_path(cfm.FORWARD_PER_PAIR):
                for i in range(NL):
                    fn(i)
                ms, _ = timed_graph(torch, fn, NL)
            res[name] = round(ms * 1e3 / (NL * T), 3)
        row = {"T": T, "us_per_token_per_layer": res,
               "speedup_fused_vs_dense": round(res["dense_fused"] / res["selected_fused"], 3),
               "fused_vs_unfused_envelope": round(res["selected_unfused"] / res["selected_fused"], 3)}
        rows.append(row)
        log(f"layer stack T={T}: {row}")
        del hs, wss, wsd
    print(json.dumps({"workload": "48-layer chained decode step, Qwen3-30B-A3B-shaped MoE blocks (H 2048, E 128, "
                                  "top-8, I 768) with RMSNorm, router and residual add; k 138 c 276 r 64",
                      "data": "synthetic", "rows": rows}), flush=True)


def recovery_sweep(torch, cfm, args):
    """Recovery rank r and the two recovery variants (every skipped channel through the map with its
    sketch activation, or the dropped candidates with their exact activation) on the Qwen3-30B-A3B-shaped
    layer ring at k 138, c 276: time per token, and the relative L2 distance of each token's output from
    the dense layer's output on the same inputs (synthetic Gaussian weights: an approximation error, not
    a model-quality figure)."""
    E, K, I, H = 128, 8, 768, 2048
    k, c = 138, 276
    NL = args.layers
    ranks = (0, 16, 32, 64, 128)
    base = []
    for l in range(NL):
        wg, wu, wd, signs = make_layer(torch, args.seed, l, E, I, H)
        base.append((wg, wu, wd, signs, cfm.sketch_build(wg, wu, signs)))
    rows = []
    for T in (1, 16):
        n = NL * 4
        x, ids, w = make_tokens(torch, args.seed + 300 + T, n, T, E, K, H)
        dense_out = torch.empty((n, T, H), dtype=torch.bfloat16, device="cuda")
        wsd = cfm.new_workspace(cfm.dense_workspace(T, K, E, I, H), "cuda")
        for i in range(n):
            wg, wu, wd, *_ = base[i % NL]
            cfm.moe_dense_forward(x[i], ids[i], w[i], wg, wu, wd, out=dense_out[i], ws=wsd)
        ms_d, _ = timed_graph(torch, lambda i: cfm.moe_dense_forward(
            x[i], ids[i], w[i], *base[i % NL][:3], out=dense_out[i], ws=wsd), n)
        ref = dense_out.float()
        for r in ranks:
            maps = [cfm.lowrank_build(b[2], r) for b in base]
            wss = cfm.new_workspace(cfm.select_workspace(T, K, E, I, H, k, c, r), "cuda")
            out = torch.empty((n, T, H), dtype=torch.bfloat16, device="cuda")
            for rec in ((cfm.RECOVER_SKETCH, cfm.RECOVER_CANDIDATES_EXACT) if r > 0 else (cfm.RECOVER_SKETCH,)):
                def sel(i, rec=rec):
                    wg, wu, wd, signs, sk = base[i % NL]
                    A, Bt = maps[i % NL]
                    cfm.moe_select_forward(x[i], ids[i], w[i], wg, wu, wd, signs, *sk, A, Bt, k, c, r,
                                           out=out[i], ws=wss, recovery=rec)
                for i in range(n):
                    sel(i)
                torch.cuda.synchronize()
                dev_ = ((out.float() - ref).norm(dim=-1) / ref.norm(dim=-1)).flatten()
                ms_s, _ = timed_graph(torch, sel, n)
                row = {"T": T, "r": r, "recovery": rec,
                       "us_per_token": round(ms_s * 1e3 / (n * T), 3),
                       "dense_us_per_token": round(ms_d * 1e3 / (n * T), 3),
                       "rel_l2_vs_dense_mean": round(float(dev_.mean()), 4),
                       "rel_l2_vs_dense_max": round(float(dev_.max()), 4)}
                rows.append(row)
                log(f"recovery sweep: {row}")
            del maps, wss, out
        # every channel a candidate (53 % budget, k 407, c = I): the variant needs no sketch
        kb, cb, rb = 407, I, 64
        maps = [cfm.lowrank_build(b[2], rb) for b in base]
        wss = cfm.new_workspace(cfm.select_workspace(T, K, E, I, H, kb, cb, rb), "cuda")
        out = torch.empty((n, T, H), dtype=torch.bfloat16, device="cuda")
        for rec in (cfm.RECOVER_SKETCH, cfm.RECOVER_CANDIDATES_EXACT):
            def selb(i, rec=rec):
                wg, wu, wd, signs, sk = base[i % NL]
                A, Bt = maps[i % NL]
                cfm.moe_select_forward(x[i], ids[i], w[i], wg, wu, wd, signs, *sk, A, Bt, kb, cb, rb,
                                       out=out[i], ws=wss, recovery=rec)
            with cfm.forward_path(cfm.FORWARD_PER_PAIR):
                for i in range(n):
                    selb(i)
                torch.cuda.synchronize()
                dev_ = ((out.float() - ref).norm(dim=-1) / ref.norm(dim=-1)).flatten()
                ms_s, _ = timed_graph(torch, selb, n)
            row = {"T": T, "r": rb, "k": kb, "c": cb, "recovery": rec,
                   "us_per_token": round(ms_s * 1e3 / (n * T), 3),
                   "dense_us_per_token": round(ms_d * 1e3 / (n * T), 3),
                   "rel_l2_vs_dense_mean": round(float(dev_.mean()), 4),
                   "rel_l2_vs_dense_max": round(float(dev_.max()), 4)}
            rows.append(row)
            log(f"recovery sweep: {row}")
        del maps, wss, out
        del wsd, dense_out, x, ids, w
    print(json.dumps({"workload": "recovery rank sweep on the Qwen3-30B-A3B-shaped layer (H 2048, E 128, top-8, "
                                  "I 768), k 138, c 276; and k 407, c = I", "data": "synthetic", "rows": rows}),
          flush=True)


def cold_measure(torch, cfm, layers, reps, warmup, seed, k=138, c=276, r=64):
    """Batch 1 on Qwen3-30B-A3B-shaped layers: every call timed on its own with HIP events, after an
    untimed write of 1 GiB that evicts the L2 and the 256 MB last-level cache, so each call reads its
    weights from HBM, and a GPU sleep that lets the host enqueue the call before the first event is
    taken. Median, p10 and p90 over the reps for the selected and the dense layer (alternating), and
    the algorithmic GB/s at the median."""
    import numpy as np
    E, I, H = layers[0][0].shape
    K = 8
    NL = len(layers)
    x, ids, w = make_tokens(torch, seed + 77, reps + warmup, 1, E, K, H)
    ws_s = cfm.new_workspace(cfm.select_workspace(1, K, E, I, H, k, c, r), "cuda")
    ws_d = cfm.new_workspace(cfm.dense_workspace(1, K, E, I, H), "cuda")
    out = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    st = torch.zeros(cfm.STATS_BYTES, dtype=torch.uint8, device="cuda")
    times = {"selected": [], "dense": []}
    bytes_ = {}
    for i in range(reps + warmup):
        wg, wu, wd, signs, sk, A, Bt = layers[i % NL]
        for name in ("selected", "dense"):
            flush.fill_(i & 255)
            # the GPU sleeps while the host enqueues the events and the call, so the events
            # bracket device work only (not the binding's argument marshalling)
            torch.cuda._sleep(2_000_000)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if name == "selected":
                cfm.moe_select_forward(x[i], ids[i], w[i], wg, wu, wd, signs, *sk, A, Bt, k, c, r, out=out, ws=ws_s,
                                       stats=st if i == 0 else None)
            else:
                cfm.moe_dense_forward(x[i], ids[i], w[i], wg, wu, wd, out=out, ws=ws_d)
            e1.record()
            torch.cuda.synchronize()
            if i >= warmup:
                times[name].append(e0.elapsed_time(e1) * 1e3)
            if i == 0 and name == "selected":
                d = cfm.decode_stats(st)
                bytes_["selected"] = sum(d[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down",
                                                        "bytes_recovery", "bytes_io"))
                bytes_["dense"] = d["bytes_dense_equiv"]
    del flush, ws_s, ws_d
    res = {}
    for name, v in times.items():
        a = np.array(v)
        med = float(np.median(a))
        res[name] = {"median_us": round(med, 3), "p10_us": round(float(np.percentile(a, 10)), 3),
                     "p90_us": round(float(np.percentile(a, 90)), 3),
                     "GBps_at_median": round(bytes_[name] / (med * 1e-6) / 1e9, 1), "bytes": bytes_[name]}
    res["speedup_at_median"] = round(res["dense"]["median_us"] / res["selected"]["median_us"], 3)
    res["reps"] = reps
    return res


def cold_timing(torch, cfm, args):
    """The cold-call measurement on its own, over args.steps reps."""
    E, K, I, H = 128, 8, 768, 2048
    r = 64
    layers = []
    for l in range(args.layers):
        wg, wu, wd, signs = make_layer(torch, args.seed, l, E, I, H)
        A, Bt = cfm.lowrank_build(wd, r)
        layers.append((wg, wu, wd, signs, cfm.sketch_build(wg, wu, signs), A, Bt))
    res = cold_measure(torch, cfm, layers, args.steps, args.warmup, args.seed)
    print(json.dumps({"workload": "Qwen3-30B-A3B-shaped MoE layer, batch 1, 18 % (k 138, c 276, r 64); "
                                  "each call after a 1 GiB flush, HIP events around the call",
                      "data": "synthetic", "reps": args.steps, "layers": args.layers, "result": res}), flush=True)


def calibrate_tau(torch, cfm, layer, x, ids, w, k, c, r, ws):
    """Offline calibration of the threshold for one layer with the library's own threshold calls: the
    largest tau (over float bit patterns, by bisection) with which the calibration pairs keep at least
    k channels each on average, i.e. the (k P)-th largest exact |h| among their candidates."""
    import struct
    wg, wu, wd, signs, sk, A, Bt = layer
    T, K = ids.shape
    cnt = torch.empty((T * K,), dtype=torch.int32, device="cuda")
    need = k * T * K

    def kept(bits):
        tau = struct.unpack("<f", struct.pack("<I", bits))[0]
        cfm.moe_select_forward_threshold(x, ids, w, wg, wu, wd, signs, *sk, A, Bt, tau, c, r, ws=ws, keep_count=cnt)
        return int(cnt.sum().item())

    lo, hi = 0, 0x7F800000                # kept(lo) >= need > kept(hi) (tau +inf keeps nothing)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if kept(mid) >= need:
            lo = mid
        else:
            hi = mid
    return struct.unpack("<f", struct.pack("<I", lo))[0]


def threshold_study(torch, cfm, args):
    """The threshold keep rule against top-k on the Qwen3-30B-A3B-shaped layer ring (c 276, r 64), batch 1.
    Per layer, tau is calibrated offline on 64 calibration tokens so that their pairs keep k channels
    each on average (k 138: 18 %; k 100: 13 %), then applied to evaluation tokens drawn the same way
    and to tokens whose RMS is 0.8x and 1.25x (a stand-in for inputs that differ from the calibration
    data): kept channels per pair, routed-expert bytes each token reads as a fraction of the dense
    layer's, and time per token, beside top-k at the same k."""
    import numpy as np
    E, K, I, H = 128, 8, 768, 2048
    c, r = 276, 64
    NL = args.layers
    log(f"threshold study: building {NL} layers ...")
    layers = []
    for l in range(NL):
        wg, wu, wd, signs = make_layer(torch, args.seed, l, E, I, H)
        A, Bt = cfm.lowrank_build(wd, r)
        layers.append((wg, wu, wd, signs, cfm.sketch_build(wg, wu, signs), A, Bt))
    Tc = 64
    xc, idc, wc = make_tokens(torch, args.seed + 900, NL, Tc, E, K, H)
    wsc = cfm.new_workspace(cfm.select_workspace(Tc, K, E, I, H, c, c, r), "cuda")
    n = NL * 8
    xe, ide, we = make_tokens(torch, args.seed + 901, n, 1, E, K, H)
    sets = {"same distribution": xe}
    for f in (0.8, 1.25):
        sets[f"RMS x{f}"] = (xe.float() * f).to(torch.bfloat16).contiguous()
    ws1 = cfm.new_workspace(cfm.select_workspace(1, K, E, I, H, c, c, r), "cuda")
    wsd = cfm.new_workspace(cfm.dense_workspace(1, K, E, I, H), "cuda")
    out = torch.empty((n, 1, H), dtype=torch.bfloat16, device="cuda")
    cnt = torch.empty((n, K), dtype=torch.int32, device="cuda")
    per_pair_fixed = I * H // 2 + 8 * I + 2 * H * r + 2 * I * r + 4 * H * c   # sketch, scales, map, candidates
    io = 2 * H + 8 * K + 2 * H
    dense_bytes = K * 6 * I * H + io
    ms_d, _ = timed_graph(torch, lambda i: cfm.moe_dense_forward(xe[i], ide[i], we[i], *layers[i % NL][:3],
                                                                 out=out[i], ws=wsd), n)
    rows = []
    for k in (138, 100):
        taus = [calibrate_tau(torch, cfm, layers[l], xc[l], idc[l], wc[l], k, c, r, wsc) for l in range(NL)]
        log(f"k {k}: calibrated tau per layer {[f'{t:.4g}' for t in taus]}")

        def topk(i, k=k):
            wg, wu, wd, signs, sk, A, Bt = layers[i % NL]
            cfm.moe_select_forward(xe[i], ide[i], we[i], wg, wu, wd, signs, *sk, A, Bt, k, c, r, out=out[i], ws=ws1)
        ms_k, _ = timed_graph(torch, topk, n)
        topk_frac = (K * (per_pair_fixed + 2 * H * k) + io) / dense_bytes
        for name, xs in sets.items():
            def thr(i, xs=xs, taus=taus):
                wg, wu, wd, signs, sk, A, Bt = layers[i % NL]
                cfm.moe_select_forward_threshold(xs[i], ide[i], we[i], wg, wu, wd, signs, *sk, A, Bt,
                                                 taus[i % NL], c, r, out=out[i], ws=ws1, keep_count=cnt[i])
            for i in range(n):
                thr(i)
            torch.cuda.synchronize()
            kc = cnt.cpu().numpy().astype(np.float64)
            frac = (kc.sum(1) * 2 * H + K * per_pair_fixed + io) / dense_bytes
            ms_t, _ = timed_graph(torch, thr, n)
            row = {"k": k, "budget_pct": round(100 * k / I, 1), "eval": name,
                   "kept_per_pair": {"mean": round(float(kc.mean()), 1), "min": int(kc.min()),
                                     "p10": float(np.percentile(kc, 10)), "p90": float(np.percentile(kc, 90)),
                                     "max": int(kc.max())},
                   "kept_mean_pct_of_I": round(100 * float(kc.mean()) / I, 2),
                   "read_frac_of_dense": {"mean": round(float(frac.mean()), 4), "min": round(float(frac.min()), 4),
                                          "max": round(float(frac.max()), 4)},
                   "topk_read_frac_of_dense": round(topk_frac, 4),
                   "us_per_token_threshold": round(ms_t * 1e3 / n, 3),
                   "us_per_token_topk": round(ms_k * 1e3 / n, 3),
                   "dense_us_per_token": round(ms_d * 1e3 / n, 3)}
            rows.append(row)
            log(f"threshold: {row}")
    print(json.dumps({"workload": "threshold keep rule vs top-k, Qwen3-30B-A3B-shaped layer (H 2048, E 128, top-8, "
                                  "I 768), c 276, r 64, batch 1; tau calibrated per layer on 64 synthetic tokens",
                      "data": "synthetic", "layers": NL, "eval_tokens": n, "rows": rows}), flush=True)


def olmoe(torch, cfm, args):
    """OLMoE-1B-7B-shaped layer (H 2048, E 64, top-8, I 1024, no per-channel scale), 64 tokens routed
    with Zipf(1.1) expert popularity, k 184, c 368, r 64: both passes and both dense kernels."""
    import numpy as np
    import synth
    E, K, I, H, r, T = 64, 8, 1024, 2048, 64, 64
    k, c = 184, 368
    L = 4
    layers = []
    for l in range(L):
        wg, wu, wd, signs = make_layer(torch, args.seed + 2000, l, E, I, H, chan_scale=False)
        sk = cfm.sketch_build(wg, wu, signs)
        A, Bt = cfm.lowrank_build(wd, r)
        layers.append((wg, wu, wd, signs, sk, A, Bt))
    n = args.warmup + 2 * max(10, args.steps // 4)
    xs, idss, ws_ = [], [], []
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed * 31 + 5)
    for i in range(n):
        ids, w = synth.routing(T, E, K, 3 + i, 0, zipf=1.1)
        idss.append(torch.from_numpy(ids).cuda())
        ws_.append(torch.from_numpy(w).cuda())
        z = torch.randn((T, H), generator=g, device="cuda")
        xs.append(z.to(torch.bfloat16))
    experts_used = [len(set(t.cpu().numpy().reshape(-1).tolist())) for t in idss[:8]]
    steps = max(10, args.steps // 4)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    wss = cfm.new_workspace(cfm.select_workspace(T, K, E, I, H, k, c, r), "cuda")
    wsd = cfm.new_workspace(cfm.dense_workspace(T, K, E, I, H), "cuda")

    def sel(i):
        wg, wu, wd, signs, sk, A, Bt = layers[i % L]
        cfm.moe_select_forward(xs[i], idss[i], ws_[i], wg, wu, wd, signs, *sk, A, Bt, k, c, r, out=out, ws=wss)

    def dense(i):
        wg, wu, wd, *_ = layers[i % L]
        cfm.moe_dense_forward(xs[i], idss[i], ws_[i], wg, wu, wd, out=out, ws=wsd)

    res = {}
    for name, path in (("grouped", cfm.FORWARD_GROUPED), ("per_pair", cfm.FORWARD_PER_PAIR)):
        with cfm.forward_path(path):
            for i in range(args.warmup):
                sel(i)
                dense(i)
            ms_s, _ = timed_graph(torch, lambda i: sel(args.warmup + i), steps)
            ms_d, _ = timed_graph(torch, lambda i: dense(args.warmup + steps + i), steps)
            kt, _ = kernel_times(torch, cfm, lambda i: sel(args.warmup + i), steps)
        res[name] = {"us_per_token": round(ms_s * 1e3 / (steps * T), 3),
                     "dense_us_per_token": round(ms_d * 1e3 / (steps * T), 3),
                     "kernels_us": {kn: round(v * 1e3, 2) for kn, v in kt.items()}}
        log(f"{name}: {res[name]}")
    st = torch.zeros(cfm.STATS_BYTES, dtype=torch.uint8, device="cuda")
    with cfm.forward_path(cfm.FORWARD_GROUPED):
        wg, wu, wd, signs, sk, A, Bt = layers[0]
        cfm.moe_select_forward(xs[0], idss[0], ws_[0], wg, wu, wd, signs, *sk, A, Bt, k, c, r, out=out, ws=wss,
                               stats=st)
    torch.cuda.synchronize()
    sd = cfm.decode_stats(st)
    nbytes = sum(sd[q] for q in ("bytes_sketch", "bytes_candidates", "bytes_down", "bytes_recovery", "bytes_io"))
    print(json.dumps({"workload": "OLMoE-1B-7B-shaped MoE layer (H 2048, E 64, top-8, I 1024), 64 tokens, "
                                  "Zipf(1.1) experts, k 184 c 368 r 64", "data": "synthetic",
                      "experts_used": experts_used, "grouped_bytes_per_step": nbytes,
                      "grouped_read_fraction_of_dense": round(nbytes / sd["bytes_dense_equiv"], 3),
                      "passes": res}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(expert-parallel sharding is not built).", file=sys.stderr)
        sys.exit(2)

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return

    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 3 times")
        return

    import calibration_free_channel_amd as cfm

    torch.manual_seed(args.seed)
    if args.stack:
        stack(torch, cfm, args)
        return
    if args.recovery:
        recovery_sweep(torch, cfm, args)
        return
    if args.layer_stack:
        layer_stack(torch, cfm, args)
        return
    if args.olmoe:
        olmoe(torch, cfm, args)
        return
    if args.threshold:
        threshold_study(torch, cfm, args)
        return
    if args.cold:
        cold_timing(torch, cfm, args)
        return
    if args.phase_trace:
        phase_trace(torch, cfm, args)
        return
    E, K, I, H = 128, 8, 768, 2048
    k, c, r = 138, 276, 64
    L = args.layers
    log(f"building {L} Qwen3-30B-A3B-shaped layers on the device ...")
    layers, t_sketch, t_lr = [], 0.0, 0.0
    lr_ws = torch.empty(cfm.lowrank_workspace(E, I, H, r), dtype=torch.uint8, device="cuda")
    for l in range(L):
        wg, wu, wd, signs = make_layer(torch, args.seed, l, E, I, H)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sk = cfm.sketch_build(wg, wu, signs)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        A, Bt = cfm.lowrank_build(wd, r, ws=lr_ws)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        t_sketch += t1 - t0
        t_lr += t2 - t1
        layers.append((wg, wu, wd, signs, sk, A, Bt))
    del lr_ws
    log(f"offline: sketch_build {t_sketch / L * 1e3:.1f} ms/layer, lowrank_build {t_lr / L * 1e3:.1f} ms/layer")

    results = {}
    batches = [int(b) for b in args.batches.split(",") if b]
    for T in batches:
        steps = args.steps if T == 1 else max(10, args.steps // 4)
        n_tok = args.warmup + 2 * steps
        x, ids, w = make_tokens(torch, args.seed + T, n_tok, T, E, K, H)
        ws_s = cfm.new_workspace(cfm.select_workspace(T, K, E, I, H, k, c, r), "cuda")
        ws_d = cfm.new_workspace(cfm.dense_workspace(T, K, E, I, H), "cuda")
        out = torch.empty((n_tok, T, H), dtype=torch.bfloat16, device="cuda")

        def sel(i):
            wg, wu, wd, signs, sk, A, Bt = layers[i % L]
            cfm.moe_select_forward(x[i], ids[i], w[i], wg, wu, wd, signs, *sk, A, Bt, k, c, r,
                                   out=out[i], ws=ws_s)

        def dense(i):
            wg, wu, wd, *_ = layers[i % L]
            cfm.moe_dense_forward(x[i], ids[i], w[i], wg, wu, wd, out=out[i], ws=ws_d)

        for i in range(args.warmup):            # untimed warmup steps
            sel(i)
            dense(i)
        torch.cuda.synchronize()
        off = args.warmup
        ms_sel, wall_sel = timed_graph(torch, lambda i: sel(off + i), steps)
        ms_den, wall_den = timed_graph(torch, lambda i: dense(off + steps + i), steps)
        kt_sel, launches_sel = kernel_times(torch, cfm, lambda i: sel(off + i), steps)
        kt_den, launches_den = kernel_times(torch, cfm, lambda i: dense(off + steps + i), steps)
        pp = None
        if T >= 8:
            # both passes forced on the same steps (the automatic choice is timed above)
            pp = {}
            for name, path in (("per_pair", cfm.FORWARD_PER_PAIR), ("grouped", cfm.FORWARD_GROUPED)):
                with cfm.forward_path(path):
                    for i in range(2):
                        sel(i)
                        dense(i)
                    ms_p, _ = timed_graph(torch, lambda i: sel(off + i), steps)
                    ms_pd, _ = timed_graph(torch, lambda i: dense(off + steps + i), steps)
                pp[name] = {"us_per_token": round(ms_p / steps * 1e3 / T, 3),
                            "dense_us_per_token": round(ms_pd / steps * 1e3 / T, 3)}
        # Bytes of the step's first call (every step draws from the same distribution). The
        # algorithmic bytes bill each used expert's rows once (the union over the pairs routed to it),
        # as the grouped pass reports them; the automatic pass's own stats also give the bytes its
        # kernels request (per pair on the per-pair pass).
        wg, wu, wd, signs, sk, A, Bt = layers[0]
        st = torch.zeros(cfm.STATS_BYTES, dtype=torch.uint8, device="cuda")
        cfm.moe_select_forward(x[0], ids[0], w[0], wg, wu, wd, signs, *sk, A, Bt, k, c, r,
                               out=out[0], ws=ws_s, stats=st)
        torch.cuda.synchronize()
        stats = cfm.decode_stats(st)
        if T > 1:
            stu = torch.zeros(cfm.STATS_BYTES, dtype=torch.uint8, device="cuda")
            with cfm.forward_path(cfm.FORWARD_GROUPED):
                cfm.moe_select_forward(x[0], ids[0], w[0], wg, wu, wd, signs, *sk, A, Bt, k, c, r,
                                       out=out[0], ws=ws_s, stats=stu)
            torch.cuda.synchronize()
            ustats = cfm.decode_stats(stu)
        else:
            ustats = stats
        bytes_sel = sum(ustats[f] for f in ("bytes_sketch", "bytes_candidates", "bytes_down",
                                            "bytes_recovery", "bytes_io"))
        bytes_den = ustats["bytes_dense_equiv"]
        us_step = ms_sel / steps * 1e3
        us_step_d = ms_den / steps * 1e3
        results[T] = dict(steps=steps, us_per_step=us_step, us_per_token=us_step / T,
                          gbps=bytes_sel / (us_step * 1e-6) / 1e9, bytes=bytes_sel,
                          bytes_requested=stats["bytes_requested"], experts_used=ustats["experts_used"],
                          dense_us_per_token=us_step_d / T,
                          dense_gbps=bytes_den / (us_step_d * 1e-6) / 1e9, dense_bytes=bytes_den,
                          speedup=us_step_d / us_step, kernels_us={n: v * 1e3 for n, v in kt_sel.items()},
                          launches_per_step=launches_sel, dense_launches_per_step=launches_den,
                          dense_kernels_us={n: v * 1e3 for n, v in kt_den.items()},
                          wall_ms=wall_sel, stats=stats, per_pair=pp)
        log(f"B={T}: selected {us_step:.2f} us/step ({us_step / T:.2f} us/token, "
            f"{results[T]['gbps']:.0f} GB/s on {bytes_sel / 1e6:.1f} MB), dense {us_step_d:.2f} us/step "
            f"({results[T]['dense_gbps']:.0f} GB/s), speedup {results[T]['speedup']:.2f}x; kernels "
            f"{ {n: round(v * 1e3, 2) for n, v in kt_sel.items()} } launches/step {launches_sel}; dense kernels "
            f"{ {n: round(v * 1e3, 2) for n, v in kt_den.items()} }; passes {pp}")
        del ws_s, ws_d, out, x, ids, w

    r1 = results[1] if 1 in results else results[batches[0]]     # (profiling runs may skip batch 1)
    # At batch 1 the whole hot path is one launch of k_select_fused per step, back to back in the
    # graph: its average duration is the timed region (HIP events on the launch stream) over the
    # launches in it, and its algorithmic bytes per launch are the call's bytes.
    roof = None
    one_launch = set(r1["launches_per_step"]) == {"k_select_fused"} and \
        abs(r1["launches_per_step"]["k_select_fused"] - 1.0) < 1e-9
    if one_launch:
        k_us = r1["us_per_step"]
        ach = r1["bytes"] / (k_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": "k_select_fused", "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
                "traffic": measured_traffic(), "bytes_per_launch": r1["bytes"],
                "bytes_requested_per_launch": r1["bytes_requested"], "avg_launch_us": round(k_us, 3),
                "avg_launch_us_source": "timed region / launches (HIP events on the launch stream)"}
    cold = None
    if 1 in results and args.cold_reps > 0:
        log("cold calls (1 GiB flush before each) ...")
        cold = cold_measure(torch, cfm, layers, args.cold_reps, 5, args.seed)
        log(f"cold: {cold}")
    line = {
        "metric": METRIC,
        "value": round(r1["us_per_token"], 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": r1["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(r1["us_per_step"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-30B-A3B-shaped MoE layer, batch-1 decode (H 2048, E 128, "
                               "top-8, I 768), 18% budget k=138 c=276 r=64",
                   "global_batch": 1, "layers_in_ring": L, "seed": args.seed},
        "hbm_GBps": round(r1["gbps"], 1),
        "hbm_frac": round(r1["gbps"] / PEAK_HBM_GBPS, 4),
        "bytes_per_step": r1["bytes"],
        "bytes_requested_per_step": r1["bytes_requested"],
        "dense": {"us_per_token": round(r1["dense_us_per_token"], 3),
                  "GBps": round(r1["dense_gbps"], 1), "hbm_frac": round(r1["dense_gbps"] / PEAK_HBM_GBPS, 4),
                  "bytes_per_step": r1["dense_bytes"]},
        "speedup_vs_dense": round(r1["speedup"], 3),
        "roofline": roof,
        "cold": cold,
        "kernels_us": {n: round(v, 3) for n, v in r1["kernels_us"].items()},
        "dense_kernels_us": {n: round(v, 3) for n, v in r1["dense_kernels_us"].items()},
        "batches": {str(T): {"us_per_token": round(v["us_per_token"], 3),
                             "GBps_on_expert_union_bytes": round(v["gbps"], 1),
                             "bytes_per_step": v["bytes"], "bytes_requested_per_step": v["bytes_requested"],
                             "experts_used": v["experts_used"],
                             "dense_us_per_token": round(v["dense_us_per_token"], 3),
                             "dense_bytes_per_step": v["dense_bytes"],
                             "speedup_vs_dense": round(v["speedup"], 3),
                             "kernels_us": {n: round(x, 3) for n, x in v["kernels_us"].items()},
                             "launches_per_step": {n: round(x, 3) for n, x in v["launches_per_step"].items()},
                             "passes": v["per_pair"]}
                    for T, v in results.items()},
        "offline_ms_per_layer": {"sketch_build": round(t_sketch / L * 1e3, 2),
                                 "lowrank_build": round(t_lr / L * 1e3, 2)},
        "cpu_baseline": None,
    }
    del layers
    torch.cuda.empty_cache()
    rd, cp = stream_gbps(torch)
    line["context"] = {"stream_read_GBps": round(rd, 1), "stream_copy_GBps": round(cp, 1),
                       "stream": "torch.sum over a 2 GiB float32 buffer (bytes read); torch copy of 1 GiB "
                                 "(bytes read + written)"}
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
