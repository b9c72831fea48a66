"""Benchmark of the MoE expert layer forward on one MI355X (gfx950).

Workload: the DeepSeek-V3 one-GPU expert-parallel share ("Mega MoE" page, Performance / Test
Configuration shapes: hidden 7168, intermediate 2048, 256 experts, top-8, 8192 tokens), this GPU
owning experts 0..31 and computing only the pairs that hit them.  Seeded synthetic inputs (no
dataset is involved: the pages do not state their routing; N(0,1) router logits stand in).

One step = one pass of the whole forward path on inputs already resident in HBM: routing
prologue, dispatch gather + L1 grouped GEMM + SwiGLU, L2 grouped GEMM + weighted combine.
value = algorithmic forward FLOPs (2*P*H*2I + 2*P*I*H on the P real local pairs, padding
excluded) / step time.  Prints one JSON line.

Flags: --gpus N (only 1 is supported: the path is one GPU's share), --steps K, --warmup W,
--workload NAME, --block-m BM, --no-cpu-baseline, --copy-calibration (also times a plain 1 GiB
device copy, for reading HBM counters against a kernel of known traffic), --replays N (the forward
captured into a HIP graph and replayed N times, each timed: median and min), --no-references
(skip the measured ceilings: 1 GiB copy bandwidth, the vendor library's dense bf16 GEMM rate and
its batched GEMM on a uniform stand-in of each forward GEMM).

--backward measures the training step of the wide-expert share instead (T 4096, H 7168, I 3072,
384 experts, 48 local, top-6): forward with the activations saved, L2 dgrad with the SwiGLU
transpose and the routing-weight gradient, dW2, dW1, and the L1 dgrad with its combine into dx;
one JSON line with per-stage times and each backward kernel against the HBM roofline (its
algorithmic bytes per launch / its time).  --mx measures the low-precision variant's forward (FP8
activations, FP4 weights, one power-of-two scale per 32 values along K; the "Mega MoE" page's FP8 x
FP4 example shapes: 384 experts, top-6, hidden 7168, intermediate 3072, 4096 tokens, this GPU
owning 48 experts).  The default run is the bf16 forward.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_workloads as mw  # noqa: E402
import token_dispatch_grouped_route_amd as moe  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
GEMM_SRC = os.path.join(ROOT, "token_dispatch_grouped_route_amd", "csrc", "moe_grouped.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm1_dsv3_share_traffic.json")
MX_SRC = os.path.join(ROOT, "token_dispatch_grouped_route_amd", "csrc", "moe_mx.hip")
MX_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mx_gemm1_wide_share_traffic.json")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def bf16_dev(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


# headers every GEMM source includes (the tile schedule lives in moe_tiles.h)
KERNEL_HEADERS = [os.path.join(ROOT, "token_dispatch_grouped_route_amd", "csrc", f) for f in ("moe_tiles.h", "moe_internal.h")]


def kernel_source_hash(src=GEMM_SRC):
    """First 16 hex digits of the sha256 of the kernel source followed by the headers it includes."""
    h = hashlib.sha256()
    for f in [src] + KERNEL_HEADERS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, path=TRAFFIC_FILE, src=GEMM_SRC):
    """HBM bytes per L1 launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source and on this workload; else None."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    if rec.get("workload", "dsv3_share_fwd") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration():
    """A plain copy of known size (1 GiB read, 1 GiB written), for HBM counter scaling."""
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(w, d, budget_s=20.0):
    """The oracle (test infrastructure) timed on the host cores on a bounded sample of tokens."""
    import oracle
    idx = d["topk_idx"]
    local = (idx >= w.e_lo) & (idx < w.e_lo + w.EL)
    toks = np.nonzero(local.any(axis=1))[0]
    rng = np.random.default_rng(0)
    toks = rng.permutation(toks)
    args = (d["x"], idx, d["topk_weights"], d["W1"], d["W2"])
    n = max(1, oracle.num_threads())   # calibrate on one token per thread
    t0 = time.perf_counter()
    oracle.forward(*args, E=w.E, e_lo=w.e_lo, tokens=toks[:n])
    dt = time.perf_counter() - t0
    n2 = int(min(len(toks), max(n, n * budget_s / max(dt, 1e-3))))
    sample = toks[:n2]
    t0 = time.perf_counter()
    oracle.forward(*args, E=w.E, e_lo=w.e_lo, tokens=sample)
    dt = time.perf_counter() - t0
    pairs = int(local[sample].sum())
    flops = w.flops_fwd(pairs)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d tokens (%d local pairs), fp64 per-token loop, %.1f s" % (len(sample), w.T, pairs, dt)}


def cpu_baseline_bwd(w, d, budget_s=20.0):
    """The oracle (test infrastructure) timed on the host cores on a bounded sample of the training
    step: one local expert per oracle thread (its weight-gradient loop runs one expert per thread)
    and a sample of the tokens routed to them; for those tokens the forward and the token-side
    backward (dx, d(topk_w)), and dW1, dW2 of the sampled experts over the sampled tokens' rows (the
    other routing ids set to -1, which the layer drops).  Credited with the step's algorithmic
    FLOPs of that work: forward 6, L2 dgrad 2 and L1 dgrad 4 x H x I per local pair of the tokens,
    dW2 2 and dW1 4 x H x I per kept pair."""
    import oracle
    idx, dy = d["topk_idx"], d["dy"]
    local = (idx >= w.e_lo) & (idx < w.e_lo + w.EL)
    rng = np.random.default_rng(0)
    nthr = max(1, oracle.num_threads())
    ex = rng.permutation(np.unique(idx[local] - w.e_lo))[:nthr]
    on_ex = local & np.isin(idx - w.e_lo, ex)
    toks = rng.permutation(np.nonzero(on_ex.any(axis=1))[0])
    x, tw, W1, W2 = d["x"], d["topk_weights"], d["W1"], d["W2"]

    def run(tk):
        sub = np.full_like(idx, -1)
        sub[tk] = np.where(on_ex[tk], idx[tk], -1)
        t0 = time.perf_counter()
        oracle.forward(x, idx, tw, W1, W2, E=w.E, e_lo=w.e_lo, tokens=tk)
        oracle.backward_tokens(x, idx, tw, W1, W2, dy, E=w.E, e_lo=w.e_lo, tokens=tk)
        oracle.backward(x, sub, tw, W1, W2, dy, E=w.E, e_lo=w.e_lo, experts=ex)
        return time.perf_counter() - t0

    # a run costs a + b x tokens (a: the experts' fp64 gradient arrays); calibrate on one and on
    # two tokens per thread
    n = min(len(toks), nthr)
    t1, t2 = run(toks[:n]), run(toks[:2 * n])
    per_tok = max((t2 - t1) / max(min(len(toks), 2 * n) - n, 1), 1e-6)
    fixed = max(t1 - per_tok * n, 0.0)
    n2 = int(min(len(toks), max(2 * n, (budget_s - fixed) / per_tok)))
    sample = toks[:n2]
    dt = run(sample)
    pairs, kept = int(local[sample].sum()), int(on_ex[sample].sum())
    flops = (12.0 * pairs + 6.0 * kept) * w.H * w.I
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "forward, dx, d(topk_w) of %d of %d tokens (%d local pairs); dW1, dW2 of %d of %d experts "
                      "over their %d rows among those tokens; fp64 loops, %.1f s"
                      % (len(sample), w.T, pairs, len(ex), w.EL, kept, dt)}


def stage_rates(ms, flops, nbytes):
    t = ms / 1e3
    return {"ms": round(ms, 4), "tflops": round(flops / t / 1e12, 1),
            "pct_bf16_peak": round(100 * flops / t / 1e12 / PEAK_BF16_TFLOPS, 2),
            "alg_gbs": round(nbytes / t / 1e9, 1), "pct_hbm_peak": round(100 * nbytes / t / 1e9 / PEAK_HBM_GBS, 2),
            "alg_flops": flops, "alg_bytes": nbytes}


def graph_replay_stats(fn, replays):
    """The forward captured once into a HIP graph; 10 warm-up replays, then `replays` replays each
    bracketed by events: median and min per replay."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            fn()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for e0, e1 in ev:
        e0.record(s)
        g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    return {"replays": replays, "median_ms": round(float(np.median(t)), 4), "min_ms": round(float(t.min()), 4)}


def references(w):
    """Measured ceilings on this GPU: a plain 1 GiB device copy (HBM read + write), a dense bf16
    GEMM of the vendor library (8192^3 through torch.matmul), and the vendor batched GEMM on a
    uniform stand-in of each forward GEMM (EL experts x round(P/EL) rows, no gather, no SwiGLU,
    no combine)."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3
    out = {}
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 10)
    out["copy_1gib_gbs"] = round(2 * src.numel() * 2 / t / 1e9, 1)
    del src, dst
    n = 8192
    A = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    B = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    t = timed(lambda: torch.matmul(A, B), 10)
    out["vendor_gemm_8192_tflops"] = round(2.0 * n ** 3 / t / 1e12, 1)
    del A, B
    rows = 256 if w.name == "dsv3_share_fwd" else max(32, int(round(w.T * w.k * w.EL / w.E / w.EL)))
    X = torch.randn(w.EL, rows, w.H, device="cuda").to(torch.bfloat16)
    W1 = torch.randn(w.EL, w.H, 2 * w.I, device="cuda").to(torch.bfloat16)
    t1 = timed(lambda: torch.bmm(X, W1), 10)
    del W1
    A2 = torch.randn(w.EL, rows, w.I, device="cuda").to(torch.bfloat16)
    W2 = torch.randn(w.EL, w.I, w.H, device="cuda").to(torch.bfloat16)
    t2 = timed(lambda: torch.bmm(A2, W2), 10)
    del X, A2, W2
    torch.cuda.empty_cache()
    out["vendor_bmm_l1_standin_ms"] = round(t1 * 1e3, 4)
    out["vendor_bmm_l2_standin_ms"] = round(t2 * 1e3, 4)
    out["standin_rows_per_expert"] = rows
    return out


def bench_backward(a):
    """Training step of the wide-expert share: forward (activations saved) + backward stages."""
    w = mw.get("wide_share_fwd_bwd" if a.workload == "dsv3_share_fwd" else a.workload)
    log("generating %s inputs (seed 0)" % w.name)
    d = mw.inputs(w, 0)
    P = mw.local_pairs(w, d["topk_idx"])
    bm = a.block_m or moe.preferred_block_m(moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=64))
    shape = moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=bm, e_lo=w.e_lo, train=True)
    x, dy = bf16_dev(d["x"]), bf16_dev(d["dy"])
    y = torch.empty(w.T, w.H, dtype=torch.bfloat16, device="cuda")
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    wts = torch.from_numpy(d["topk_weights"]).cuda()
    W1p, W2p = moe.alloc_packed(shape)
    W1, W2 = bf16_dev(d["W1"]), bf16_dev(d["W2"])
    moe.pack_weights(shape, W1, W2, W1p, W2p)
    del W1, W2
    ws = moe.alloc_workspace(shape)
    dW1p, dW2p = torch.empty_like(W1p), torch.empty_like(W2p)
    dx = torch.empty_like(x)
    dtw = torch.empty_like(wts)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if a.copy_calibration:
        copy_calibration()
    stages = (("forward_train", lambda: moe.forward(shape, x, idx, wts, W1p, W2p, ws, y)),
              ("dgrad_swiglu_bwd", lambda: moe.bwd_gemm2_dgrad(shape, dy, wts, W2p, ws, fuse_swiglu_bwd=True,
                                                               dtopk_w=dtw)),
              ("wgrad2", lambda: moe.wgrad2(shape, dy, ws, dW2p)),
              ("wgrad1", lambda: moe.wgrad1(shape, x, ws, dW1p)),
              ("dgrad1_combine", lambda: moe.bwd_gemm1_dgrad_combine(shape, W1p, ws, dx)))
    log("warmup %d" % a.warmup)
    for _ in range(a.warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    log("timing %d training steps" % a.steps)
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    for i in range(a.steps):
        ev[i][0].record(s)
        for j, (_, fn) in enumerate(stages):
            fn()
            ev[i][j + 1].record(s)
    torch.cuda.synchronize()
    st = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(len(stages))] for i in range(a.steps)])
    st_ms = st.mean(axis=0)
    ms = st.sum(axis=1).mean()

    idx_np = d["topk_idx"]
    local = (idx_np >= w.e_lo) & (idx_np < w.e_lo + w.EL)
    nonempty = len(np.unique(idx_np[local]))
    tok_local = int(local.any(axis=1).sum())
    H, I, EL = w.H, w.I, w.EL
    # algorithmic HBM bytes and FLOPs per launch of each backward kernel (real rows only, every
    # tensor at the method's bf16 size; the fp32 pre-activation and the hi / lo operand pairs are
    # this design's precision choice and are not counted)
    # dgrad: W2 once, dy rows of tokens with a local pair, the pre-activation read (it also gives
    # the activation for d(topk_w) and dW2's operand) and dhgu written; dgrad1: W1 once, dhgu rows
    # read, dx rows of tokens with a local pair written
    alg = {
        "dgrad_swiglu_bwd": (nonempty * H * I * 2 + tok_local * H * 2 + P * 2 * I * 2 * 2,
                             2.0 * P * H * I),
        "wgrad2": (EL * H * I * 2 + P * I * 2 + tok_local * H * 2, 2.0 * P * H * I),
        "wgrad1": (EL * 2 * I * H * 2 + P * 2 * I * 2 + tok_local * H * 2, 2.0 * P * H * 2 * I),
        "dgrad1_combine": (nonempty * 2 * I * H * 2 + P * 2 * I * 2 + tok_local * H * 2, 2.0 * P * 2 * I * H),
    }
    roof = {}
    for j, (name, _) in enumerate(stages):
        if name not in alg:
            continue
        b, f = alg[name]
        t = st_ms[j] / 1e3
        # the roof the kernel's arithmetic intensity meets first (HBM below the ridge, MFMA above)
        if f / b < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
            r = {"bound": "hbm", "achieved": b / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        else:
            r = {"bound": "mfma", "achieved": f / t / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        r.update({"frac": r["achieved"] / r["peak"], "traffic": None, "alg_bytes_per_launch": b,
                  "alg_flops_per_launch": f, "intensity_flop_per_byte": round(f / b, 1),
                  "hbm_frac": b / t / 1e9 / PEAK_HBM_GBS, "mfma_frac": f / t / 1e12 / PEAK_BF16_TFLOPS})
        roof[name] = r
    flops = w.flops_fwd(P) + sum(v[1] for v in alg.values())
    value = flops / (ms / 1e3) / 1e12
    out = {
        "metric": "MoE layer training step (fwd + L2 dgrad + SwiGLU bwd + d topk_w + dW2 + dW1 + L1 dgrad + "
                  "combine) TFLOP/s on 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) logits, x, dy, scaled weights)",
        "config": {"workload": w.name, "T": w.T, "H": H, "I": I, "E": w.E, "EL": EL, "k": w.k,
                   "block_m": bm, "local_pairs": P, "parallelism": "none (1 GPU share)"},
        "stages_ms": {name: round(st_ms[j], 4) for j, (name, _) in enumerate(stages)},
        "roofline": roof,
    }
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle, bounded sample of the training step)")
        out["cpu_baseline"] = cpu_baseline_bwd(w, d)
    print(json.dumps(out), flush=True)


PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA (the FP8 x FP4 instruction is priced at the rate of its FP8 operand)


def cpu_baseline_mx(w, d, budget_s=12.0):
    """The MX oracle timed on the host cores on a bounded sample of tokens (the oracle's FP8 / FP4
    casts of the inputs are made beforehand for the experts the sample touches, untimed)."""
    import oracle
    idx = d["topk_idx"]
    local = (idx >= w.e_lo) & (idx < w.e_lo + w.EL)
    toks = np.random.default_rng(0).permutation(np.nonzero(local.any(axis=1))[0])[:192]
    sel = idx[toks]
    experts = sorted(set((sel[(sel >= w.e_lo) & (sel < w.e_lo + w.EL)] - w.e_lo).tolist()))
    xc, xs = oracle.mx_quantize(oracle.MX_FP8, mw.bf16_bits_to_f32(d["x"]).astype(np.float64))
    codes = []
    for W in (d["W1"], d["W2"]):
        EL, K, N = W.shape
        c, sc = np.zeros((EL, N, K), np.uint8), np.zeros((EL, N, K // 32), np.uint8)
        for e in experts:
            c[e], sc[e] = oracle.mx_quantize(oracle.MX_FP4, np.ascontiguousarray(
                mw.bf16_bits_to_f32(W[e]).astype(np.float64).T))
        codes += [c, sc]
    run = lambda tk: oracle.forward_mx(xc, xs, idx, d["topk_weights"], *codes, E=w.E, e_lo=w.e_lo, tokens=tk)
    n = max(1, oracle.num_threads())
    t0 = time.perf_counter()
    run(toks[:n])
    dt = time.perf_counter() - t0
    n2 = int(min(len(toks), max(n, n * budget_s / max(dt, 1e-3))))
    sample = toks[:n2]
    t0 = time.perf_counter()
    run(sample)
    dt = time.perf_counter() - t0
    pairs = int(local[sample].sum())
    return {"value": w.flops_fwd(pairs) / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d tokens (%d local pairs), fp64 per-token loop on decoded FP8 / FP4 values, %.1f s"
                      % (len(sample), w.T, pairs, dt)}


def bench_mx(a):
    """Forward of the low-precision variant: FP8 activations, FP4 weights, block scales per 32."""
    w = mw.get("wide_share_mx_fwd" if a.workload == "dsv3_share_fwd" else a.workload)
    log("generating %s inputs (seed 0)" % w.name)
    d = mw.inputs(w, 0)
    P = mw.local_pairs(w, d["topk_idx"])
    bm = a.block_m or 64   # MX tiles follow the real 32-row groups (an expert of this share in one tile) at any block_m
    shape = moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=bm, e_lo=w.e_lo)
    x = bf16_dev(d["x"])
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    wts = torch.from_numpy(d["topk_weights"]).cuda()
    xq, xs = moe.mx_cast_fp8(x)
    w1q, w1s, w2q, w2s = moe.mx_alloc_packed(shape)
    W1, W2 = bf16_dev(d["W1"]), bf16_dev(d["W2"])
    moe.mx_pack_weights(shape, W1, W2, w1q, w1s, w2q, w2s)
    del W1, W2
    ws = moe.alloc_workspace(shape)
    y = torch.empty(w.T, w.H, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if a.copy_calibration:
        copy_calibration()
    fwd = lambda: moe.forward_mx(shape, xq, xs, idx, wts, w1q, w1s, w2q, w2s, ws, y)
    log("warmup %d" % a.warmup)
    for _ in range(a.warmup):
        fwd()
    torch.cuda.synchronize()
    log("timing %d MX forward steps" % a.steps)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(a.steps):
        fwd()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    log("timing %d staged MX steps" % a.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(a.steps)]
    for i in range(a.steps):
        ev[i][0].record(s)
        moe.route_prologue(shape, idx, ws)
        ev[i][1].record(s)
        moe.mx_dispatch_gemm1(shape, xq, xs, w1q, w1s, ws)
        ev[i][2].record(s)
        moe.mx_gemm2_combine(shape, w2q, w2s, wts, ws, y)
        ev[i][3].record(s)
        moe.mx_cast_fp8(x, xq, xs)   # not part of the step: the caller's cast of bf16 x, for reference
        ev[i][4].record(s)
    torch.cuda.synchronize()
    st = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(4)] for i in range(a.steps)])
    st_ms = st.mean(axis=0)
    graph = graph_replay_stats(fwd, a.replays) if a.replays > 0 else None

    idx_np = d["topk_idx"]
    local = (idx_np >= w.e_lo) & (idx_np < w.e_lo + w.EL)
    nonempty = len(np.unique(idx_np[local]))
    tok_local = int(local.any(axis=1).sum())
    H, I = w.H, w.I
    fp4 = lambda n, kk: n * kk // 2 + n * kk // 32          # FP4 codes + one scale byte per 32
    fp8 = lambda r, kk: r * kk + r * kk // 32
    # L1: each non-empty expert's W1 once, the FP8 x rows of tokens with a local pair once, the FP8
    # activation rows written once, the pair id of each row; L2: W2 once, the activation rows once,
    # y written once
    l1_bytes = nonempty * fp4(2 * I, H) + fp8(tok_local, H) + fp8(P, I) + P * 4
    l1_flops = 2.0 * P * H * 2 * I
    l2_bytes = nonempty * fp4(H, I) + fp8(P, I) + w.T * H * 2
    l2_flops = 2.0 * P * I * H
    l1_s = st_ms[1] / 1e3
    ridge = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if l1_flops / l1_bytes < ridge:
        roof = {"bound": "hbm", "achieved": l1_bytes / l1_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": l1_bytes / l1_s / 1e9 / PEAK_HBM_GBS}
    else:
        roof = {"bound": "mfma", "achieved": l1_flops / l1_s / 1e12, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": l1_flops / l1_s / 1e12 / PEAK_FP8_TFLOPS}
    roof.update({"traffic": measured_traffic(w.name, MX_TRAFFIC_FILE, MX_SRC),
                 "kernel": "MX gemm1 stage: x scale bytes into row order, then one launch of dispatch gather "
                           "of FP8 x + L1 + clamped SwiGLU + FP8 cast",
                 "alg_bytes_per_launch": l1_bytes, "alg_flops_per_launch": l1_flops,
                 "intensity_flop_per_byte": round(l1_flops / l1_bytes, 1),
                 "hbm_frac": l1_bytes / l1_s / 1e9 / PEAK_HBM_GBS,
                 "mfma_frac": l1_flops / l1_s / 1e12 / PEAK_FP8_TFLOPS})
    rates = lambda ms_, f, b: {"ms": round(ms_, 4), "tflops": round(f / (ms_ / 1e3) / 1e12, 1),
                               "alg_gbs": round(b / (ms_ / 1e3) / 1e9, 1),
                               "pct_hbm_peak": round(100 * b / (ms_ / 1e3) / 1e9 / PEAK_HBM_GBS, 2),
                               "alg_flops": f, "alg_bytes": b}
    value = w.flops_fwd(P) / (ms / 1e3) / 1e12
    out = {
        "metric": "MoE layer fwd, FP8 activations x FP4 weights (block scales per 32), TFLOP/s on 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 -> fp32", "data": "synthetic (seeded N(0,1) logits, x, scaled weights)",
        "config": {"workload": w.name, "T": w.T, "H": H, "I": I, "E": w.E, "EL": w.EL, "k": w.k,
                   "block_m": bm, "local_pairs": P, "clamp": 10.0, "parallelism": "none (1 GPU share)"},
        "stages_ms": {"prologue": round(st_ms[0], 4), "mx_dispatch_gemm1": round(st_ms[1], 4),
                      "mx_gemm2_combine": round(st_ms[2], 4), "staged_total": round(st_ms[:3].sum(), 4),
                      "x_cast_fp8_not_in_step": round(st_ms[3], 4)},
        "stages": {"mx_dispatch_gemm1": rates(st_ms[1], l1_flops, l1_bytes),
                   "mx_gemm2_combine": rates(st_ms[2], l2_flops, l2_bytes)},
        "roofline": roof,
    }
    if graph:
        out["graph_replay"] = graph
    if not a.no_cpu_baseline:
        log("timing the MX oracle on a CPU sample")
        out["cpu_baseline"] = cpu_baseline_mx(w, d)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3_share_fwd")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--backward", action="store_true")
    ap.add_argument("--mx", action="store_true", help="the FP8 x FP4 variant's forward")
    ap.add_argument("--replays", type=int, default=100, help="graph replays timed one by one (0: skip)")
    ap.add_argument("--no-references", action="store_true", help="skip the copy / vendor-GEMM references")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the experts; runs on more than one GPU are not "
              "part of this path (cross-GPU dispatch/combine is out of scope). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    torch.cuda.set_device(0)
    if a.backward:
        return bench_backward(a)
    if a.mx:
        return bench_mx(a)
    w = mw.get(a.workload)
    log("generating %s inputs (seed 0)" % w.name)
    d = mw.inputs(w, 0)
    P = mw.local_pairs(w, d["topk_idx"])
    flops = w.flops_fwd(P)
    bm = a.block_m or moe.preferred_block_m(moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=64))
    shape = moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=bm, e_lo=w.e_lo)

    x, y = bf16_dev(d["x"]), torch.empty(w.T, w.H, dtype=torch.bfloat16, device="cuda")
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    wts = torch.from_numpy(d["topk_weights"]).cuda()
    W1p, W2p = moe.alloc_packed(shape)
    W1, W2 = bf16_dev(d["W1"]), bf16_dev(d["W2"])
    moe.pack_weights(shape, W1, W2, W1p, W2p)
    del W1, W2
    ws = moe.alloc_workspace(shape)
    act = moe.ws_region(ws, shape, "act")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    if a.copy_calibration:
        copy_calibration()

    # the measured ceilings run first: besides their own figures they bring the GPU to the clock a
    # busy serving loop runs at (the shader clock ramps up over the first ~40 ms of work)
    refs = None
    if not a.no_references:
        log("measuring the copy and vendor-GEMM references")
        refs = references(w)

    fwd = lambda: moe.forward(shape, x, idx, wts, W1p, W2p, ws, y)
    log("warmup %d" % a.warmup)
    for _ in range(a.warmup):
        fwd()
    torch.cuda.synchronize()

    # headline: K fused forwards
    log("timing %d fused forward steps" % a.steps)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(a.steps):
        fwd()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps

    # per stage: the same kernels through the stage entry points, events between stages
    log("timing %d staged steps" % a.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    for i in range(a.steps):
        ev[i][0].record(s)
        moe.route_prologue(shape, idx, ws)
        ev[i][1].record(s)
        moe.dispatch_gemm1(shape, x, W1p, ws, act_out=act)
        ev[i][2].record(s)
        moe.gemm2_combine(shape, act, W2p, wts, ws, y)
        ev[i][3].record(s)
    torch.cuda.synchronize()
    st = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(3)] for i in range(a.steps)])
    st_ms = st.mean(axis=0)

    graph = graph_replay_stats(fwd, a.replays) if a.replays > 0 else None

    R = int(moe.ws_region(ws, shape, "meta")[0].item())
    # algorithmic bytes of the L1 launch: each non-empty local expert's W1 once, the x rows of
    # tokens with a local pair once, the SwiGLU output rows written once, the pair ids of the rows
    idx_np = d["topk_idx"]
    local = (idx_np >= w.e_lo) & (idx_np < w.e_lo + w.EL)
    nonempty = len(np.unique(idx_np[local]))
    tok_local = int(local.any(axis=1).sum())
    l1_flops = 2.0 * P * w.H * 2 * w.I
    l1_bytes = nonempty * 2 * w.I * w.H * 2 + tok_local * w.H * 2 + P * w.I * 2 + P * 4
    l1_s = st_ms[1] / 1e3
    traffic = measured_traffic(w.name)
    # the bound is the roof the kernel's arithmetic intensity (algorithmic FLOP per algorithmic
    # byte) meets first: HBM below the ridge (peak FLOP/s / peak B/s), MFMA above it
    if l1_flops / l1_bytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": l1_bytes / l1_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": l1_bytes / l1_s / 1e9 / PEAK_HBM_GBS}
    else:
        roof = {"bound": "mfma", "achieved": l1_flops / l1_s / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": l1_flops / l1_s / 1e12 / PEAK_BF16_TFLOPS}
    roof.update({"traffic": traffic, "kernel": "gemm1 (dispatch gather + L1 NT + SwiGLU)",
                 "alg_bytes_per_launch": l1_bytes, "alg_flops_per_launch": l1_flops,
                 "intensity_flop_per_byte": round(l1_flops / l1_bytes, 1),
                 "hbm_frac": l1_bytes / l1_s / 1e9 / PEAK_HBM_GBS,
                 "mfma_frac": l1_flops / l1_s / 1e12 / PEAK_BF16_TFLOPS})

    # per stage: algorithmic FLOPs and bytes (real rows only) over the event-timed stage; L2 +
    # combine must read each non-empty expert's W2 and the act rows once and write y once (the fp32
    # staging of multi-pair tokens is this design's, not the method's, so it is not counted)
    l2_flops = 2.0 * P * w.I * w.H
    l2_bytes = nonempty * w.H * w.I * 2 + P * w.I * 2 + w.T * w.H * 2
    stages = {"prologue": {"ms": round(st_ms[0], 4), "alg_bytes": w.T * w.k * 4},
              "dispatch_gemm1_swiglu": stage_rates(st_ms[1], l1_flops, l1_bytes),
              "gemm2_combine": stage_rates(st_ms[2], l2_flops, l2_bytes)}

    value = flops / (ms / 1e3) / 1e12
    out = {
        "metric": "MoE layer fwd TFLOP/s on 1 MI355X (% of bf16 MFMA peak); per-stage ms",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) logits, x, scaled weights)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "EL": w.EL, "k": w.k,
                   "block_m": bm, "local_pairs": P, "padded_rows": R, "parallelism": "none (1 GPU share)"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "stages_ms": {"prologue": round(st_ms[0], 4), "dispatch_gemm1_swiglu": round(st_ms[1], 4),
                      "gemm2_combine": round(st_ms[2], 4), "staged_total": round(st_ms.sum(), 4)},
        "stages": stages,
        "roofline": roof,
    }
    if graph:
        out["graph_replay"] = graph
    if refs is not None:
        out["references"] = refs
    if not a.no_cpu_baseline:
        log("timing the oracle on a CPU sample")
        out["cpu_baseline"] = cpu_baseline(w, d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
