"""GPU parity of the forward path against the CPU oracle, through the C ABI.

Routing tables must match bit for bit (including the -1 fills); every floating-point output
must satisfy |gpu - oracle| <= 2e-2 * rms(oracle) + (the element's own rounding to bf16, half
an ulp) for every element, rms over the compared array (check_bf16).  Sizes:
reduced shapes that span several tiles with ragged per-expert tails are compared in full; the
five workloads at their full sizes are compared on sampled tokens (tokens with zero, one and
several local pairs), plus properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import token_dispatch_grouped_route_amd as moe
from gpu_helpers import (assert_tables_equal, bits_host, check_bf16, check_f32, f64_host, layer,
                         sample_tokens, tables)

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def route_only(w, idx, bm):
    d = {"topk_idx": idx, "topk_weights": np.ones(idx.shape, np.float32),
         "x": np.zeros((w.T, w.H), np.uint16)}
    ns = layer(w, d, bm, weights=False)
    moe.route_prologue(ns.shape, ns.idx, ns.ws)
    torch.cuda.synchronize()
    return tables(ns)


# ------------------------------------------------------------------------------------------
# Routing prologue
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("bm", [32, 64, 128, 256])
def test_route_tables_bit_exact(cfg, bm):
    w = mw.get(cfg)
    idx, _ = mw.routing(w, 0)
    got = route_only(w, idx, bm)
    assert_tables_equal(got, oracle.route(idx, w.E, w.e_lo, w.EL, bm))


@pytest.mark.parametrize("case", ["empty", "none_local", "all_dropped", "k1", "dups", "shard",
                                  "one_expert", "many_experts", "ragged_chunks", "many_chunks"])
def test_route_edge_cases(case):
    rng = np.random.default_rng(21)
    T, E, EL, e_lo, k = 300, 16, 4, 0, 3
    if case == "empty":
        T = 0
    elif case == "shard":
        e_lo = 12
    elif case == "one_expert":
        EL = 1
    elif case == "many_experts":
        T, E, EL, k = 700, 2048, 1024, 8
    elif case == "ragged_chunks":
        T, E, EL, k = 5000, 64, 48, 7      # pair chunks of 2048 split tokens
    elif case == "many_chunks":
        T, E, EL, k = 40000, 256, 64, 8    # chunk histograms too large for one block's LDS
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if case == "none_local":
        idx = rng.integers(EL, E, size=(T, k)).astype(np.int32)
    elif case == "all_dropped":
        idx = rng.integers(E, 3 * E, size=(T, k)).astype(np.int32)
        idx[::2] = -idx[::2]
    elif case == "k1":
        k = 1
        idx = rng.integers(0, EL, size=(T, 1)).astype(np.int32)
    elif case == "dups":
        idx[:, 1] = idx[:, 0] % EL
        idx[:, 2] = idx[:, 0] % EL
    w = mw.Workload("edge", T=T, H=128, I=128, E=E, EL=EL, k=k, e_lo=e_lo)
    for bm in (32, 64, 256):
        got = route_only(w, idx, bm)
        assert_tables_equal(got, oracle.route(idx, E, e_lo, EL, bm))


def test_route_is_deterministic():
    w = mw.get(3)
    idx, _ = mw.routing(w, 0)
    a = route_only(w, idx, 128)
    b = route_only(w, idx, 128)
    assert_tables_equal(a, b)


# ------------------------------------------------------------------------------------------
# Forward on reduced shapes, compared in full
# ------------------------------------------------------------------------------------------
REDUCED = [
    # several M tiles per expert, ragged tails, a shard with e_lo > 0 and non-local pairs; the
    # N sizes select every forward tile width (L1 2I % 512 or only % 256, L2 H % 512, % 256, % 128)
    mw.Workload("reduced_shard", T=333, H=384, I=384, E=12, EL=6, k=3, e_lo=3),
    mw.Workload("reduced_all_local", T=500, H=256, I=128, E=8, EL=8, k=4),
    mw.Workload("reduced_k1", T=200, H=128, I=128, E=4, EL=4, k=1),
    mw.Workload("reduced_wide", T=700, H=512, I=256, E=10, EL=5, k=2),
]


@pytest.mark.parametrize("bm", [32, 64, 128, 256])
@pytest.mark.parametrize("w", REDUCED, ids=[r.name for r in REDUCED])
def test_forward_reduced_full_compare(w, bm):
    d = mw.inputs(w, 3)
    ns = layer(w, d, bm)
    moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
    torch.cuda.synchronize()
    assert_tables_equal(tables(ns), oracle.route(d["topk_idx"], w.E, w.e_lo, w.EL, bm))
    ref = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
    got = f64_host(ns.y)
    assert np.all(np.isfinite(got))
    check_bf16(got, ref, TOL, "y (%s, bm %d)" % (w.name, bm))
    nloc = tables(ns)["tok_nloc"]
    assert np.all(got[nloc == 0] == 0.0)


# Experts of 9 and 18 groups of 32 rows (one and two M tiles of nine groups in the L1 tile that
# takes nine, the ninth group's MFMAs in VGPR form) next to experts of 7-13 and 26 groups (tiles
# of 5-8 groups).  H = 640: a K loop with a tail slot and 128-column L2 tiles.
NINE = mw.Workload("reduced_nine", T=1500, H=640, I=256, E=8, EL=8, k=2, zipf_s=0.6)


def nine_group_tiles(counts):
    """M tiles of nine 32-row groups: an expert of g <= 18 groups is cut into ceil(g / 9) tiles,
    a larger one into ceil(g / 8), the group counts of its tiles differing by at most one."""
    g = -(-np.asarray(counts) // 32)
    tiles = np.where(g <= 18, -(-g // 9), -(-g // 8))
    base, rem = g // np.maximum(tiles, 1), g % np.maximum(tiles, 1)
    return int(np.sum(np.where(base == 9, tiles, np.where(base == 8, rem, 0))))


@pytest.mark.parametrize("bm", [32, 128])
def test_forward_nine_group_tiles(bm):
    d = mw.inputs(NINE, 5)
    assert NINE.T * NINE.k <= 512 * NINE.E   # the launch that uses nine-group tiles
    counts = np.bincount(d["topk_idx"].ravel(), minlength=NINE.E)
    assert nine_group_tiles(counts) >= 3, counts
    ns = layer(NINE, d, bm)
    s = ns.shape
    R = moe.workspace_layout(s)["rows_capacity"]
    hgu = torch.zeros(R, 2 * NINE.I, dtype=torch.float32, device="cuda")
    act = torch.zeros(R, NINE.I, dtype=torch.bfloat16, device="cuda")
    moe.route_prologue(s, ns.idx, ns.ws)
    moe.dispatch_gemm1(s, ns.x, ns.W1p, ns.ws, act_out=act, hgu_out=hgu)
    moe.forward(s, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
    torch.cuda.synchronize()
    t = tables(ns)
    real = np.nonzero(t["row_pair"] >= 0)[0]
    h_ref, a_ref = oracle.l1_rows(d["x"], d["topk_idx"], d["W1"], NINE.E, NINE.e_lo, t["row_pair"][real])
    check_f32(f64_host(hgu)[real], h_ref, TOL, "hgu (nine-group tiles, bm %d)" % bm)
    check_bf16(f64_host(act)[real], a_ref, TOL, "act (nine-group tiles, bm %d)" % bm)
    pad = np.setdiff1d(np.arange(t["num_rows"]), real)
    assert np.all(f64_host(act)[pad] == 0.0) and np.all(f64_host(hgu)[pad] == 0.0)
    ref = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=NINE.E)
    check_bf16(f64_host(ns.y), ref, TOL, "y (nine-group tiles, bm %d)" % bm)


def test_forward_tiny_workload_full_compare():
    w = mw.get(0)
    d = mw.inputs(w, 0)
    for bm in (64, 128):
        ns = layer(w, d, bm)
        moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
        torch.cuda.synchronize()
        ref = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E)
        check_bf16(f64_host(ns.y), ref, TOL, "y (%s, bm %d)" % (w.name, bm))


def packed_reference(W, I=None):
    """The packed layout as include/moe.h states it: logical [EL, K, N] -> [EL, N * K] with
    element (n, k) at ((n / 32) * (K / 16) + k / 16) * 512 + ((k / 8) % 2 * 32 + n % 32) * 8
    + k % 8, where for W1 (I given) logical column c becomes packed column
    ((c mod I) / 32) * 64 + (c >= I) * 32 + c mod 32."""
    EL, K, N = W.shape
    c = np.arange(N)
    n = (c % I) // 32 * 64 + (c >= I) * 32 + c % 32 if I is not None else c
    k = np.arange(K)[:, None]
    pos = ((n[None, :] // 32) * (K // 16) + k // 16) * 512 + ((k // 8) % 2 * 32 + n[None, :] % 32) * 8 + k % 8
    assert np.array_equal(np.sort(pos.reshape(-1)), np.arange(N * K))
    out = np.empty((EL, N * K), np.uint16)
    out[:, pos.reshape(-1)] = W.reshape(EL, -1)
    return out


@pytest.mark.parametrize("w", [REDUCED[0], REDUCED[3]], ids=["shard", "wide"])
def test_pack_weights_follows_the_documented_layout(w):
    d = mw.inputs(w, 4)
    ns = layer(w, d, 64)
    assert tuple(ns.W1p.shape) == (w.EL, 2 * w.I * w.H) and tuple(ns.W2p.shape) == (w.EL, w.H * w.I)
    assert np.array_equal(bits_host(ns.W1p), packed_reference(d["W1"], w.I))
    assert np.array_equal(bits_host(ns.W2p), packed_reference(d["W2"]))
    W1, W2 = torch.empty(w.EL, w.H, 2 * w.I, dtype=torch.bfloat16, device="cuda"), \
        torch.empty(w.EL, w.I, w.H, dtype=torch.bfloat16, device="cuda")
    moe.unpack_weights(ns.shape, ns.W1p, ns.W2p, W1, W2)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(W1), d["W1"]) and np.array_equal(bits_host(W2), d["W2"])


def test_stages_match_oracle_and_fused_forward():
    """prologue -> dispatch_gemm1 (fp32 pre-activation and SwiGLU outputs) -> standalone SwiGLU ->
    gemm2_combine, each compared with the oracle; staging the fused-SwiGLU output through
    gemm2_combine reproduces the fused forward's y bit for bit."""
    w = REDUCED[0]
    d = mw.inputs(w, 5)
    bm = 64
    ns = layer(w, d, bm)
    s = ns.shape
    R = moe.workspace_layout(s)["rows_capacity"]
    hgu = torch.zeros(R, 2 * w.I, dtype=torch.float32, device="cuda")
    act = torch.zeros(R, w.I, dtype=torch.bfloat16, device="cuda")
    act2 = torch.zeros(R, w.I, dtype=torch.bfloat16, device="cuda")
    moe.route_prologue(s, ns.idx, ns.ws)
    moe.dispatch_gemm1(s, ns.x, ns.W1p, ns.ws, act_out=act, hgu_out=hgu)
    moe.swiglu(s, hgu, ns.ws, act2)
    y_staged = torch.empty_like(ns.y)
    moe.gemm2_combine(s, act2, ns.W2p, ns.wts, ns.ws, y_staged)
    y_fused_act = torch.empty_like(ns.y)
    moe.gemm2_combine(s, act, ns.W2p, ns.wts, ns.ws, y_fused_act)
    moe.forward(s, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
    torch.cuda.synchronize()
    assert torch.equal(y_fused_act, ns.y)

    t = tables(ns)
    real = np.nonzero(t["row_pair"] >= 0)[0]
    pairs = t["row_pair"][real]
    h_ref, a_ref = oracle.l1_rows(d["x"], d["topk_idx"], d["W1"], w.E, w.e_lo, pairs)
    check_f32(f64_host(hgu)[real], h_ref, TOL, "hgu (L1, fp32)")
    check_bf16(f64_host(act)[real], a_ref, TOL, "act (fused SwiGLU)")
    # the standalone SwiGLU on the GPU's own fp32 pre-activations
    hv = f64_host(hgu)[:t["num_rows"]]
    check_bf16(f64_host(act2)[:t["num_rows"]], oracle.swiglu(hv), TOL, "act (standalone SwiGLU)")
    # padding rows inside segments carry zeros
    pad = np.setdiff1d(np.arange(t["num_rows"]), real)
    assert np.all(f64_host(act)[pad] == 0.0) and np.all(f64_host(hgu)[pad] == 0.0)
    ref = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
    check_bf16(f64_host(ns.y), ref, TOL, "y (fused)")
    check_bf16(f64_host(y_staged), ref, TOL, "y (staged)")


def test_forward_is_deterministic_and_graph_capturable():
    w = REDUCED[1]
    d = mw.inputs(w, 6)
    ns = layer(w, d, 64)
    args = (ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws)
    y0 = torch.empty_like(ns.y)
    moe.forward(*args, y0)
    moe.forward(*args, ns.y)
    torch.cuda.synchronize()
    assert torch.equal(y0, ns.y)

    yg = torch.full_like(ns.y, float("nan"))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        moe.forward(*args, yg)   # warm up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            moe.forward(*args, yg)
    torch.cuda.current_stream().wait_stream(stream)
    for i in range(3):
        yg.fill_(float("nan"))
        ns.ws.fill_(0x7f)        # stale workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0), "replay %d differs" % i
        moe.forward(*args, ns.y)  # eager work between replays
        torch.cuda.synchronize()


def test_dropped_ids_are_counted_and_ignored():
    w = REDUCED[0]
    d = mw.inputs(w, 7)
    idx = d["topk_idx"].copy()
    idx[::5, 0] = w.E + 3
    idx[1::7, 1] = -2
    d2 = dict(d, topk_idx=idx)
    ns = layer(w, d2, 64)
    moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
    torch.cuda.synchronize()
    t = tables(ns)
    assert t["dropped"] == int(np.sum((idx < 0) | (idx >= w.E)))
    ref = oracle.forward(d["x"], idx, d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
    check_bf16(f64_host(ns.y), ref, TOL, "y (dropped ids)")


def test_errors_are_reported_before_launch():
    w = REDUCED[0]
    d = mw.inputs(w, 8)
    ns = layer(w, d, 64)
    with pytest.raises(moe.MoeError, match="workspace"):
        moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws[:1024], ns.y)
    with pytest.raises(moe.MoeError, match="misaligned"):
        xs = torch.empty(ns.x.numel() + 8, dtype=torch.bfloat16, device="cuda")[1:1 + ns.x.numel()]
        moe.forward(ns.shape, xs.view_as(ns.x), ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
    with pytest.raises(moe.MoeError, match="train"):
        moe.swiglu_bwd(ns.shape, ns.ws)


# ------------------------------------------------------------------------------------------
# Full-size workloads, sampled tokens
# ------------------------------------------------------------------------------------------
_FULL = {}


def full_inputs(cfg):
    if cfg not in _FULL:
        _FULL.clear()
        w = mw.get(cfg)
        _FULL[cfg] = (w, mw.inputs(w, 0))
    return _FULL[cfg]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_forward_full_size_sampled(cfg):
    w, d = full_inputs(cfg)
    bm = moe.preferred_block_m(moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=64))
    ns = layer(w, d, bm)
    moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
    torch.cuda.synchronize()
    t = tables(ns)
    assert_tables_equal(t, oracle.route(d["topk_idx"], w.E, w.e_lo, w.EL, bm))
    y = f64_host(ns.y)
    assert np.all(np.isfinite(y))
    assert np.all(y[t["tok_nloc"] == 0] == 0.0)
    tok = sample_tokens(t["tok_nloc"], 48, seed=cfg)
    ref = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo,
                         tokens=tok)
    check_bf16(y[tok], ref, TOL, "y (%s, bm %d, %d sampled tokens)" % (w.name, bm, len(tok)))
