"""GPU parity of the backward stages against the CPU oracle, through the C ABI.

Covers L2 dgrad (NN) with and without the SwiGLU transpose in its epilogue, the gradient of
the routing weights, the standalone SwiGLU backward, dW2 and dW1 with a variable K (rows per
expert, including experts without rows, whose gradients must be exact zeros) and the L1 dgrad
(NN) with its combine back to token order (dx).

Acceptance is the forward's: every bf16 output (dW1, dW2, dx, the dhgu rows) within 2e-2 * rms of
the oracle plus the element's own rounding to bf16 (check_bf16); every fp32 output or hi + lo
pair (d(topk_w), dact, the saved pre-activation, the weighted activation) within 2e-2 * rms
(check_f32).  The oracle computes in fp64 from the bf16 inputs.  Row intermediates are also
checked link by link: dhgu against the oracle's SwiGLU transpose evaluated on the GPU's own saved
pre-activation and dact.  Tokens with no local pair (dx) and pairs this GPU does not handle
(d(topk_w)) must be exact zeros.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import token_dispatch_grouped_route_amd as moe
from gpu_helpers import check_bf16, check_f32, f64_host, layer, tables, unpacked

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


REDUCED = [
    mw.Workload("wide_reduced", T=64, H=256, I=128, E=48, EL=6, k=6, backward=True),
    mw.Workload("bwd_ragged_shard", T=301, H=384, I=256, E=10, EL=5, k=3, e_lo=2, backward=True),
    # about 256 rows per expert: the weight gradients run on the forward pipeline (block_m >= 64)
    mw.Workload("bwd_many_rows", T=1024, H=512, I=256, E=8, EL=4, k=2, e_lo=2, backward=True),
    # about 512 rows per expert and EL * H <= R_max: the L1 dgrad also runs as the forward's L2
    mw.Workload("bwd_many_rows_narrow", T=2048, H=256, I=128, E=8, EL=4, k=2, e_lo=2, backward=True),
]


def with_empty_expert(w, d):
    """Routing where local expert 1 receives no pair (its ids move to local expert 0)."""
    idx = d["topk_idx"].copy()
    idx[idx == w.e_lo + 1] = w.e_lo
    return dict(d, topk_idx=idx)


def run_forward_backward(w, d, bm):
    ns = layer(w, d, bm, train=True)
    moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
    s1, s2 = moe.packed_sizes(ns.shape)
    ns.dW1p = torch.full(s1, float("nan"), dtype=torch.bfloat16, device="cuda")
    ns.dW2p = torch.full(s2, float("nan"), dtype=torch.bfloat16, device="cuda")
    ns.dx = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ns.dtw = torch.full((w.T, w.k), float("nan"), dtype=torch.float32, device="cuda")
    moe.backward(ns.shape, ns.x, ns.dy, ns.wts, ns.W2p, ns.ws, ns.dW1p, ns.dW2p, w1p=ns.W1p, dx=ns.dx,
                 dtopk_w=ns.dtw)
    torch.cuda.synchronize()
    return ns


def check_token_grads(w, d, ns, tokens, what):
    args = (d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dx_ref, dw_ref = oracle.backward_tokens(*args, E=w.E, e_lo=w.e_lo, tokens=tokens)
    dx = f64_host(ns.dx)[tokens]
    dw = ns.dtw.cpu().double().numpy()[tokens]
    check_bf16(dx, dx_ref, TOL, "dx " + what)
    check_f32(dw, dw_ref, TOL, "d(topk_w) " + what)
    local = (d["topk_idx"] >= w.e_lo) & (d["topk_idx"] < w.e_lo + w.EL)
    assert np.all(dw[~local[tokens]] == 0.0), "pairs this GPU does not handle must get exact zeros"
    assert np.all(dx[~local[tokens].any(axis=1)] == 0.0), "tokens with no local pair must get exact zeros"


def oracle_rows(w, d, pairs):
    args = (d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dA, dH = oracle.backward_rows(*args, E=w.E, e_lo=w.e_lo, pairs=pairs)
    h, a = oracle.l1_rows(d["x"], d["topk_idx"], d["W1"], w.E, w.e_lo, pairs)
    return dA, dH, h, a


def ws_f64(ns, name, rows=None):
    v = f64_host(moe.ws_region(ns.ws, ns.shape, name))
    return v if rows is None else v[rows]


def check_row_links(w, d, ns, rows, what):
    """Row intermediates of the given ws rows: the saved fp32 pre-activation against the oracle's
    L1 rows; the weighted activation (hi + lo) against w * SwiGLU of that pre-activation; dhgu (hi,
    and hi + lo) against the oracle's SwiGLU transpose of the oracle's dA on the GPU's own saved
    pre-activation."""
    pairs = tables(ns)["row_pair"][rows]
    dA, _, h_ref, _ = oracle_rows(w, d, pairs)
    hgu = ws_f64(ns, "hgu", rows)
    check_f32(hgu, h_ref, TOL, "hgu " + what)
    wts = d["topk_weights"].reshape(-1)[pairs].astype(np.float64)[:, None]
    wact = ws_f64(ns, "wact", rows) + ws_f64(ns, "wact_lo", rows)
    check_f32(wact, wts * oracle.swiglu(hgu), TOL, "w*act (hi+lo) " + what)
    ref = oracle.swiglu_bwd(hgu, dA)
    check_bf16(ws_f64(ns, "dhgu", rows), ref, TOL, "dhgu " + what)
    check_f32(ws_f64(ns, "dhgu", rows) + ws_f64(ns, "dhgu_lo", rows), ref, TOL, "dhgu (hi+lo) " + what)


def pairs_of_expert(tab):
    def rows_of(e):
        o, c = tab["padded_offsets"][e], tab["counts"][e]
        return tab["row_pair"][o:o + c].astype(np.int64)
    return rows_of


@pytest.mark.parametrize("bm", [32, 64, 128, 256])
@pytest.mark.parametrize("w", REDUCED, ids=[r.name for r in REDUCED])
def test_backward_reduced_full_compare(w, bm):
    d = with_empty_expert(w, mw.inputs(w, 9))
    ns = run_forward_backward(w, d, bm)
    t = tables(ns)
    args = (d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dW1, dW2 = oracle.backward(*args, E=w.E, e_lo=w.e_lo)
    g1, g2 = unpacked(ns, ns.dW1p, ns.dW2p)
    tag = "(%s, bm %d)" % (w.name, bm)
    check_bf16(g1, dW1, TOL, "dW1 " + tag)
    check_bf16(g2, dW2, TOL, "dW2 " + tag)
    assert np.all(g1[1] == 0.0) and np.all(g2[1] == 0.0), "expert without rows must get exact zeros"
    real = np.nonzero(t["row_pair"] >= 0)[0]
    check_row_links(w, d, ns, real, tag)
    check_token_grads(w, d, ns, np.arange(w.T), tag)


def test_backward_token_grads_edge_routing():
    """Dropped ids, a duplicated expert in one token, tokens with no local pair and tokens whose
    only local pair is the single one (direct store) next to multi-pair tokens (staged sum)."""
    w = REDUCED[1]
    d = mw.inputs(w, 12)
    idx = d["topk_idx"].copy()
    idx[0] = [w.E + 3, -1, w.E]                  # all dropped
    idx[1] = [w.e_lo, w.e_lo, w.e_lo]            # one expert three times
    idx[2] = [0, 1, w.e_lo + w.EL]               # none local (shard starts at e_lo = 2)
    idx[3] = [w.e_lo + 1, w.E + 1, w.E - 1]      # one local pair, one dropped, one remote
    d = dict(d, topk_idx=idx)
    ns = run_forward_backward(w, d, 64)
    check_token_grads(w, d, ns, np.arange(w.T), "(edge routing)")
    assert np.all(f64_host(ns.dx)[[0, 2]] == 0.0)


def test_backward_is_deterministic():
    w = REDUCED[1]
    d = mw.inputs(w, 13)
    a = run_forward_backward(w, d, 64)
    b = run_forward_backward(w, d, 64)
    for n in ("dx", "dtw", "dW1p", "dW2p"):
        assert torch.equal(getattr(a, n).view(torch.int16) if getattr(a, n).dtype == torch.bfloat16
                           else getattr(a, n).view(torch.int32),
                           getattr(b, n).view(torch.int16) if getattr(b, n).dtype == torch.bfloat16
                           else getattr(b, n).view(torch.int32)), n


def test_backward_stages_match_oracle_and_fused():
    w = REDUCED[1]
    d = mw.inputs(w, 10)
    bm = 64
    ns = run_forward_backward(w, d, bm)
    s = ns.shape
    t = tables(ns)
    real = np.nonzero(t["row_pair"] >= 0)[0]
    dA, _, _, _ = oracle_rows(w, d, t["row_pair"][real])
    wact_fused = moe.ws_region(ns.ws, s, "wact").clone(), moe.ws_region(ns.ws, s, "wact_lo").clone()

    dtw = torch.full_like(ns.dtw, float("nan"))
    moe.bwd_gemm2_dgrad(s, ns.dy, ns.wts, ns.W2p, ns.ws, fuse_swiglu_bwd=False, dtopk_w=dtw)
    torch.cuda.synchronize()
    assert torch.equal(dtw, ns.dtw), "d(topk_w) does not depend on the SwiGLU-transpose path"
    assert torch.equal(moe.ws_region(ns.ws, s, "wact"), wact_fused[0])
    assert torch.equal(moe.ws_region(ns.ws, s, "wact_lo"), wact_fused[1])
    dact = ws_f64(ns, "dact")
    check_f32(dact[real], dA, TOL, "dact (L2 dgrad)")
    pad = np.setdiff1d(np.arange(t["num_rows"]), real)
    assert np.all(dact[pad] == 0.0)

    moe.swiglu_bwd(s, ns.ws)
    torch.cuda.synchronize()
    hgu = ws_f64(ns, "hgu")
    ref_local = oracle.swiglu_bwd(hgu[real], dact[real])
    check_bf16(ws_f64(ns, "dhgu")[real], ref_local, TOL, "swiglu_bwd (standalone)")
    check_f32(ws_f64(ns, "dhgu")[real] + ws_f64(ns, "dhgu_lo")[real], ref_local, TOL,
              "swiglu_bwd (standalone, hi+lo)")
    assert np.all(ws_f64(ns, "dhgu")[pad] == 0.0)

    dW1p = torch.empty_like(ns.dW1p)
    dW2p = torch.empty_like(ns.dW2p)
    moe.wgrad2(s, ns.dy, ns.ws, dW2p)
    moe.wgrad1(s, ns.x, ns.ws, dW1p)
    torch.cuda.synchronize()
    assert torch.equal(dW2p, ns.dW2p), "dW2 does not depend on the SwiGLU-transpose path"
    args = (d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dW1, dW2 = oracle.backward(*args, E=w.E, e_lo=w.e_lo)
    g1, g2 = unpacked(ns, dW1p, dW2p)
    check_bf16(g1, dW1, TOL, "dW1 (staged)")
    check_bf16(g2, dW2, TOL, "dW2 (staged)")

    # L1 dgrad + combine on the standalone SwiGLU transpose's dhgu
    ns.dx = torch.full_like(ns.dx, float("nan"))
    ns.dtw = dtw
    moe.bwd_gemm1_dgrad_combine(s, ns.W1p, ns.ws, ns.dx)
    torch.cuda.synchronize()
    check_token_grads(w, d, ns, np.arange(w.T), "(staged)")


def test_backward_full_size_sampled_experts():
    w = mw.get(4)
    d = mw.inputs(w, 0)
    bm = moe.preferred_block_m(moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=64))
    ns = run_forward_backward(w, d, bm)
    t = tables(ns)
    counts = t["counts"]
    experts = sorted({int(np.argmin(counts)), int(np.argmax(counts)), w.EL // 2})
    args = (d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dW1, dW2 = oracle.backward(*args, E=w.E, e_lo=w.e_lo, experts=experts)
    g1, g2 = unpacked(ns, ns.dW1p, ns.dW2p)
    for i, e in enumerate(experts):
        check_bf16(g1[e], dW1[i], TOL, "dW1[%d] (%d rows, %s)" % (e, counts[e], w.name))
        check_bf16(g2[e], dW2[i], TOL, "dW2[%d] (%d rows, %s)" % (e, counts[e], w.name))
    rng = np.random.default_rng(4)
    real = np.nonzero(t["row_pair"] >= 0)[0]
    rows = np.sort(rng.choice(real, size=24, replace=False))
    check_row_links(w, d, ns, rows, "(sampled rows, %s)" % w.name)
    from gpu_helpers import sample_tokens
    tokens = sample_tokens(t["tok_nloc"], 18, seed=5)
    check_token_grads(w, d, ns, tokens, "(sampled tokens, %s)" % w.name)


@pytest.mark.parametrize("case", ["empty_batch", "none_local", "one_expert_takes_all"])
def test_degenerate_routing_forward_and_backward(case):
    """The method's degenerate cases end to end: no tokens at all; tokens none of whose pairs
    this GPU handles (y, dx, d(topk_w) and every dW exactly zero); every pair on one expert (the
    other experts' weight gradients exactly zero)."""
    w = mw.Workload("degenerate", T=96, H=256, I=128, E=12, EL=4, k=2, e_lo=4, backward=True)
    if case == "empty_batch":
        w = mw.scaled(w, T=0)
    d = mw.inputs(w, 14)
    idx = d["topk_idx"].copy()
    if case == "none_local":
        idx = np.where((idx >= w.e_lo) & (idx < w.e_lo + w.EL), idx + w.EL, idx) % w.E
        idx = np.where((idx >= w.e_lo) & (idx < w.e_lo + w.EL), 0, idx).astype(np.int32)
    elif case == "one_expert_takes_all":
        idx[:] = w.e_lo + 2
    d = dict(d, topk_idx=idx)
    ns = run_forward_backward(w, d, 64)
    t = tables(ns)
    local = (idx >= w.e_lo) & (idx < w.e_lo + w.EL)
    assert int(t["counts"].sum()) == int(local.sum())
    g1, g2 = unpacked(ns, ns.dW1p, ns.dW2p)
    empty = np.nonzero(t["counts"] == 0)[0]
    assert np.all(g1[empty] == 0.0) and np.all(g2[empty] == 0.0)
    if w.T == 0:
        return
    y = f64_host(ns.y)
    ref = oracle.forward(d["x"], idx, d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
    if case == "none_local":
        assert np.all(y == 0.0) and np.all(f64_host(ns.dx) == 0.0) and torch.all(ns.dtw == 0)
        assert np.all(g1 == 0.0) and np.all(g2 == 0.0)
    else:
        check_bf16(y, ref, TOL, "y (%s)" % case)
        check_token_grads(w, d, ns, np.arange(w.T), "(%s)" % case)
        args = (d["x"], idx, d["topk_weights"], d["W1"], d["W2"], d["dy"])
        dW1, dW2 = oracle.backward(*args, E=w.E, e_lo=w.e_lo)
        check_bf16(g1, dW1, TOL, "dW1 (%s)" % case)
        check_bf16(g2, dW2, TOL, "dW2 (%s)" % case)
@pytest.mark.parametrize("bm", [32, 64])
def test_weight_gradients_at_the_row_depth_boundaries(bm):
    """Experts whose rows sit at the edges of the few-rows weight gradients' K depths: at most
    one 64-deep step (64), a second, 32-deep step held in LDS with the first (65, 96), and the
    general loop that reloads the LDS tiles per step (97), next to an expert without rows and one
    with a single row."""
    w = mw.Workload("wgrad_depths", T=200, H=256, I=128, E=8, EL=6, k=2, backward=True)
    want = [64, 65, 96, 97, 0, 1]
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(want)])
    ids = np.concatenate([ids, np.full(w.T * w.k - ids.size, w.E - 1, np.int32)])
    ids = np.random.default_rng(15).permutation(ids).reshape(w.T, w.k)
    d = dict(mw.inputs(w, 15), topk_idx=ids)
    ns = run_forward_backward(w, d, bm)
    assert tables(ns)["counts"][:w.EL].tolist() == want
    args = (d["x"], ids, d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dW1, dW2 = oracle.backward(*args, E=w.E, e_lo=w.e_lo)
    g1, g2 = unpacked(ns, ns.dW1p, ns.dW2p)
    tag = "(row depths, bm %d)" % bm
    check_bf16(g1, dW1, TOL, "dW1 " + tag)
    check_bf16(g2, dW2, TOL, "dW2 " + tag)
    assert np.all(g1[4] == 0.0) and np.all(g2[4] == 0.0), "expert without rows must get exact zeros"
    check_token_grads(w, d, ns, np.arange(w.T), tag)


def test_backward_is_graph_capturable():
    """The fused backward (dgrad with d(topk_w), dW2, dW1, dx) captured into a HIP graph replays
    bit-identically to the eager call, with eager work and a stale workspace between replays."""
    w = REDUCED[1]
    d = mw.inputs(w, 15)
    ns = run_forward_backward(w, d, 64)
    ref = {n: getattr(ns, n).clone() for n in ("dx", "dtw", "dW1p", "dW2p")}
    out = {n: torch.full_like(t, float("nan")) for n, t in ref.items()}
    args = (ns.shape, ns.x, ns.dy, ns.wts, ns.W2p, ns.ws)
    kw = dict(w1p=ns.W1p, dx=out["dx"], dtopk_w=out["dtw"])
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        moe.backward(*args, out["dW1p"], out["dW2p"], **kw)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            moe.backward(*args, out["dW1p"], out["dW2p"], **kw)
    torch.cuda.current_stream().wait_stream(stream)
    for i in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        stage = moe.ws_region(ns.ws, ns.shape, "stage")
        stage.fill_(float("nan"))    # stale staging rows between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(out[n], ref[n]), "replay %d: %s differs" % (i, n)
        moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)   # eager work between
        torch.cuda.synchronize()


def test_max_local_experts_forward_and_backward():
    """EL = 1024 (the largest the ABI accepts, four experts per thread of the forward's tile-prefix
    scan): the last expert's prefix entry must be written, so every expert's rows reach the GEMMs.
    Forward and backward against the oracle on a small batch spread over 1024 local experts."""
    w = mw.Workload("max_experts", T=256, H=128, I=128, E=1024, EL=1024, k=4, backward=True)
    d = mw.inputs(w, 16)
    idx = d["topk_idx"].copy()
    idx[0, 0] = w.EL - 1          # the last local expert holds rows
    idx[1, :] = [w.EL - 1, w.EL - 2, 0, 5]
    d = dict(d, topk_idx=idx)
    ns = run_forward_backward(w, d, 64)
    t = tables(ns)
    assert t["counts"][w.EL - 1] >= 2
    ref = oracle.forward(d["x"], idx, d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
    check_bf16(f64_host(ns.y), ref, TOL, "y (EL = 1024)")
    args = (d["x"], idx, d["topk_weights"], d["W1"], d["W2"], d["dy"])
    experts = [0, 5, w.EL - 2, w.EL - 1]
    dW1, dW2 = oracle.backward(*args, E=w.E, e_lo=w.e_lo, experts=experts)
    g1, g2 = unpacked(ns, ns.dW1p, ns.dW2p)
    for i, e in enumerate(experts):
        check_bf16(g1[e], dW1[i], TOL, "dW1[%d] (EL = 1024)" % e)
        check_bf16(g2[e], dW2[i], TOL, "dW2[%d] (EL = 1024)" % e)
    check_token_grads(w, d, ns, np.arange(w.T), "(EL = 1024)")


def test_autograd_op_matches_the_entry_points():
    """moe_layer (one torch.autograd op over moe_forward / moe_backward) gives the entry points' y,
    dx, d(topk_w), dW1 and dW2 bit for bit, and y and the gradients agree with the oracle."""
    w = REDUCED[1]
    d = mw.inputs(w, 17)
    ns = run_forward_backward(w, d, 64)
    x = ns.x.clone().requires_grad_(True)
    tw = ns.wts.clone().requires_grad_(True)
    W1p = ns.W1p.clone().requires_grad_(True)
    W2p = ns.W2p.clone().requires_grad_(True)
    ws = moe.alloc_workspace(ns.shape)
    y = moe.moe_layer(x, ns.idx, tw, W1p, W2p, ns.shape, ws)
    y.backward(ns.dy)
    torch.cuda.synchronize()
    assert torch.equal(y.detach().view(torch.int16), ns.y.view(torch.int16))
    assert torch.equal(x.grad.view(torch.int16), ns.dx.view(torch.int16))
    assert torch.equal(tw.grad, ns.dtw)
    assert torch.equal(W1p.grad.view(torch.int16), ns.dW1p.view(torch.int16))
    assert torch.equal(W2p.grad.view(torch.int16), ns.dW2p.view(torch.int16))
    ref = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
    check_bf16(f64_host(y.detach()), ref, TOL, "y (autograd op)")
    check_token_grads(w, d, SimpleNamespace(dx=x.grad, dtw=tw.grad), np.arange(w.T), "(autograd op)")
