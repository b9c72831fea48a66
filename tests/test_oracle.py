"""Pins of the CPU oracle to things other than itself (CPU only, no GPU).

Each pin ties an oracle function to a library routine, an invariant, a closed form, a
hand-derived table or torch autograd, chosen so that a plausible mistake in the oracle (a
swapped gate/up, a weight applied twice, a wrong stable order, a wrong pad, a sign slip in the
SwiGLU derivative, a wrong operand in a weight gradient) fails at least one of them.  The
mutation tests at the bottom plant such mistakes in a copy of the oracle and check that.

Passages followed: "Mega MoE" page, Pipeline (forward and backward) and Implementation Map
(dispatch prologue); "How Mega MoE Overlaps ..." page, Block-M alignment.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F = torch.nn.functional


def f64(bits):
    return torch.from_numpy(mw.bf16_bits_to_f32(bits).astype(np.float64))


def small_case(T=48, H=64, I=32, E=8, EL=8, k=2, e_lo=0, seed=1):
    w = mw.Workload("t", T=T, H=H, I=I, E=E, EL=EL, k=k, e_lo=e_lo)
    d = mw.inputs(w, seed)
    return w, d


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale) if a.size else 0.0


# ----------------------------------------------------------------------------------------
# Library formulations (torch fp64 matmul / silu / autograd), independent of the oracle.
# ----------------------------------------------------------------------------------------
def dense_ffn(X, W1e, W2e):
    """SwiGLU FFN of one expert applied to every row of X with torch's matmul and silu."""
    I = W2e.shape[0]
    h = X @ W1e
    return (F.silu(h[:, :I]) * h[:, I:]) @ W2e


def masked_dense_moe(x, idx, wts, W1, W2, E, e_lo):
    """Every local expert applied densely to all tokens, then mixed with the routing weights
    of the slots that selected it (duplicate slots add)."""
    X, W1t, W2t = f64(x), f64(W1), f64(W2)
    idx_t = torch.from_numpy(idx.astype(np.int64))
    wt = torch.from_numpy(wts.astype(np.float64))
    y = torch.zeros(X.shape, dtype=torch.float64)
    for e in range(W1.shape[0]):
        coef = (wt * (idx_t == e_lo + e)).sum(1)
        if torch.any(coef != 0):
            y += coef[:, None] * dense_ffn(X, W1t[e], W2t[e])
    return y.numpy()


def route_by_sort(idx, E, e_lo, EL, BM):
    """Routing tables from a stable library sort of the local pairs by expert."""
    T, k = idx.shape
    ids = idx.reshape(-1).astype(np.int64)
    valid = (ids >= 0) & (ids < E)
    e = ids - e_lo
    local = valid & (e >= 0) & (e < EL)
    p_loc = np.nonzero(local)[0]
    order = np.argsort(e[p_loc], kind="stable")
    sp, se = p_loc[order], e[p_loc][order]
    counts = np.bincount(se, minlength=EL)
    padded = -(-counts // BM) * BM
    offs = np.concatenate([[0], np.cumsum(padded)])
    starts = np.concatenate([[0], np.cumsum(counts)])[:-1]
    rows = offs[se] + (np.arange(len(sp)) - starts[se])
    R = -(-(T * k + EL * (BM - 1)) // BM) * BM
    row_pair = -np.ones(R, np.int64)
    row_pair[rows] = sp
    pair_row = -np.ones(T * k, np.int64)
    pair_row[sp] = rows
    m0 = np.arange(R // BM) * BM
    te = np.searchsorted(offs, m0, side="right") - 1
    te[m0 >= offs[-1]] = -1
    return {
        "counts": counts, "padded_offsets": offs, "row_pair": row_pair, "pair_row": pair_row,
        "tile_expert": te, "tok_nloc": local.reshape(T, k).sum(1),
        "num_rows": int(offs[-1]), "dropped": int((~valid).sum()),
    }


# ----------------------------------------------------------------------------------------
# Pins as plain functions (reused by the mutation tests)
# ----------------------------------------------------------------------------------------
def pin_route_golden():
    g = json.load(open(os.path.join(GOLDEN, "brute4_routing.json")))
    r = oracle.route(np.array(g["topk_idx"], np.int32), g["E"], g["e_lo"], g["EL"], g["BM"])
    for key, val in g["expected"].items():
        got = r[key]
        if isinstance(val, list):
            assert list(np.asarray(got)) == val, (key, got, val)
        else:
            assert got == val, (key, got, val)


def pin_route_sort(idx, E, e_lo, EL, BM):
    r = oracle.route(idx, E, e_lo, EL, BM)
    s = route_by_sort(idx, E, e_lo, EL, BM)
    for key in s:
        assert np.array_equal(np.asarray(r[key]), np.asarray(s[key])), key


def pin_forward_k1_dense(seed=3):
    """top-k = 1 with weight 1 is a dense per-expert FFN on the tokens routed to each expert."""
    w, d = small_case(T=40, H=64, I=32, E=4, EL=4, k=1, seed=seed)
    ones = np.ones((w.T, 1), np.float32)
    y = oracle.forward(d["x"], d["topk_idx"], ones, d["W1"], d["W2"], E=w.E)
    X, W1, W2 = f64(d["x"]), f64(d["W1"]), f64(d["W2"])
    ref = np.zeros_like(y)
    for e in range(w.EL):
        rows = np.nonzero(d["topk_idx"][:, 0] == e)[0]
        if len(rows):
            ref[rows] = dense_ffn(X[rows], W1[e], W2[e]).numpy()
    assert rel_err(y, ref) < 1e-12


def pin_forward_masked_dense(seed=4):
    w, d = small_case(T=37, H=64, I=48, E=10, EL=4, k=3, e_lo=3, seed=seed)
    idx = d["topk_idx"].copy()
    idx[0] = [4, 4, 5]        # duplicate local expert in one token
    idx[1] = [10, -1, 3]      # two ids outside [0, E), one local
    idx[2] = [0, 1, 9]        # valid ids, none local
    y = oracle.forward(d["x"], idx, d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
    ref = masked_dense_moe(d["x"], idx, d["topk_weights"], d["W1"], d["W2"], w.E, w.e_lo)
    assert rel_err(y, ref) < 1e-12
    assert np.all(y[2] == 0.0)


def pin_forward_linear_in_weights(seed=5):
    w, d = small_case(seed=seed)
    args = (d["x"], d["topk_idx"])
    W = (d["W1"], d["W2"])
    y1 = oracle.forward(*args, d["topk_weights"], *W, E=w.E)
    for alpha in (4.0, -0.5):      # powers of two: the scaled fp32 weights are exact
        y2 = oracle.forward(*args, np.float32(alpha) * d["topk_weights"], *W, E=w.E)
        assert rel_err(y2, alpha * y1) < 1e-12
    rng = np.random.default_rng(9)
    wa = rng.standard_normal(d["topk_weights"].shape).astype(np.float32)
    wb = rng.standard_normal(d["topk_weights"].shape).astype(np.float32)
    ya = oracle.forward(*args, wa, *W, E=w.E)
    yb = oracle.forward(*args, wb, *W, E=w.E)
    yab = oracle.forward(*args, (wa.astype(np.float64) + wb).astype(np.float32), *W, E=w.E)
    # wa + wb is rounded to fp32; compare against the exact-sum prediction at fp32 precision
    assert rel_err(yab, ya + yb) < 1e-6


# ----------------------------------------------------------------------------------------
# Routing tables
# ----------------------------------------------------------------------------------------
def test_route_brute_force_golden():
    pin_route_golden()


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("BM", [32, 64, 128, 256])
def test_route_matches_stable_sort_on_workloads(cfg, BM):
    w = mw.get(cfg)
    idx, _ = mw.routing(w, 0)
    pin_route_sort(idx, w.E, w.e_lo, w.EL, BM)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5])
def test_route_invariants(cfg):
    w = mw.get(cfg)
    idx, _ = mw.routing(w, 0)
    BM = 64
    r = oracle.route(idx, w.E, w.e_lo, w.EL, BM)
    P = mw.local_pairs(w, idx)
    assert r["counts"].sum() == P
    if w.EL == w.E:
        assert P == w.T * w.k and np.all(r["pair_row"] >= 0)
    offs = r["padded_offsets"]
    assert np.all(np.diff(offs) >= 0) and np.all(offs % BM == 0)
    assert np.all(np.diff(offs) - r["counts"] < BM) and np.all(np.diff(offs) >= r["counts"])
    rp, pr = r["row_pair"], r["pair_row"]
    real = np.nonzero(rp >= 0)[0]
    assert len(real) == P and len(np.unique(rp[real])) == P
    assert np.all(pr[rp[real]] == real)
    for e in range(w.EL):
        seg = rp[offs[e]:offs[e] + r["counts"][e]]
        assert np.all(seg >= 0) and np.all(np.diff(seg) > 0)
        assert np.all(idx.reshape(-1)[seg] == w.e_lo + e)
        assert np.all(rp[offs[e] + r["counts"][e]:offs[e + 1]] == -1)
    assert r["num_rows"] == offs[-1]
    assert r["tok_nloc"].sum() == P
    if cfg == 3:
        assert np.sum(r["counts"] == 0) >= 1


@pytest.mark.parametrize("case", ["empty", "none_local", "all_dropped", "k1", "dups", "shard"])
def test_route_edge_cases(case):
    rng = np.random.default_rng(11)
    E, EL, e_lo, k, T = 16, 4, 0, 3, 50
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if case == "empty":
        idx = np.zeros((0, k), np.int32)
    elif case == "none_local":
        idx = rng.integers(EL, E, size=(T, k)).astype(np.int32)
    elif case == "all_dropped":
        idx = rng.integers(E, 3 * E, size=(T, k)).astype(np.int32)
        idx[::2] = -idx[::2]
    elif case == "k1":
        idx = rng.integers(0, EL, size=(T, 1)).astype(np.int32)
    elif case == "dups":
        idx[:, 1] = idx[:, 0]
        idx[:, 2] = idx[:, 0]
        idx[:, 0] %= EL
    elif case == "shard":
        e_lo = 12
    for BM in (1, 2, 32, 64):
        pin_route_sort(idx, E, e_lo, EL, BM)
    r = oracle.route(idx, E, e_lo, EL, 32)
    if case in ("empty", "none_local", "all_dropped"):
        assert r["num_rows"] == 0 and np.all(r["row_pair"] == -1) and np.all(r["tile_expert"] == -1)
    if case == "all_dropped":
        assert r["dropped"] == idx.size


# ----------------------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------------------
def test_forward_k1_equals_dense_per_expert_ffn():
    pin_forward_k1_dense()


def test_forward_matches_masked_dense_library_composition():
    pin_forward_masked_dense()


def test_forward_tiny_workload_matches_masked_dense():
    w = mw.get(0)
    d = mw.inputs(w, 0)
    y = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E)
    ref = masked_dense_moe(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], w.E, 0)
    assert rel_err(y, ref) < 1e-12


def test_forward_linear_in_routing_weights():
    pin_forward_linear_in_weights()


def test_forward_token_permutation_equivariance():
    w, d = small_case(seed=6)
    y = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E)
    perm = np.random.default_rng(2).permutation(w.T)
    yp = oracle.forward(d["x"][perm], d["topk_idx"][perm], d["topk_weights"][perm],
                        d["W1"], d["W2"], E=w.E)
    assert np.array_equal(yp, y[perm])


def test_forward_slot_permutation_invariance():
    w, d = small_case(k=3, seed=7)
    y = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E)
    s = [2, 0, 1]
    ys = oracle.forward(d["x"], d["topk_idx"][:, s], d["topk_weights"][:, s], d["W1"], d["W2"], E=w.E)
    assert rel_err(ys, y) < 1e-13


def test_forward_duplicate_pairs_add_and_dropped_ids_contribute_nothing():
    w, d = small_case(k=2, seed=8)
    idx = d["topk_idx"].copy()
    idx[:, 1] = idx[:, 0]
    wts = d["topk_weights"]
    y = oracle.forward(d["x"], idx, wts, d["W1"], d["W2"], E=w.E)
    merged = (wts[:, :1].astype(np.float64) + wts[:, 1:]).astype(np.float32)
    y1 = oracle.forward(d["x"], idx[:, :1], merged, d["W1"], d["W2"], E=w.E)
    assert rel_err(y, y1) < 1e-6
    bad = d["topk_idx"].copy()
    bad[:, 1] = np.where(np.arange(w.T) % 2 == 0, w.E, -3)
    zw = wts.copy()
    zw[:, 1] = 0.0
    yb = oracle.forward(d["x"], bad, wts, d["W1"], d["W2"], E=w.E)
    yz = oracle.forward(d["x"], d["topk_idx"], zw, d["W1"], d["W2"], E=w.E)
    assert np.array_equal(yb, yz)


def test_forward_expert_shards_sum_to_all_local():
    full = mw.Workload("t", T=32, H=64, I=32, E=8, EL=8, k=3)
    d = mw.inputs(full, 12)
    y = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=8)
    acc = np.zeros_like(y)
    for s in range(4):
        sh = mw.scaled(full, EL=2, e_lo=2 * s)
        W1, W2 = mw.weights(sh, 12)
        acc += oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], W1, W2, E=8, e_lo=2 * s)
    assert rel_err(acc, y) < 1e-13


def test_forward_token_subset_rows_match_full():
    w, d = small_case(seed=13)
    y = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E)
    sub = np.array([5, 0, 47, 5])
    ys = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E, tokens=sub)
    assert np.array_equal(ys, y[sub])


def test_l1_rows_match_library_matmul_and_silu():
    w, d = small_case(E=8, EL=3, e_lo=2, k=2, seed=14)
    idx = d["topk_idx"]
    pairs = np.arange(w.T * w.k)
    h, a = oracle.l1_rows(d["x"], idx, d["W1"], w.E, w.e_lo, pairs)
    X, W1 = f64(d["x"]), f64(d["W1"])
    for p in pairs:
        e = idx.reshape(-1)[p] - w.e_lo
        if 0 <= e < w.EL:
            href = (X[p // w.k] @ W1[e]).numpy()
            assert rel_err(h[p], href) < 1e-12
            aref = (F.silu(torch.from_numpy(href[:w.I])) * torch.from_numpy(href[w.I:])).numpy()
            assert rel_err(a[p], aref) < 1e-12
        else:
            assert np.all(h[p] == 0) and np.all(a[p] == 0)


# ----------------------------------------------------------------------------------------
# SwiGLU closed forms and autograd
# ----------------------------------------------------------------------------------------
def test_swiglu_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 2.0], np.float32)
    u = np.array([5.0, 1.0, 1.0, 1.0, 1.0, -0.5], np.float32)
    hgu = mw.f32_to_bf16_bits(np.concatenate([g, u])[None, :])
    a = oracle.swiglu(hgu)[0]
    e1 = 1.0 / (1.0 + np.exp(-1.0))      # sigmoid(1) = 0.7310585786300049
    assert a[0] == 0.0
    assert abs(a[1] - e1) < 1e-15 and abs(a[2] + (1 - e1)) < 1e-15
    assert abs(a[3] - 30.0) < 1e-11 and abs(a[4]) < 1e-11
    assert abs(a[5] - (-0.5 * 2.0 / (1.0 + np.exp(-2.0)))) < 1e-15


def test_swiglu_fwd_bwd_match_torch_autograd():
    rng = np.random.default_rng(15)
    n, I = 33, 24
    hgu = mw.f32_to_bf16_bits(3 * rng.standard_normal((n, 2 * I)).astype(np.float32))
    da = mw.f32_to_bf16_bits(rng.standard_normal((n, I)).astype(np.float32))
    h = f64(hgu).requires_grad_(True)
    a = F.silu(h[:, :I]) * h[:, I:]
    a.backward(f64(da))
    assert rel_err(oracle.swiglu(hgu), a.detach().numpy()) < 1e-13
    assert rel_err(oracle.swiglu_bwd(hgu, f64(da).numpy()), h.grad.numpy()) < 1e-13


def test_swiglu_on_real_valued_rows_matches_torch_autograd():
    """The SwiGLU functions also take the [gate | up] rows as real values (the saved fp32
    pre-activation of a training forward): fp64 rows that no bf16 or fp32 pattern holds."""
    rng = np.random.default_rng(16)
    n, I = 29, 40
    hv = 4 * rng.standard_normal((n, 2 * I))
    da = rng.standard_normal((n, I))
    h = torch.from_numpy(hv.copy()).requires_grad_(True)
    a = F.silu(h[:, :I]) * h[:, I:]
    a.backward(torch.from_numpy(da))
    assert rel_err(oracle.swiglu(hv), a.detach().numpy()) < 1e-13
    assert rel_err(oracle.swiglu_bwd(hv, da), h.grad.numpy()) < 1e-13
    # bf16 bit patterns and the same values given as reals agree exactly
    bits = mw.f32_to_bf16_bits(hv.astype(np.float32))
    vals = mw.bf16_bits_to_f32(bits).astype(np.float64)
    assert np.array_equal(oracle.swiglu(bits), oracle.swiglu(vals))
    assert np.array_equal(oracle.swiglu_bwd(bits, da), oracle.swiglu_bwd(vals, da))


# ----------------------------------------------------------------------------------------
# Backward (weight gradients and per-pair intermediates) against torch autograd
# ----------------------------------------------------------------------------------------
def autograd_backward(x, idx, wts, W1b, W2b, dyb, E, e_lo, token_grads=None):
    X, dy = f64(x), f64(dyb)
    W1 = f64(W1b).requires_grad_(True)
    W2 = f64(W2b).requires_grad_(True)
    idx_t = torch.from_numpy(idx.astype(np.int64))
    wt = torch.from_numpy(wts.astype(np.float64))
    if token_grads is not None:
        X.requires_grad_(True)
        wt.requires_grad_(True)
    EL, _, N = W1b.shape
    I = N // 2
    y = torch.zeros(X.shape, dtype=torch.float64)
    per_slot = {}
    for j in range(idx.shape[1]):
        for e in range(EL):
            coef = wt[:, j] * (idx_t[:, j] == e_lo + e)
            if not torch.any(coef != 0):
                continue
            h = X @ W1[e]
            h.retain_grad()
            a = F.silu(h[:, :I]) * h[:, I:]
            a.retain_grad()
            y = y + coef[:, None] * (a @ W2[e])
            per_slot[(j, e)] = (h, a)
    (y * dy).sum().backward()
    if token_grads is not None:
        token_grads["x"] = X.grad.numpy()
        token_grads["w"] = wt.grad.numpy()
    return W1.grad.numpy(), W2.grad.numpy(), per_slot


@pytest.mark.parametrize("shape", ["tiny", "wide_reduced"])
def test_backward_matches_torch_autograd(shape):
    if shape == "tiny":
        w = mw.scaled(mw.get(0), backward=True)
    else:
        w = mw.scaled(mw.get(4), T=64, H=256, I=128, E=48, EL=6)
    d = mw.inputs(w, 0)
    idx = d["topk_idx"].copy()
    if shape == "wide_reduced":
        idx[:, 0] = np.where(np.arange(w.T) < 20, 1, idx[:, 0])    # one busier expert
    args = (d["x"], idx, d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dW1, dW2 = oracle.backward(*args, E=w.E, e_lo=w.e_lo)
    gW1, gW2, per_slot = autograd_backward(*args, w.E, w.e_lo)
    assert rel_err(dW1, gW1) < 1e-12 and rel_err(dW2, gW2) < 1e-12
    counts = np.bincount(idx.reshape(-1)[(idx.reshape(-1) >= 0) & (idx.reshape(-1) < w.EL)],
                         minlength=w.EL)
    for e in np.nonzero(counts == 0)[0]:
        assert np.all(dW1[e] == 0) and np.all(dW2[e] == 0)
    pairs = np.arange(w.T * w.k)
    dA, dH = oracle.backward_rows(*args, E=w.E, e_lo=w.e_lo, pairs=pairs)
    for p in pairs[::3]:
        t, j = divmod(int(p), w.k)
        e = int(idx[t, j]) - w.e_lo
        if 0 <= e < w.EL:
            h, a = per_slot[(j, e)]
            assert rel_err(dA[p], a.grad[t].numpy()) < 1e-12
            assert rel_err(dH[p], h.grad[t].numpy()) < 1e-12


@pytest.mark.parametrize("shape", ["tiny", "wide_reduced", "shard"])
def test_backward_tokens_match_torch_autograd(shape):
    """dx and d(topk_weights) of the oracle against torch autograd of the layer in fp64: the
    gradient of sum(y * dy) with respect to x and to the routing weights (pairs that are not
    local get 0, since y is this GPU's partial sum)."""
    if shape == "tiny":
        w = mw.scaled(mw.get(0), backward=True)
    elif shape == "wide_reduced":
        w = mw.scaled(mw.get(4), T=64, H=256, I=128, E=48, EL=6)
    else:
        w = mw.scaled(mw.get(4), T=40, H=128, I=64, E=16, EL=4, e_lo=8)
    d = mw.inputs(w, 0)
    idx = d["topk_idx"].copy()
    if shape != "tiny":
        idx[3, 0] = w.E + 5           # dropped id
        idx[5, 1] = idx[5, 0]         # duplicated expert in one token
    args = (d["x"], idx, d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dx, dw = oracle.backward_tokens(*args, E=w.E, e_lo=w.e_lo)
    g = {}
    autograd_backward(*args, w.E, w.e_lo, token_grads=g)
    assert rel_err(dx, g["x"]) < 1e-12 and rel_err(dw, g["w"]) < 1e-12
    local = (idx >= w.e_lo) & (idx < w.e_lo + w.EL)
    assert np.all(dw[~local] == 0)
    assert np.all(dx[~local.any(axis=1)] == 0)
    sub = np.array([7, 2, 5])
    dx2, dw2 = oracle.backward_tokens(*args, E=w.E, e_lo=w.e_lo, tokens=sub)
    assert np.array_equal(dx2, dx[sub]) and np.array_equal(dw2, dw[sub])


def test_backward_tokens_weight_gradient_is_forward_row_dot():
    """With k = 1 and weight 1, d(topk_weights)[t] = <dy[t], y[t]>: the forward output row
    is the unweighted L2 row of the token's only pair."""
    w = mw.Workload("t", T=24, H=64, I=32, E=4, EL=4, k=1, backward=True)
    d = mw.inputs(w, 3)
    wts = np.ones((w.T, 1), np.float32)
    args = (d["x"], d["topk_idx"], wts, d["W1"], d["W2"])
    y = oracle.forward(*args, E=w.E)
    _, dw = oracle.backward_tokens(*args, d["dy"], E=w.E)
    assert rel_err(dw[:, 0], np.sum(f64(d["dy"]).numpy() * y, axis=1)) < 1e-12


def test_backward_expert_without_rows_is_exact_zero():
    w = mw.Workload("t", T=16, H=32, I=16, E=4, EL=4, k=1, backward=True)
    d = mw.inputs(w, 2)
    idx = np.zeros((w.T, 1), np.int32)
    dW1, dW2 = oracle.backward(d["x"], idx, d["topk_weights"], d["W1"], d["W2"], d["dy"], E=4)
    assert np.all(dW1[1:] == 0) and np.all(dW2[1:] == 0) and np.any(dW1[0] != 0)


# ----------------------------------------------------------------------------------------
# Mutation checks: a planted mistake in a copy of the oracle must fail a pin.
# ----------------------------------------------------------------------------------------
def _backward_pin():
    test_backward_matches_torch_autograd("tiny")


def _backward_tokens_pin():
    test_backward_tokens_match_torch_autograd("wide_reduced")


MUTATIONS = [
    ("gate/up swapped", "a[c] = silu(h[c]) * h[I + c];", "a[c] = silu(h[I + c]) * h[c];",
     pin_forward_k1_dense),
    ("weight applied twice", "acc[m] += w * o[m];", "acc[m] += w * w * o[m];",
     pin_forward_linear_in_weights),
    ("pad one block too many", "int32_t padded = (counts[e] + BM - 1) / BM * BM;",
     "int32_t padded = (counts[e] + BM) / BM * BM;", pin_route_golden),
    ("reverse order within expert", "int32_t row = next[e]++;",
     "int32_t row = padded_offsets[e] + counts[e] - 1 - (next[e]++ - padded_offsets[e]);",
     pin_route_golden),
    ("dropped range off by one", "if (id < 0 || id >= E) ++dropped;",
     "if (id < 0 || id > E) ++dropped;", pin_route_golden),
    ("silu derivative sign", "dhgu[c] = dA[c] * u * sg * (1.0 + g * (1.0 - sg));",
     "dhgu[c] = dA[c] * u * sg * (1.0 - g * (1.0 - sg));", _backward_pin),
    ("dW2 uses pre-activation", "row[m] += a[c] * dO[m];", "row[m] += h[c] * dO[m];",
     _backward_pin),
    ("dx through the transposed W1 index", "for (int n = 0; n < 2 * I; ++n) d += bf16_value(wrow[n]) * dhgu[n];",
     "for (int n = 0; n < 2 * I; ++n) d += bf16_value(W1e[(size_t)n * H + q]) * dhgu[n];",
     _backward_tokens_pin),
    ("dtopk_w from the weighted row", "for (int m = 0; m < H; ++m) s += bf16_value(dyrow[m]) * o[m];",
     "for (int m = 0; m < H; ++m) s += bf16_value(dyrow[m]) * o[m] * topk_w[(int64_t)t * k + j];",
     _backward_tokens_pin),
    ("slot weight index", "const double w = (double)topk_w[(int64_t)t * k + j];",
     "const double w = (double)topk_w[(int64_t)t * k];", pin_forward_masked_dense),
]


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, pin, tmp_path, monkeypatch):
    src = open(oracle._SRC).read()
    assert old in src, "mutation anchor not found: " + name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o",
                           str(so), str(mutated), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.configure(ctypes.CDLL(str(so))))
    with pytest.raises(AssertionError):
        pin()
