"""A sweep of small shapes through the whole layer, forward and backward, each compared in full with
the oracle: widths that are not multiples of 256 (the 128-column tiles of both GEMM directions),
experts with up to eight 32-row groups, shards that start mid-range, top-8 routing, one local
expert, hundreds of local experts, and every block_m.  Inputs are the seeded generators' (N(0,1)
logits, top-k by value, softmax weights), with one local expert emptied so its gradients must be
exact zeros."""
import numpy as np
import pytest

import torch

import moe_workloads as mw
import oracle
import token_dispatch_grouped_route_amd as moe
from gpu_helpers import check_bf16, check_f32, f64_host, layer, unpacked

pytestmark = pytest.mark.gpu
TOL = 2e-2

SWEEP = [
    (mw.Workload("sw_i384", T=200, H=256, I=384, E=16, EL=5, k=4, e_lo=3, backward=True), 64),
    (mw.Workload("sw_h640", T=150, H=640, I=128, E=12, EL=12, k=3, backward=True), 32),
    (mw.Workload("sw_k8", T=96, H=384, I=256, E=64, EL=8, k=8, e_lo=56, backward=True), 128),
    (mw.Workload("sw_el1", T=333, H=128, I=128, E=4, EL=1, k=2, e_lo=2, backward=True), 256),
    (mw.Workload("sw_groups", T=700, H=256, I=384, E=6, EL=3, k=2, backward=True), 64),
    (mw.Workload("sw_el200", T=64, H=128, I=256, E=300, EL=200, k=6, e_lo=50, backward=True), 32),
]


def emptied(w, d):
    """Local expert 0 receives no pair (its ids move to the next local expert); a one-expert shard
    keeps its routing."""
    if w.EL == 1:
        return d
    idx = d["topk_idx"].copy()
    idx[idx == w.e_lo] = w.e_lo + 1
    return dict(d, topk_idx=idx)


@pytest.mark.parametrize("w,bm", SWEEP, ids=[w.name for w, _ in SWEEP])
def test_sweep_forward_and_backward_full_compare(w, bm):
    d = emptied(w, mw.inputs(w, 21))
    ns = layer(w, d, bm, train=True)
    print("[sweep] %s bm %d" % (w.name, bm), flush=True)
    moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
    s1, s2 = moe.packed_sizes(ns.shape)
    dW1p = torch.full(s1, float("nan"), dtype=torch.bfloat16, device="cuda")
    dW2p = torch.full(s2, float("nan"), dtype=torch.bfloat16, device="cuda")
    dx = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dtw = torch.full((w.T, w.k), float("nan"), dtype=torch.float32, device="cuda")
    moe.backward(ns.shape, ns.x, ns.dy, ns.wts, ns.W2p, ns.ws, dW1p, dW2p, w1p=ns.W1p, dx=dx, dtopk_w=dtw)
    torch.cuda.synchronize()

    tag = "(%s, bm %d)" % (w.name, bm)
    y_ref = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
    check_bf16(f64_host(ns.y), y_ref, TOL, "y " + tag)
    args = (d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], d["dy"])
    dW1, dW2 = oracle.backward(*args, E=w.E, e_lo=w.e_lo)
    g1, g2 = unpacked(ns, dW1p, dW2p)
    check_bf16(g1, dW1, TOL, "dW1 " + tag)
    check_bf16(g2, dW2, TOL, "dW2 " + tag)
    if w.EL > 1:
        assert np.all(g1[0] == 0.0) and np.all(g2[0] == 0.0), "an expert without rows must get exact zeros"
    dx_ref, dw_ref = oracle.backward_tokens(*args, E=w.E, e_lo=w.e_lo, tokens=np.arange(w.T))
    check_bf16(f64_host(dx), dx_ref, TOL, "dx " + tag)
    check_f32(dtw.cpu().double().numpy(), dw_ref, TOL, "d(topk_w) " + tag)
