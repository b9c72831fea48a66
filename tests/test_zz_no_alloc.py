"""The allocation-free forward (moe_forward_noalloc) against the forward with a caller workspace
(moe_forward), through the C ABI: two calls in a row on the library's one scratch array, the
second on a smaller shape (so the array holds the first call's contents), each bit for bit equal
to moe_forward and within the forward's bar of the oracle; a shape whose workspace exceeds the
fixed scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import token_dispatch_grouped_route_amd as moe
from gpu_helpers import check_bf16, f64_host, layer

pytestmark = pytest.mark.gpu


def test_forward_noalloc_matches_forward_on_two_calls():
    cases = [
        (mw.Workload("noalloc_large", T=512, H=1024, I=512, E=16, EL=8, k=4, e_lo=4), 64, 31),
        (mw.Workload("noalloc_small", T=100, H=512, I=256, E=8, EL=8, k=2), 128, 32),
    ]
    for w, bm, seed in cases:
        d = mw.inputs(w, seed)
        ns = layer(w, d, bm)
        assert moe.workspace_bytes(ns.shape) <= moe.NOALLOC_SCRATCH_BYTES
        moe.forward(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, ns.ws, ns.y)
        y2 = torch.full_like(ns.y, float("nan"))
        moe.forward_noalloc(ns.shape, ns.x, ns.idx, ns.wts, ns.W1p, ns.W2p, y2)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), ns.y.view(torch.int16)), "%s: differs from moe_forward" % w.name
        ref = oracle.forward(d["x"], d["topk_idx"], d["topk_weights"], d["W1"], d["W2"], E=w.E, e_lo=w.e_lo)
        check_bf16(f64_host(y2), ref, 2e-2, "y (no-alloc forward, %s)" % w.name)
        del ns, y2
        torch.cuda.empty_cache()


def test_forward_noalloc_refuses_shapes_beyond_its_scratch():
    s = moe.make_shape(8192, 7168, 2048, 256, 32, 8, block_m=128)
    assert moe.workspace_bytes(s) > moe.NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="scratch"):
        moe.lib()   # the size check runs before any pointer is looked at
        import ctypes
        st = moe.lib().moe_forward_noalloc(ctypes.byref(s), None, None, None, dummy.data_ptr(), dummy.data_ptr(),
                                           None, None)
        moe._check(st, "moe_forward_noalloc")
    t = moe.make_shape(64, 256, 128, 8, 8, 2, block_m=64, train=True)
    with pytest.raises(moe.MoeError, match="size"):
        import ctypes
        moe._check(moe.lib().moe_forward_noalloc(ctypes.byref(t), None, None, None, dummy.data_ptr(),
                                                 dummy.data_ptr(), None, None), "moe_forward_noalloc")
