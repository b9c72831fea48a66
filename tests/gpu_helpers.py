"""Helpers shared by the GPU tests: moving the seeded inputs to the device and running the
library through its binding.  No arithmetic of the layer lives here."""
from types import SimpleNamespace

import numpy as np
import torch

import token_dispatch_grouped_route_amd as moe

TABLES = ("counts", "padded_offsets", "row_pair", "pair_row", "tile_expert", "tok_nloc")


def bf16_dev(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def bits_host(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f64_host(t):
    return t.float().cpu().double().numpy()


def rel_max_err(got, ref):
    """max |got - ref| / rms(ref) over the whole array."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / rms)


def bf16_half_ulp(v):
    """Largest error of rounding a value of magnitude |v| to bf16 (half an ulp of its binade)."""
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(v)   # v = m * 2**e with m in [0.5, 1): the ulp is 2**(e - 8)
    return np.where(v > 0, np.ldexp(1.0, e - 9), 0.0)


def bf16_out_err(got, ref):
    """Acceptance measure for a bf16 output: max over elements of |got - ref| minus the element's
    own rounding to bf16 (half an ulp at max(|got|, |ref|)), over rms(ref).  The bound 2e-2
    applies to this: the error of the computation, with the output dtype's rounding on top."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    excess = np.abs(got - ref) - bf16_half_ulp(np.maximum(np.abs(got), np.abs(ref)))
    m = float(np.max(excess)) if got.size else 0.0
    return max(m, 0.0) / rms if rms > 0 else max(m, 0.0)


# (what, error beyond the output's rounding / rms, raw max|err| / rms) of every check this process
# made; conftest.py writes them out when MOE_PARITY_LOG names a file.
RECORDS = []


def check_bf16(got, ref, tol, what=""):
    """A bf16 output: every element within tol * rms(ref) plus its own rounding to bf16."""
    e, raw = bf16_out_err(got, ref), rel_max_err(got, ref)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    print("[parity] %-34s err beyond bf16 rounding %.3e  raw max|err|/rms %.3e" % (what, e, raw))
    RECORDS.append((what, e, raw))
    assert e <= tol, "%s: error beyond bf16 rounding %.4g > %.3g (raw max|err|/rms %.4g)" % (what, e, tol, raw)
    return e, raw


def check_f32(got, ref, tol, what=""):
    """An fp32 output (or a hi + lo pair): max|got - ref| <= tol * rms(ref), no rounding allowance."""
    raw = rel_max_err(got, ref)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    print("[parity] %-34s raw max|err|/rms %.3e" % (what, raw))
    RECORDS.append((what, raw, raw))
    assert raw <= tol, "%s: max|err|/rms %.4g > %.3g" % (what, raw, tol)
    return raw


def layer(w, d, block_m, train=False, weights=True):
    """Device copies of the inputs, packed weights, a workspace and the output buffer."""
    shape = moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=block_m, e_lo=w.e_lo, train=train)
    ns = SimpleNamespace(w=w, shape=shape)
    ns.idx = torch.from_numpy(np.ascontiguousarray(d["topk_idx"], np.int32)).cuda()
    ns.wts = torch.from_numpy(np.ascontiguousarray(d["topk_weights"], np.float32)).cuda()
    ns.x = bf16_dev(d["x"])
    if "dy" in d:
        ns.dy = bf16_dev(d["dy"])
    if weights:
        ns.W1p, ns.W2p = moe.alloc_packed(shape)
        W1, W2 = bf16_dev(d["W1"]), bf16_dev(d["W2"])
        moe.pack_weights(shape, W1, W2, ns.W1p, ns.W2p)
        del W1, W2
    ns.ws = moe.alloc_workspace(shape)
    ns.y = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    return ns


def unpacked(ns, dw1p, dw2p):
    """Logical [EL, H, 2I] / [EL, I, H] copies (f64, host) of packed weight gradients."""
    s = ns.shape
    W1 = torch.empty(s.EL, s.H, 2 * s.I, dtype=torch.bfloat16, device="cuda")
    W2 = torch.empty(s.EL, s.I, s.H, dtype=torch.bfloat16, device="cuda")
    moe.unpack_weights(s, dw1p, dw2p, W1, W2)
    torch.cuda.synchronize()
    return f64_host(W1), f64_host(W2)


def tables(ns):
    t = {n: moe.ws_region(ns.ws, ns.shape, n).cpu().numpy() for n in TABLES}
    meta = moe.ws_region(ns.ws, ns.shape, "meta").cpu().numpy()
    t["num_rows"], t["dropped"] = int(meta[0]), int(meta[1])
    return t


def assert_tables_equal(got, ref):
    for n in TABLES:
        assert np.array_equal(got[n], ref[n]), "table %s differs" % n
    assert got["num_rows"] == ref["num_rows"] and got["dropped"] == ref["dropped"]


def sample_tokens(tok_nloc, n, seed=0):
    """Tokens to compare at full size: some with no, one and several local pairs, plus the
    first and last token."""
    rng = np.random.default_rng(seed)
    T = len(tok_nloc)
    pick = {0, T - 1}
    for cls in (tok_nloc == 0, tok_nloc == 1, tok_nloc >= 2):
        ids = np.nonzero(cls)[0]
        if len(ids):
            pick.update(rng.choice(ids, size=min(len(ids), n // 3), replace=False).tolist())
    return np.array(sorted(pick), np.int64)
