"""GPU parity of the MX variant (FP8 activations, FP4 weights, power-of-two scales per 32 values
along K) against the CPU oracle, through the C ABI.  The casts are integer results and must match
bit for bit: both sides round the same exactly scaled values."""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import token_dispatch_grouped_route_amd as moe
from gpu_helpers import RECORDS, bf16_dev, bf16_half_ulp, check_bf16, f64_host, rel_max_err

pytestmark = pytest.mark.gpu
FP8, FP4 = oracle.MX_FP8, oracle.MX_FP4


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def special_rows(rng, T, H):
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0] = 0.0                                    # a zero row: exponent 0, all codes zero
    x[1, :64] = -0.0
    x[2] *= 1e-30                                 # tiny: exponents near the bottom
    x[3] *= 1e30                                  # huge
    x[4, :32] = np.arange(32) * 0.5 + 0.25        # values that round at ties after scaling
    x[5, ::3] = -x[5, ::3] * 1000
    return mw.f32_to_bf16_bits(x)


@pytest.mark.parametrize("T,H", [(37, 256), (300, 7168)])
def test_fp8_cast_bit_exact(T, H):
    bits = special_rows(np.random.default_rng(T), T, H)
    codes, scales = moe.mx_cast_fp8(bf16_dev(bits))
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(FP8, mw.bf16_bits_to_f32(bits).astype(np.float64))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def unpack_fp4(wq, ws, EL, N, K, I=None):
    """Codes [EL, N, K] and scales [EL, N, K / 32] in logical column order, read through the layout
    documented for moe_mx_pack_weights (I given: W1, whose column n is packed column
    ((n mod I) / 32) * 64 + (n >= I) * 32 + n mod 32; the scales of a column group hold four
    64-deep K steps per lane dword)."""
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    pc = ((n % I) // 32) * 64 + (n >= I) * 32 + n % 32 if I is not None else n
    j = k // 64
    blk = (pc // 32) * (K // 64) + j
    lane = pc % 32 + 32 * ((k % 64) // 32)
    byte = (blk * 64 + lane) * 16 + (k % 32) // 2
    shift = 4 * ((k % 32) % 2)
    sidx = ((pc // 32) * (K // 64) * 64 + (j // 4) * 256 + lane * 4 + j % 4)[:, ::32]
    codes = np.zeros((EL, N, K), np.uint8)
    scales = np.zeros((EL, N, K // 32), np.uint8)
    for e in range(EL):
        d = wq[e * N * K // 2:(e + 1) * N * K // 2]
        codes[e] = (d[byte] >> shift) & 15
        scales[e] = ws[e * N * K // 32:(e + 1) * N * K // 32][sidx]
    return codes, scales


@pytest.mark.parametrize("shape", [(3, 256, 256), (2, 768, 512)])
def test_fp4_pack_bit_exact_in_documented_layout(shape):
    EL, H, I = shape
    w = mw.Workload("mxpack", T=8, H=H, I=I, E=EL, EL=EL, k=1)
    W1, W2 = mw.weights(w, 3)
    W1[0, :64, 5] = 0                              # a zero block
    W1[1, :, 7] = mw.f32_to_bf16_bits(mw.bf16_bits_to_f32(W1[1, :, 7]) * 3000.0)   # large blocks
    s = moe.make_shape(8, H, I, EL, EL, 1, block_m=64)
    w1q, w1s, w2q, w2s = moe.mx_alloc_packed(s)
    moe.mx_pack_weights(s, bf16_dev(W1), bf16_dev(W2), w1q, w1s, w2q, w2s)
    torch.cuda.synchronize()
    for W, q, sc, N, K, Iarg in ((W1, w1q, w1s, 2 * I, H, I), (W2, w2q, w2s, H, I, None)):
        codes, scales = unpack_fp4(q.cpu().numpy(), sc.cpu().numpy(), EL, N, K, Iarg)
        Wt = np.ascontiguousarray(mw.bf16_bits_to_f32(W).astype(np.float64).transpose(0, 2, 1))   # [EL, N, K]
        rc, rs = oracle.mx_quantize(FP4, Wt)
        assert np.array_equal(scales, rs)
        assert np.array_equal(codes, rc)


REDUCED = [
    mw.Workload("mx_shard", T=333, H=256, I=256, E=12, EL=6, k=3, e_lo=3),
    mw.Workload("mx_all_local", T=500, H=512, I=256, E=8, EL=8, k=4),
]
U32 = 2.0 ** -24          # unit roundoff of fp32
FP8_MAX = 448.0


def oracle_weight_codes(W, experts):
    """The oracle's FP4 codes and scales of bf16 weights W [EL, K, N] in [EL, N, K] order, for the
    listed experts only (zero elsewhere)."""
    EL, K, N = W.shape
    codes, scales = np.zeros((EL, N, K), np.uint8), np.zeros((EL, N, K // 32), np.uint8)
    for e in experts:
        Wt = np.ascontiguousarray(mw.bf16_bits_to_f32(W[e]).astype(np.float64).T)
        codes[e], scales[e] = oracle.mx_quantize(FP4, Wt)
    return codes, scales


def mx_layer(w, d, bm, x_scale=1.0, experts=None):
    """Device inputs of the MX forward: x cast on the GPU, weights packed on the GPU; the oracle's
    codes of the same inputs (bit-identical, by the tests above), for the given local experts
    (all by default)."""
    s = moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=bm, e_lo=w.e_lo)
    xbits = d["x"] if x_scale == 1.0 else mw.f32_to_bf16_bits(mw.bf16_bits_to_f32(d["x"]) * x_scale)
    xq, xs = moe.mx_cast_fp8(bf16_dev(xbits))
    w1q, w1s, w2q, w2s = moe.mx_alloc_packed(s)
    moe.mx_pack_weights(s, bf16_dev(d["W1"]), bf16_dev(d["W2"]), w1q, w1s, w2q, w2s)
    ws = moe.alloc_workspace(s)
    y = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    idx = torch.from_numpy(np.ascontiguousarray(d["topk_idx"], np.int32)).cuda()
    wts = torch.from_numpy(np.ascontiguousarray(d["topk_weights"], np.float32)).cuda()
    oc = oracle.mx_quantize(FP8, mw.bf16_bits_to_f32(xbits).astype(np.float64))
    experts = range(w.EL) if experts is None else experts
    ref_codes = oc + oracle_weight_codes(d["W1"], experts) + oracle_weight_codes(d["W2"], experts)
    return s, (xq, xs, idx, wts, w1q, w1s, w2q, w2s, ws, y), ref_codes


def gpu_act(ws, s, w):
    """The FP8 activation rows the MX forward leaves in the workspace's act region (codes
    [R_max, I], then the scale bytes slot-major, [I / 256][R_max][8]), as [R_max, I] codes and
    [R_max, I / 32] scales, and the pair id of each row."""
    L = moe.workspace_layout(s)
    R, off = L["rows_capacity"], L["act"]
    codes = ws[off:off + R * w.I].cpu().numpy().reshape(R, w.I)
    slots = ws[off + R * w.I:off + R * w.I + R * (w.I // 32)].cpu().numpy().reshape(w.I // 256, R, 8)
    scales = np.ascontiguousarray(slots.transpose(1, 0, 2)).reshape(R, w.I // 32)
    return codes, scales, moe.ws_region(ws, s, "row_pair").cpu().numpy()


def fp8_half_step(v, scale_codes):
    """Half the spacing of FP8 E4M3 values (times the block's scale) at the magnitude of each v."""
    sc = np.exp2(np.repeat(scale_codes.astype(np.float64) - 127, 32, axis=-1))
    mag = np.abs(v) / sc
    e = np.maximum(np.floor(np.log2(np.maximum(mag, 2.0 ** -30))), -6)   # subnormals share 2**-9
    return 0.5 * np.exp2(e - 3) * sc


# Accuracy of the gfx950 scaled MFMA (32x32x64, FP8 x FP4): one instruction's result differs from
# the exact C + sum of its 64 products by up to EPS_MMA * (sum |products| + |C|); the instruction
# sums well below fp32 precision.  The K loop chains the instructions through C, so a dot product
# of K terms errs by up to EPS_MMA * sum over 64-deep steps s of (S_s + |C_s|), C_s being the
# partial sum before step s.  test_mx_chained_mfma_error_within_eps_mma measures the constant on
# the product path (the MX L2 GEMM's fp32 results) and checks that it holds.
EPS_MMA = 2.0 ** -12


def chained_mma_bound(x, w):
    """Error bound of the chained scaled MFMA for the dot products of rows x[i] and w[i]."""
    p = (x * w).reshape(len(x), -1, 64)
    steps = p.sum(axis=2)
    c = np.cumsum(steps, axis=1) - steps        # partial sum entering each step
    return EPS_MMA * (np.abs(p).sum(axis=2) + np.abs(c)).sum(axis=1)


def act_delta(w, d, ref_codes, pairs, ri, ci, a, clamp):
    """Bound on |GPU activation before its FP8 cast - exact activation| at elements (ri, ci) of the
    rows of the given pair ids (a: the exact rows): the chained MFMA bounds of gate and up carried
    through the derivatives of the clamped SwiGLU, plus a few fp32 ulps for the activation itself."""
    xc, xs, w1c, w1s = ref_codes[:4]
    p = pairs[ri]
    t, e = p // w.k, d["topk_idx"].reshape(-1)[p] - w.e_lo
    xr = oracle.mx_dequantize(FP8, xc[t], xs[t])
    wg = oracle.mx_dequantize(FP4, w1c[e, ci], w1s[e, ci])
    wu = oracle.mx_dequantize(FP4, w1c[e, w.I + ci], w1s[e, w.I + ci])
    g, u = np.sum(xr * wg, axis=1), np.sum(xr * wu, axis=1)
    bg, bu = chained_mma_bound(xr, wg), chained_mma_bound(xr, wu)
    if clamp > 0:
        g, u = np.minimum(g, clamp), np.clip(u, -clamp, clamp)
    sg = 1.0 / (1.0 + np.exp(-g))
    return bg * np.abs(u * sg * (1 + g * (1 - sg))) + bu * np.abs(g * sg) + 16 * U32 * np.abs(a[ri, ci])


def check_act_link(w, d, ref_codes, pairs, gc, gs, clamp=10.0):
    """L1 link: the GPU's FP8 activation rows for the given pair ids against the oracle's fp64 L1.
    The GPU decides each code on a value its matrix core computed with the error bound above, the
    oracle on an exact one, so a code may differ where the two values straddle a rounding
    boundary.  Every GPU value must be the FP8 rounding, at the GPU's block scale, of a value within
    delta of the oracle's: the bounds of gate and up carried through the derivatives of the clamped
    SwiGLU, plus a few fp32 ulps for the activation itself.  Block scales must agree unless the
    block maximum lies within its delta of a boundary 448 * 2**E."""
    xc, xs, w1c, w1s = ref_codes[:4]
    a = oracle.mx_l1_rows(xc, xs, d["topk_idx"], w1c, w1s, w.E, w.e_lo, pairs, clamp)
    rc, rs = oracle.mx_quantize(FP8, a)
    smis = gs != rs
    check = (gc != rc) | np.repeat(smis, 32, axis=1)
    print("[parity] act codes: %d of %d differ, %d of %d block scales" % (np.sum(gc != rc), gc.size,
                                                                        smis.sum(), smis.size))
    assert check.mean() <= 5e-3, "too many activation codes differ"
    ri, ci = np.nonzero(check)
    if len(ri):
        delta = act_delta(w, d, ref_codes, pairs, ri, ci, a, clamp)
        gv = oracle.mx_dequantize(FP8, gc, gs)[ri, ci]
        over = np.abs(a[ri, ci] - gv) - fp8_half_step(gv[:, None], gs[ri, ci // 32][:, None])[:, 0] - delta
        print("[parity] act codes outside their rounding interval by at most %.3f of delta" % np.max(
            (np.abs(a[ri, ci] - gv) - fp8_half_step(gv[:, None], gs[ri, ci // 32][:, None])[:, 0]) / delta))
        assert np.all(over <= 0), "activation code outside its rounding interval by %.3g" % over.max()
        if smis.any():
            bi, bj = np.nonzero(smis)
            amax = np.abs(a).reshape(len(a), -1, 32).max(axis=2)[bi, bj]
            edge = FP8_MAX * np.exp2(np.minimum(gs, rs)[bi, bj].astype(np.float64) - 127)
            dmax = np.zeros(smis.shape)
            np.maximum.at(dmax, (ri, ci // 32), delta)
            assert np.all(np.abs(amax - edge) <= dmax[bi, bj]), "block scale differs away from a boundary"


def check_l2_link(w, d, ref_codes, y, tokens, pair_row, gc, gs):
    """L2 + combine link: y of the given tokens against the oracle's L2 evaluated on the GPU's own
    FP8 activation rows, weighted and summed per token, to the same bar as the bf16 forward
    (2e-2 of rms beyond y's own rounding to bf16)."""
    w2c, w2s = ref_codes[4:]
    ref = np.zeros((len(tokens), w.H))
    for j in range(w.k):
        p = tokens * w.k + j
        r = pair_row[p]
        e = np.where(r >= 0, d["topk_idx"][tokens, j] - w.e_lo, -1).astype(np.int32)
        rr = np.maximum(r, 0)
        o = oracle.mx_l2_rows(w2c, w2s, e, gc[rr], gs[rr])
        ref += d["topk_weights"][tokens, j].astype(np.float64)[:, None] * o
    return check_bf16(y[tokens], ref, 2e-2, "y (MX, on the GPU's act)")


def check_end_to_end(w, d, ref_codes, y, tokens, pair_row, gc, gs, clamp=10.0, what=""):
    """End to end: y of the given tokens against the oracle's own MX forward (its activation codes
    decided on exact L1 values).  The GPU decides each activation code on a value its matrix core
    computed within delta of the exact one (act_delta), so a code may differ from the oracle's where
    the two values fall on either side of a rounding boundary: the two decoded values then differ
    by at most delta plus half an FP8 step at each of them (check_act_link admits only such codes).
    Each element of y may also differ by the effect of its token's rows' differing codes: that
    bound times |w_j| * |W2[e_j][i, m]|, summed over the differing codes i.  The bar is the
    forward's (2e-2 * rms beyond y's own rounding to bf16) plus that allowance, per element."""
    xc, xs, w1c, w1s, w2c, w2s = ref_codes
    ref = oracle.forward_mx(xc, xs, d["topk_idx"], d["topk_weights"], w1c, w1s, w2c, w2s, E=w.E, e_lo=w.e_lo,
                            clamp=clamp, tokens=tokens)
    allow = np.zeros((len(tokens), w.H))
    w2_cache = {}
    nflip = 0
    for j in range(w.k):
        p = tokens * w.k + j
        r = pair_row[p]
        sel = np.nonzero(r >= 0)[0]
        if len(sel) == 0:
            continue
        a = oracle.mx_l1_rows(xc, xs, d["topk_idx"], w1c, w1s, w.E, w.e_lo, p[sel], clamp)
        rc, rs = oracle.mx_quantize(FP8, a)
        g_c, g_s = gc[r[sel]], gs[r[sel]]
        flip = (g_c != rc) | np.repeat(g_s != rs, 32, axis=1)
        if not flip.any():
            continue
        ri, ci = np.nonzero(flip)
        ga = oracle.mx_dequantize(FP8, g_c, g_s)[ri, ci]
        ra = oracle.mx_dequantize(FP8, rc, rs)[ri, ci]
        bound = (act_delta(w, d, ref_codes, p[sel], ri, ci, a, clamp) +
                 fp8_half_step(ga[:, None], g_s[ri, ci // 32][:, None])[:, 0] +
                 fp8_half_step(ra[:, None], rs[ri, ci // 32][:, None])[:, 0])
        assert np.all(np.abs(ga - ra) <= bound), "a differing activation code outside its bound"
        nflip += len(ri)
        for n in np.unique(ri):
            e = int(d["topk_idx"][tokens[sel[n]], j]) - w.e_lo
            if e not in w2_cache:
                w2_cache[e] = np.abs(oracle.mx_dequantize(FP4, w2c[e], w2s[e]))   # [H, I]
            m = ri == n
            wj = abs(float(d["topk_weights"][tokens[sel[n]], j]))
            allow[sel[n]] += wj * (w2_cache[e][:, ci[m]] @ bound[m])
    rms = np.sqrt(np.mean(ref * ref))
    own = bf16_half_ulp(np.maximum(np.abs(y[tokens]), np.abs(ref)))
    diff = np.abs(y[tokens] - ref)
    beyond = max(float(np.max(diff - own - allow)), 0.0) / rms if diff.size else 0.0
    raw = rel_max_err(y[tokens], ref)
    print("[parity] y (MX end to end%s): %d differing codes, error beyond rounding and code allowance "
          "%.3e, raw max|err|/rms %.3e" % (what, nflip, beyond, raw))
    RECORDS.append(("y (MX end to end%s)" % what, beyond, raw))
    assert beyond <= 2e-2, "MX y differs from the oracle beyond rounding and codes by %.3g of rms" % beyond


def run_mx_forward(w, d, bm, x_scale=1.0, clamp=10.0, experts=None):
    s, args, ref_codes = mx_layer(w, d, bm, x_scale, experts)
    moe.forward_mx(s, *args, clamp=clamp)
    torch.cuda.synchronize()
    gc, gs, row_pair = gpu_act(args[8], s, w)
    pair_row = moe.ws_region(args[8], s, "pair_row").cpu().numpy()
    return f64_host(args[-1]), ref_codes, gc, gs, row_pair, pair_row


@pytest.mark.parametrize("bm", [32, 64, 128, 256])
@pytest.mark.parametrize("w", REDUCED, ids=[r.name for r in REDUCED])
def test_mx_forward_reduced_link_by_link(w, bm):
    d = mw.inputs(w, 21)
    y, ref_codes, gc, gs, row_pair, pair_row = run_mx_forward(w, d, bm)
    assert np.all(np.isfinite(y))
    rows = np.nonzero(row_pair >= 0)[0]
    local = (d["topk_idx"] >= w.e_lo) & (d["topk_idx"] < w.e_lo + w.EL)
    assert len(rows) == local.sum()
    check_act_link(w, d, ref_codes, row_pair[rows], gc[rows], gs[rows])
    check_l2_link(w, d, ref_codes, y, np.arange(w.T), pair_row, gc, gs)
    assert np.all(y[~local.any(axis=1)] == 0.0)
    check_end_to_end(w, d, ref_codes, y, np.arange(w.T), pair_row, gc, gs, what=", %s, bm %d" % (w.name, bm))


def test_mx_forward_clamp_active():
    w = REDUCED[1]
    d = mw.inputs(w, 22)
    y, ref_codes, gc, gs, row_pair, pair_row = run_mx_forward(w, d, 64, x_scale=12.0)
    rows = np.nonzero(row_pair >= 0)[0]
    check_act_link(w, d, ref_codes, row_pair[rows], gc[rows], gs[rows], clamp=10.0)
    check_l2_link(w, d, ref_codes, y, np.arange(w.T), pair_row, gc, gs)
    check_end_to_end(w, d, ref_codes, y, np.arange(w.T), pair_row, gc, gs, clamp=10.0, what=", clamp active")
    xc, xs, w1c, w1s = ref_codes[:4]
    a10 = oracle.mx_l1_rows(xc, xs, d["topk_idx"], w1c, w1s, w.E, w.e_lo, row_pair[rows], 10.0)
    a0 = oracle.mx_l1_rows(xc, xs, d["topk_idx"], w1c, w1s, w.E, w.e_lo, row_pair[rows], 0.0)
    assert np.mean(a10 != a0) > 0.05, "the case must exercise the clamp"


def test_mx_forward_full_size_sampled():
    """The pages' low-precision workload on one GPU's share (384 experts, top-6, H 7168, I 3072,
    4096 tokens, 48 experts local), sampled tokens checked link by link."""
    w = mw.get("wide_share_mx_fwd")
    d = mw.inputs(w, 0)
    print("[mx full] inputs ready", flush=True)
    nloc = ((d["topk_idx"] >= w.e_lo) & (d["topk_idx"] < w.e_lo + w.EL)).sum(axis=1)
    tok = np.sort(np.random.default_rng(5).choice(np.nonzero(nloc)[0], 16, replace=False))
    sel = d["topk_idx"][tok]
    experts = sorted(set((sel[(sel >= w.e_lo) & (sel < w.e_lo + w.EL)] - w.e_lo).tolist()))
    bm = moe.preferred_block_m(moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=64, e_lo=w.e_lo))
    y, ref_codes, gc, gs, row_pair, pair_row = run_mx_forward(w, d, bm, experts=experts)
    print("[mx full] forward done, oracle codes of %d experts ready" % len(experts), flush=True)
    assert np.all(np.isfinite(y))
    assert np.all(y[nloc == 0] == 0.0)
    pairs = (tok[:, None] * w.k + np.arange(w.k)[None, :]).reshape(-1)
    pairs = pairs[pair_row[pairs] >= 0]
    r = pair_row[pairs]
    assert np.array_equal(row_pair[r], pairs)
    check_act_link(w, d, ref_codes, pairs, gc[r], gs[r])
    print("[mx full] act link done", flush=True)
    check_l2_link(w, d, ref_codes, y, tok, pair_row, gc, gs)
    check_end_to_end(w, d, ref_codes, y, tok, pair_row, gc, gs, what=", %s, sampled tokens" % w.name)


def test_mx_chained_mfma_error_within_eps_mma():
    """EPS_MMA pinned on the product path.  With every token holding 4 local pairs, the MX L2 GEMM's
    combine stages every row's fp32 result times the routing weight in ws stage; divided by the
    weight, that is the chained scaled-MFMA dot product of the GPU's own FP8 activation row with the
    FP4 W2 column (K = I, 64-deep steps).  Against the exact fp64 value (the oracle's L2 row on the
    same codes) the error must stay within EPS_MMA * sum over steps of (S_s + |C_s|), plus a few fp32
    ulps for the weight's multiply and divide.  The largest error / that sum (the effective
    per-instruction unit) and the mean are printed."""
    w = REDUCED[1]
    d = mw.inputs(w, 25)
    s, args, ref_codes = mx_layer(w, d, 64)
    moe.forward_mx(s, *args)
    torch.cuda.synchronize()
    ws = args[8]
    gc, gs, row_pair = gpu_act(ws, s, w)
    stage = moe.ws_region(ws, s, "stage").cpu().numpy()
    rows = np.nonzero(row_pair >= 0)[0][:192]
    p = row_pair[rows]
    wts = d["topk_weights"].reshape(-1)[p].astype(np.float64)
    assert np.all(((d["topk_idx"] >= w.e_lo) & (d["topk_idx"] < w.e_lo + w.EL)).sum(axis=1) >= 2)
    got = stage[rows].astype(np.float64) / wts[:, None]
    e = (d["topk_idx"].reshape(-1)[p] - w.e_lo).astype(np.int32)
    w2c, w2s = ref_codes[4:]
    exact = oracle.mx_l2_rows(w2c, w2s, e, gc[rows], gs[rows])
    a = oracle.mx_dequantize(FP8, gc[rows], gs[rows])
    W2 = {int(x): oracle.mx_dequantize(FP4, w2c[x], w2s[x]) for x in np.unique(e)}   # [H, I]
    unit = np.zeros_like(exact)
    for n in range(len(rows)):
        unit[n] = chained_mma_bound(np.broadcast_to(a[n], W2[int(e[n])].shape), W2[int(e[n])]) / EPS_MMA
    err = np.abs(got - exact)
    eff = err / np.maximum(unit, 1e-300)
    print("[parity] chained scaled MFMA over %d dot products of K = %d: max error / sum_s(S_s + |C_s|) = "
          "2^%.2f (mean 2^%.2f); EPS_MMA = 2^-12" % (err.size, w.I, np.log2(eff.max()), np.log2(eff.mean())))
    RECORDS.append(("MX chained MFMA: max error / sum_s(S_s + |C_s|), K = %d" % w.I, float(eff.max()),
                    float(eff.mean())))
    assert np.all(err <= EPS_MMA * unit + 4 * U32 * np.abs(exact)), "the chained MFMA error exceeds EPS_MMA"


def test_mx_stage_entry_points_match_the_fused_forward():
    """route_prologue + mx_dispatch_gemm1 + mx_gemm2_combine give the fused MX forward's y bit for bit."""
    w = REDUCED[0]
    d = mw.inputs(w, 23)
    s, args, _ = mx_layer(w, d, 32, experts=[])
    xq, xs, idx, wts, w1q, w1s, w2q, w2s, ws, y = args
    moe.forward_mx(s, *args)
    y2 = torch.full_like(y, float("nan"))
    moe.route_prologue(s, idx, ws)
    moe.mx_dispatch_gemm1(s, xq, xs, w1q, w1s, ws)
    moe.mx_gemm2_combine(s, w2q, w2s, wts, ws, y2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_mx_rejects_unsupported_shapes():
    """H and I must be multiples of 256 for the pack and every MX GEMM entry point."""
    w = mw.Workload("mx_bad", T=16, H=128, I=256, E=4, EL=4, k=2)
    d = mw.inputs(w, 1)
    s = moe.make_shape(w.T, w.H, w.I, w.E, w.EL, w.k, block_m=32)
    w1q, w1s, w2q, w2s = moe.mx_alloc_packed(s)
    with pytest.raises(moe.MoeError, match="size"):
        moe.mx_pack_weights(s, bf16_dev(d["W1"]), bf16_dev(d["W2"]), w1q, w1s, w2q, w2s)
    xq, xs = moe.mx_cast_fp8(bf16_dev(d["x"]))
    idx = torch.from_numpy(np.ascontiguousarray(d["topk_idx"], np.int32)).cuda()
    wts = torch.from_numpy(np.ascontiguousarray(d["topk_weights"], np.float32)).cuda()
    ws = moe.alloc_workspace(s)
    y = torch.empty(w.T, w.H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="size"):
        moe.forward_mx(s, xq, xs, idx, wts, w1q, w1s, w2q, w2s, ws, y)
    with pytest.raises(moe.MoeError, match="size"):
        moe.mx_dispatch_gemm1(s, xq, xs, w1q, w1s, ws)
    with pytest.raises(moe.MoeError, match="size"):
        moe.mx_gemm2_combine(s, w2q, w2s, wts, ws, y)
    torch.cuda.synchronize()


def test_mx_forward_is_deterministic_and_graph_capturable():
    """Two eager MX forwards give the same y bit for bit; the MX forward captured into a HIP graph
    replays it bit for bit over a stale workspace, with eager work between the replays."""
    w = REDUCED[0]
    d = mw.inputs(w, 24)
    s, args, _ = mx_layer(w, d, 64, experts=[])
    *inputs, ws, y = args
    y0 = torch.empty_like(y)
    moe.forward_mx(s, *inputs, ws, y0)
    moe.forward_mx(s, *inputs, ws, y)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y.view(torch.int16))
    yg = torch.full_like(y, float("nan"))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        moe.forward_mx(s, *inputs, ws, yg)   # warm up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            moe.forward_mx(s, *inputs, ws, yg)
    torch.cuda.current_stream().wait_stream(stream)
    for i in range(3):
        yg.fill_(float("nan"))
        ws.fill_(0x7f)   # stale workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg.view(torch.int16), y0.view(torch.int16)), "replay %d differs" % i
        moe.forward_mx(s, *inputs, ws, y)   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("case", ["empty_batch", "none_local", "one_expert_takes_all"])
def test_mx_degenerate_routing(case):
    """No tokens at all; tokens none of whose pairs this GPU handles (y exactly zero); every pair on
    one expert (several M tiles of one expert, checked link by link)."""
    w = mw.Workload("mx_degenerate", T=96, H=256, I=256, E=12, EL=4, k=2, e_lo=4)
    if case == "empty_batch":
        w = mw.scaled(w, T=0)
    d = mw.inputs(w, 15)
    idx = d["topk_idx"].copy()
    if case == "none_local":
        idx = np.where((idx >= w.e_lo) & (idx < w.e_lo + w.EL), idx + w.EL, idx) % w.E
        idx = np.where((idx >= w.e_lo) & (idx < w.e_lo + w.EL), 0, idx).astype(np.int32)
    elif case == "one_expert_takes_all":
        idx[:] = w.e_lo + 2
    d = dict(d, topk_idx=idx)
    y, ref_codes, gc, gs, row_pair, pair_row = run_mx_forward(w, d, 64)
    local = (idx >= w.e_lo) & (idx < w.e_lo + w.EL)
    rows = np.nonzero(row_pair >= 0)[0]
    assert len(rows) == int(local.sum())
    if w.T == 0:
        return
    if case == "none_local":
        assert np.all(y == 0.0)
        return
    check_act_link(w, d, ref_codes, row_pair[rows], gc[rows], gs[rows])
    check_l2_link(w, d, ref_codes, y, np.arange(w.T), pair_row, gc, gs)
    check_end_to_end(w, d, ref_codes, y, np.arange(w.T), pair_row, gc, gs, what=", " + case)
