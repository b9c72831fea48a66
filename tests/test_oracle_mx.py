"""Pins of the oracle's MX variant (FP8 activations, FP4 weights, power-of-two scales per 32
values along K; "How Mega MoE Overlaps ..." page, Code Example), CPU only.

Each pin ties the oracle to something other than itself: PyTorch's own float8_e4m3fn cast (an
independent library routine for OCP FP8 rounding), a brute-force nearest-value search over the
eight FP4 magnitudes, the defining inequalities of the block exponent, the reduction of the MX
forward to the already pinned bf16 forward on dequantized inputs, and a dense torch composition
for the SwiGLU clamp.  Planted mistakes in a copy of the oracle must fail a pin.
"""
import ctypes
import subprocess

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_workloads as mw
import oracle

FP8, FP4 = oracle.MX_FP8, oracle.MX_FP4
E2M1_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def bf16_bits(v):
    """bf16 bit patterns of values that bf16 represents exactly (asserted)."""
    f = np.asarray(v, np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(v, np.float64)), "value not exact in fp32"
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def pin_fp8_matches_torch(seed=0):
    rng = np.random.default_rng(seed)
    v = rng.uniform(-448, 448, size=(400, 32))
    v[:, 0] = 448.0                      # block amax 448: exponent 0, codes = the cast itself
    v[0, 1:9] = [0, -0.0, 1e-6, -1e-6, 2 ** -9, 3 * 2 ** -10, 0.5 * (1 + 1.125), 17.0]   # ties, subnormals
    codes, scales = oracle.mx_quantize(FP8, v)
    assert np.all(scales == 127)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref), "FP8 codes differ from torch float8_e4m3fn"


def pin_fp4_brute_force(seed=1):
    rng = np.random.default_rng(seed)
    v = rng.uniform(-6, 6, size=(300, 32))
    v[:, 0] = 6.0
    v[0, 1:16] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -2.5, -5.0, 4.9, 0.0, 3.1, 5.5]
    codes, scales = oracle.mx_quantize(FP4, v)
    assert np.all(scales == 127)
    for val, c in zip(v.ravel(), codes.ravel()):
        a = abs(val)
        d = [abs(a - m) for m in E2M1_MAG]
        best = min(d)
        cands = [i for i, x in enumerate(d) if x == best]
        want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]   # tie: even mantissa
        assert c & 7 == want, (val, c)
        assert (c >> 3) == (1 if (val < 0 or (val == 0 and np.signbit(val))) else 0)


def pin_block_exponent(seed=2):
    rng = np.random.default_rng(seed)
    for fmt, vmax in ((FP8, 448.0), (FP4, 6.0)):
        v = rng.standard_normal((500, 32)) * np.exp(rng.uniform(-20, 20, size=(500, 1)))
        v[3] = 0.0
        codes, scales = oracle.mx_quantize(fmt, v)
        E = scales.astype(np.int64) - 127
        amax = np.abs(v).max(axis=1)
        nz = amax > 0
        assert np.all(amax[nz] <= vmax * 2.0 ** E[nz, 0])          # nothing saturates
        assert np.all(amax[nz] > vmax * 2.0 ** (E[nz, 0] - 1))     # the smallest such exponent
        assert scales[3, 0] == 127 and np.all(codes[3] == 0)
        dq = oracle.mx_dequantize(fmt, codes, scales)
        # round to nearest: the error is at most half the spacing at the block's largest binade
        mb = 3 if fmt == FP8 else 1
        assert np.all(np.abs(dq - v) <= 2.0 ** (np.floor(np.log2(vmax)) - mb - 1 + E) + 1e-300)


def quantized_layer(w, d):
    """MX codes of a workload's inputs: x per token (blocks along H), W1 per output column (blocks
    along H), W2 per output column (blocks along I)."""
    x = mw.bf16_bits_to_f32(d["x"]).astype(np.float64)
    W1 = mw.bf16_bits_to_f32(d["W1"]).astype(np.float64)          # [EL, H, 2I]
    W2 = mw.bf16_bits_to_f32(d["W2"]).astype(np.float64)          # [EL, I, H]
    xc, xs = oracle.mx_quantize(FP8, x)
    w1c, w1s = oracle.mx_quantize(FP4, np.ascontiguousarray(W1.transpose(0, 2, 1)))   # [EL, 2I, H]
    w2c, w2s = oracle.mx_quantize(FP4, np.ascontiguousarray(W2.transpose(0, 2, 1)))   # [EL, H, I]
    return xc, xs, w1c, w1s, w2c, w2s


def pin_mx_forward_reduces_to_bf16_forward(seed=4):
    """Without the activation cast and the clamp, the MX forward is the bf16 forward of the
    dequantized inputs (which bf16 holds exactly)."""
    w = mw.Workload("mx", T=40, H=128, I=64, E=8, EL=4, k=2, e_lo=2)
    d = mw.inputs(w, seed)
    xc, xs, w1c, w1s, w2c, w2s = quantized_layer(w, d)
    y = oracle.forward_mx(xc, xs, d["topk_idx"], d["topk_weights"], w1c, w1s, w2c, w2s, E=w.E, e_lo=w.e_lo,
                          clamp=0, quant_act=False)
    xq = bf16_bits(oracle.mx_dequantize(FP8, xc, xs))
    W1q = bf16_bits(oracle.mx_dequantize(FP4, w1c, w1s).transpose(0, 2, 1))
    W2q = bf16_bits(oracle.mx_dequantize(FP4, w2c, w2s).transpose(0, 2, 1))
    ref = oracle.forward(xq, d["topk_idx"], d["topk_weights"], W1q, W2q, E=w.E, e_lo=w.e_lo)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def pin_clamp_and_act_cast_dense(seed=5):
    """k = 1, weight 1, activations large enough to clamp: a dense torch composition (clamp, silu,
    the activation cast through this module's quantizer) per expert."""
    w = mw.Workload("mxc", T=48, H=64, I=32, E=4, EL=4, k=1)
    d = mw.inputs(w, seed)
    d["x"] = mw.f32_to_bf16_bits(mw.bf16_bits_to_f32(d["x"]) * 12.0)   # pre-activations reach past 10
    xc, xs, w1c, w1s, w2c, w2s = quantized_layer(w, d)
    wts = np.ones((w.T, 1), np.float32)
    y = oracle.forward_mx(xc, xs, d["topk_idx"], wts, w1c, w1s, w2c, w2s, E=w.E, clamp=10.0, quant_act=True)
    X = torch.from_numpy(oracle.mx_dequantize(FP8, xc, xs))
    W1 = torch.from_numpy(oracle.mx_dequantize(FP4, w1c, w1s)).transpose(1, 2)
    W2 = torch.from_numpy(oracle.mx_dequantize(FP4, w2c, w2s)).transpose(1, 2)
    ref = np.zeros_like(y)
    clamped = 0
    for e in range(w.EL):
        rows = np.nonzero(d["topk_idx"][:, 0] == e)[0]
        if len(rows) == 0:
            continue
        h = X[rows] @ W1[e]
        clamped += int((h[:, :w.I] > 10).sum() + (h[:, w.I:].abs() > 10).sum())
        a = F.silu(h[:, :w.I].clamp(max=10.0)) * h[:, w.I:].clamp(-10.0, 10.0)
        ac, as_ = oracle.mx_quantize(FP8, a.numpy())
        ref[rows] = (torch.from_numpy(oracle.mx_dequantize(FP8, ac, as_)) @ W2[e]).numpy()
    assert clamped > 0, "the case must exercise the clamp"
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_mx_rows_compose_to_the_mx_forward():
    """L1 rows, the FP8 cast of each row, L2 rows and the weighted sum per token reproduce the MX
    forward (the row functions the GPU parity tests use link by link)."""
    w = mw.Workload("mxr", T=36, H=128, I=64, E=9, EL=3, k=3, e_lo=2)
    d = mw.inputs(w, 7)
    xc, xs, w1c, w1s, w2c, w2s = quantized_layer(w, d)
    y = oracle.forward_mx(xc, xs, d["topk_idx"], d["topk_weights"], w1c, w1s, w2c, w2s, E=w.E, e_lo=w.e_lo)
    pairs = np.arange(w.T * w.k)
    a = oracle.mx_l1_rows(xc, xs, d["topk_idx"], w1c, w1s, w.E, w.e_lo, pairs)
    ac, as_ = oracle.mx_quantize(FP8, a)
    ids = d["topk_idx"].reshape(-1) - w.e_lo
    ex = np.where((ids >= 0) & (ids < w.EL), ids, -1)
    o = oracle.mx_l2_rows(w2c, w2s, ex, ac, as_)
    ref = (o * d["topk_weights"].reshape(-1, 1).astype(np.float64)).reshape(w.T, w.k, w.H).sum(axis=1)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(y))
    assert np.all(a[ex < 0] == 0) and np.all(o[ex < 0] == 0)


def test_fp8_cast_matches_torch_float8_e4m3fn():
    pin_fp8_matches_torch()


def test_fp4_cast_is_nearest_with_ties_to_even():
    pin_fp4_brute_force()


def test_block_exponent_is_the_smallest_without_saturation():
    pin_block_exponent()


def test_mx_round_trip_of_representable_values():
    for fmt, ebits, mbits, bias in ((FP8, 4, 3, 7), (FP4, 2, 1, 1)):
        n = 1 << (1 + ebits + mbits)
        codes = np.arange(n, dtype=np.uint8)
        if fmt == FP8:
            codes = codes[(codes & 0x7F) != 0x7F]      # the two NaN codes
        codes = np.concatenate([codes, np.zeros((-len(codes)) % 32, np.uint8)]).reshape(-1, 32)
        scales = np.full((codes.shape[0], 1), 127, np.uint8)
        v = oracle.mx_dequantize(fmt, codes, scales)
        vmax = 448.0 if fmt == FP8 else 6.0
        assert np.max(np.abs(v)) == vmax
        v[:, 0] = vmax                                  # keep every block at exponent 0
        codes[:, 0] = oracle.mx_quantize(fmt, v)[0][:, 0]
        c2, s2 = oracle.mx_quantize(fmt, v)
        assert np.all(s2 == 127) and np.array_equal(c2, codes)


def test_mx_forward_reduces_to_bf16_forward():
    pin_mx_forward_reduces_to_bf16_forward()


def test_mx_forward_clamp_and_activation_cast():
    pin_clamp_and_act_cast_dense()


def test_mx_forward_token_subset_and_non_local():
    w = mw.Workload("mxs", T=30, H=64, I=32, E=10, EL=3, k=3, e_lo=4)
    d = mw.inputs(w, 6)
    q = quantized_layer(w, d)
    args = (q[0], q[1], d["topk_idx"], d["topk_weights"]) + q[2:]
    y = oracle.forward_mx(*args, E=w.E, e_lo=w.e_lo)
    sub = np.array([5, 0, 29])
    assert np.array_equal(oracle.forward_mx(*args, E=w.E, e_lo=w.e_lo, tokens=sub), y[sub])
    local = (d["topk_idx"] >= w.e_lo) & (d["topk_idx"] < w.e_lo + w.EL)
    assert np.all(y[~local.any(axis=1)] == 0)


MUTATIONS = [
    ("exact powers take one exponent too many", "while (E < 127 && amax > vmax * pow2i(E)) ++E;",
     "while (E < 127 && amax >= vmax * pow2i(E)) ++E;", pin_fp8_matches_torch),
    ("ties to the odd mantissa", "(err == best_err && (m & 1) == 0)", "(err == best_err && (m & 1) == 1)",
     pin_fp8_matches_torch),
    ("FP4 ties to the odd mantissa", "(err == best_err && (m & 1) == 0)", "(err == best_err && (m & 1) == 1)",
     pin_fp4_brute_force),
    ("clamp of up on one side only", "if (u < -clamp) u = -clamp;", "", pin_clamp_and_act_cast_dense),
    ("activation cast skipped", "if (quant_act) {", "if (0) {", pin_clamp_and_act_cast_dense),
    ("W2 blocks along the wrong axis", "w2_scales + row * (I / 32), wr);", "w2_scales + (size_t)e * H * (I / 32) + m % (I / 32), wr);",
     pin_mx_forward_reduces_to_bf16_forward),
]


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mx_pins_catch_planted_mistake(name, old, new, pin, tmp_path, monkeypatch):
    src = open(oracle._SRC).read()
    assert old in src, "mutation anchor not found: " + name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(mutated), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.configure(ctypes.CDLL(str(so))))
    with pytest.raises(AssertionError):
        pin()
