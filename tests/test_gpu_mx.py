"""GPU parity of the MX variant (FP8 activations, FP4 weights, power-of-two scales per 32 values
along K) against the CPU oracle, through the C ABI.  The casts are integer results and must match
bit for bit: both sides round the same exactly scaled values."""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import token_dispatch_grouped_route_amd as moe
from gpu_helpers import bf16_dev

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
    ((n mod I) / 32) * 64 + (n >= I) * 32 + n mod 32)."""
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    pc = ((n % I) // 32) * 64 + (n >= I) * 32 + n % 32 if I is not None else n
    blk = (pc // 32) * (K // 64) + k // 64
    lane = pc % 32 + 32 * ((k % 64) // 32)
    byte = (blk * 64 + lane) * 16 + (k % 32) // 2
    shift = 4 * ((k % 32) % 2)
    sidx = (blk * 64 + lane)[:, ::32]
    codes = np.zeros((EL, N, K), np.uint8)
    scales = np.zeros((EL, N, K // 32), np.uint8)
    for e in range(EL):
        d = wq[e * N * K // 2:(e + 1) * N * K // 2]
        codes[e] = (d[byte] >> shift) & 15
        scales[e] = ws[e * N * K // 32:(e + 1) * N * K // 32][sidx]
    return codes, scales


@pytest.mark.parametrize("shape", [(3, 256, 128), (2, 384, 256)])
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
