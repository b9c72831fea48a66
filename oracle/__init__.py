"""CPU oracle of the MoE expert layer (one GPU's share of the experts).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path (the HIP library and its binding).  The arithmetic
lives in ``moe_oracle.c`` (plain C, fp64 on the bf16 input values); this module only compiles
it with gcc and marshals numpy arrays through ctypes.

Every function follows the "Mega MoE" page (Pipeline; Implementation Map) and the Block-M
alignment section of the "How Mega MoE Overlaps ..." page; see the C file for the per-function
passages and the readings taken where the pages leave a step open.

Pins (the tests that tie each function to something other than itself) are in
``tests/test_oracle.py``; no function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def configure(lib):
    """Declare the C signatures on a loaded oracle library (also used on mutated copies that
    the tests build to check that the pins catch planted mistakes)."""
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int, ctypes.c_int64
    lib.oracle_rows_capacity.restype = i64
    lib.oracle_rows_capacity.argtypes = [i32, i32, i32, i32]
    lib.oracle_num_threads.restype = i32
    lib.oracle_route.argtypes = [i32] * 6 + [P] * 8
    lib.oracle_forward.argtypes = [i32] * 7 + [P] * 5 + [P, i32, P]
    lib.oracle_l1_rows.argtypes = [i32] * 7 + [P] * 3 + [P, i32, P, P]
    lib.oracle_swiglu.argtypes = [i64, i32, P, P]
    lib.oracle_swiglu_bwd.argtypes = [i64, i32, P, P, P]
    lib.oracle_backward_rows.argtypes = [i32] * 7 + [P] * 6 + [P, i32, P, P]
    lib.oracle_backward.argtypes = [i32] * 7 + [P] * 6 + [P, i32, P, P]
    lib.oracle_backward_tokens.argtypes = [i32] * 7 + [P] * 6 + [P, i32, P, P]
    lib.oracle_mx_quantize.argtypes = [i32, i64, P, P, P]
    lib.oracle_mx_dequantize.argtypes = [i32, i64, P, P, P]
    lib.oracle_forward_mx.argtypes = [i32] * 7 + [P] * 8 + [ctypes.c_double, i32, P, i32, P]
    lib.oracle_mx_l1_rows.argtypes = [i32] * 7 + [P] * 5 + [ctypes.c_double, P, i32, P]
    lib.oracle_mx_l2_rows.argtypes = [i32] * 3 + [P] * 3 + [i32, P, P, P]
    for f in ("oracle_route", "oracle_forward", "oracle_l1_rows", "oracle_swiglu",
              "oracle_swiglu_bwd", "oracle_backward_rows", "oracle_backward",
              "oracle_backward_tokens", "oracle_mx_quantize", "oracle_mx_dequantize",
              "oracle_forward_mx", "oracle_mx_l1_rows", "oracle_mx_l2_rows"):
        getattr(lib, f).restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = configure(ctypes.CDLL(build()))
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def rows_capacity(T: int, k: int, EL: int, BM: int) -> int:
    return int(_load().oracle_rows_capacity(T, k, EL, BM))


def route(topk_idx, E: int, e_lo: int, EL: int, BM: int) -> dict:
    """Routing tables of the dispatch prologue (all int32, -1 = no entry)."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    R = rows_capacity(T, k, EL, BM)
    out = {
        "counts": np.zeros(EL, np.int32),
        "padded_offsets": np.zeros(EL + 1, np.int32),
        "row_pair": np.zeros(R, np.int32),
        "pair_row": np.zeros(T * k, np.int32),
        "tile_expert": np.zeros(R // BM, np.int32),
        "tok_nloc": np.zeros(T, np.int32),
    }
    meta = np.zeros(2, np.int32)
    rc = _load().oracle_route(T, k, E, e_lo, EL, BM, _p(idx), _p(out["counts"]),
                              _p(out["padded_offsets"]), _p(out["row_pair"]), _p(out["pair_row"]),
                              _p(out["tile_expert"]), _p(out["tok_nloc"]), _p(meta))
    if rc != 0:
        raise ValueError("oracle_route failed: %d" % rc)
    out["num_rows"] = int(meta[0])
    out["dropped"] = int(meta[1])
    return out


def _shape(x, W1, W2, topk_idx):
    T, H = x.shape
    EL, H1, N = W1.shape
    I = N // 2
    assert H1 == H and W2.shape == (EL, I, H), "weights must be [EL,H,2I] and [EL,I,H]"
    assert topk_idx.shape[0] == T
    return T, H, I, EL, topk_idx.shape[1]


def forward(x, topk_idx, topk_w, W1, W2, E: int, e_lo: int = 0, tokens=None) -> np.ndarray:
    """y rows (fp64, [len(tokens), H]) for the given tokens (default: all)."""
    x, idx, w = _c(x, np.uint16), _c(topk_idx, np.int32), _c(topk_w, np.float32)
    W1, W2 = _c(W1, np.uint16), _c(W2, np.uint16)
    T, H, I, EL, k = _shape(x, W1, W2, idx)
    tok = _c(np.arange(T) if tokens is None else tokens, np.int32)
    y = np.zeros((len(tok), H), np.float64)
    rc = _load().oracle_forward(T, H, I, E, e_lo, EL, k, _p(x), _p(idx), _p(w), _p(W1), _p(W2),
                                _p(tok), len(tok), _p(y))
    if rc != 0:
        raise MemoryError("oracle_forward failed: %d" % rc)
    return y


def l1_rows(x, topk_idx, W1, E: int, e_lo: int, pairs):
    """Pre-activation [gate | up] rows h [n, 2I] and SwiGLU rows a [n, I] for given pair ids."""
    x, idx, W1 = _c(x, np.uint16), _c(topk_idx, np.int32), _c(W1, np.uint16)
    T, H = x.shape
    EL, _, N = W1.shape
    I, k = N // 2, idx.shape[1]
    pr = _c(pairs, np.int32)
    h = np.zeros((len(pr), N), np.float64)
    a = np.zeros((len(pr), I), np.float64)
    _load().oracle_l1_rows(T, H, I, E, e_lo, EL, k, _p(x), _p(idx), _p(W1), _p(pr), len(pr), _p(h), _p(a))
    return h, a


def _rows_values(hgu):
    """[gate | up] rows as fp64 values: uint16 arrays are bf16 bit patterns, anything else is
    taken as real values (e.g. fp32 rows)."""
    a = np.asarray(hgu)
    if a.dtype == np.uint16:
        return (np.ascontiguousarray(a).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return _c(a, np.float64)


def swiglu(hgu) -> np.ndarray:
    """silu(gate) * up on [gate | up] rows (bf16 bits or real values); returns fp64 [n, I]."""
    hgu = _rows_values(hgu)
    n, N = hgu.shape
    a = np.zeros((n, N // 2), np.float64)
    _load().oracle_swiglu(n, N // 2, _p(hgu), _p(a))
    return a


def swiglu_bwd(hgu, da) -> np.ndarray:
    """Gradient of silu(gate) * up w.r.t. [gate | up] (rows as bf16 bits or real values) for an
    upstream gradient da (fp64 values, [n, I])."""
    hgu, da = _rows_values(hgu), _c(da, np.float64)
    n, N = hgu.shape
    assert da.shape == (n, N // 2)
    d = np.zeros((n, N), np.float64)
    _load().oracle_swiglu_bwd(n, N // 2, _p(hgu), _p(da), _p(d))
    return d


def backward_rows(x, topk_idx, topk_w, W1, W2, dy, E: int, e_lo: int, pairs):
    """Per-pair L2 dgrad dA [n, I] and SwiGLU-transposed dHgu [n, 2I] for given pair ids."""
    x, idx, w = _c(x, np.uint16), _c(topk_idx, np.int32), _c(topk_w, np.float32)
    W1, W2, dy = _c(W1, np.uint16), _c(W2, np.uint16), _c(dy, np.uint16)
    T, H, I, EL, k = _shape(x, W1, W2, idx)
    pr = _c(pairs, np.int32)
    dA = np.zeros((len(pr), I), np.float64)
    dh = np.zeros((len(pr), 2 * I), np.float64)
    rc = _load().oracle_backward_rows(T, H, I, E, e_lo, EL, k, _p(x), _p(idx), _p(w), _p(W1), _p(W2),
                                      _p(dy), _p(pr), len(pr), _p(dA), _p(dh))
    if rc != 0:
        raise MemoryError("oracle_backward_rows failed: %d" % rc)
    return dA, dh


def backward(x, topk_idx, topk_w, W1, W2, dy, E: int, e_lo: int = 0, experts=None):
    """dW1 [n, H, 2I] and dW2 [n, I, H] (fp64, logical layouts) for the given local experts."""
    x, idx, w = _c(x, np.uint16), _c(topk_idx, np.int32), _c(topk_w, np.float32)
    W1, W2, dy = _c(W1, np.uint16), _c(W2, np.uint16), _c(dy, np.uint16)
    T, H, I, EL, k = _shape(x, W1, W2, idx)
    ex = _c(np.arange(EL) if experts is None else experts, np.int32)
    dW1 = np.zeros((len(ex), H, 2 * I), np.float64)
    dW2 = np.zeros((len(ex), I, H), np.float64)
    rc = _load().oracle_backward(T, H, I, E, e_lo, EL, k, _p(x), _p(idx), _p(w), _p(W1), _p(W2),
                                 _p(dy), _p(ex), len(ex), _p(dW1), _p(dW2))
    if rc != 0:
        raise MemoryError("oracle_backward failed: %d" % rc)
    return dW1, dW2


def backward_tokens(x, topk_idx, topk_w, W1, W2, dy, E: int, e_lo: int = 0, tokens=None):
    """Token-side gradients for the given tokens (default: all): dx [n, H] (the L1 dgrad rows
    summed back to token order) and dtopk_w [n, k] (<dy[t], o_p> for each local pair, else 0),
    fp64."""
    x, idx, w = _c(x, np.uint16), _c(topk_idx, np.int32), _c(topk_w, np.float32)
    W1, W2, dy = _c(W1, np.uint16), _c(W2, np.uint16), _c(dy, np.uint16)
    T, H, I, EL, k = _shape(x, W1, W2, idx)
    tok = _c(np.arange(T) if tokens is None else tokens, np.int32)
    dx = np.zeros((len(tok), H), np.float64)
    dw = np.zeros((len(tok), k), np.float64)
    rc = _load().oracle_backward_tokens(T, H, I, E, e_lo, EL, k, _p(x), _p(idx), _p(w), _p(W1),
                                        _p(W2), _p(dy), _p(tok), len(tok), _p(dx), _p(dw))
    if rc != 0:
        raise MemoryError("oracle_backward_tokens failed: %d" % rc)
    return dx, dw


MX_FP8, MX_FP4 = 0, 1


def mx_quantize(fmt: int, values):
    """Cast values (last axis a multiple of 32) in blocks of 32 along the last axis: codes (uint8,
    one code per byte, same shape) and UE8M0 scale bytes (shape [..., n / 32]).  fmt: MX_FP8
    (E4M3) or MX_FP4 (E2M1)."""
    v = _c(values, np.float64)
    codes = np.zeros(v.shape, np.uint8)
    scales = np.zeros(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    if _load().oracle_mx_quantize(fmt, v.size, _p(v), _p(codes), _p(scales)) != 0:
        raise ValueError("mx_quantize: the last axis must be a multiple of 32")
    return codes, scales


def mx_dequantize(fmt: int, codes, scales) -> np.ndarray:
    c, sc = _c(codes, np.uint8), _c(scales, np.uint8)
    v = np.zeros(c.shape, np.float64)
    if _load().oracle_mx_dequantize(fmt, c.size, _p(c), _p(sc), _p(v)) != 0:
        raise ValueError("mx_dequantize: the last axis must be a multiple of 32")
    return v


def forward_mx(x_codes, x_scales, topk_idx, topk_w, w1_codes, w1_scales, w2_codes, w2_scales, E: int,
               e_lo: int = 0, clamp: float = 10.0, quant_act: bool = True, tokens=None) -> np.ndarray:
    """MX forward (fp64) for the given tokens on quantized inputs: x [T, H] FP8 codes + [T, H/32]
    scales; W1 as [EL, 2I, H] FP4 codes + [EL, 2I, H/32] scales (column-major: blocks along H);
    W2 as [EL, H, I] codes + [EL, H, I/32] scales.  clamp <= 0 disables the SwiGLU clamp."""
    xc, xs = _c(x_codes, np.uint8), _c(x_scales, np.uint8)
    idx, w = _c(topk_idx, np.int32), _c(topk_w, np.float32)
    w1c, w1s, w2c, w2s = (_c(a, np.uint8) for a in (w1_codes, w1_scales, w2_codes, w2_scales))
    T, H = xc.shape
    EL, N, _ = w1c.shape
    I, k = N // 2, idx.shape[1]
    assert w2c.shape == (EL, H, I) and xs.shape == (T, H // 32)
    tok = _c(np.arange(T) if tokens is None else tokens, np.int32)
    y = np.zeros((len(tok), H), np.float64)
    rc = _load().oracle_forward_mx(T, H, I, E, e_lo, EL, k, _p(xc), _p(xs), _p(idx), _p(w), _p(w1c), _p(w1s),
                                   _p(w2c), _p(w2s), float(clamp), int(bool(quant_act)), _p(tok), len(tok),
                                   _p(y))
    if rc != 0:
        raise MemoryError("oracle_forward_mx failed: %d" % rc)
    return y


def mx_l1_rows(x_codes, x_scales, topk_idx, w1_codes, w1_scales, E: int, e_lo: int, pairs, clamp=10.0):
    """MX L1 rows a [n, I] (fp64, before the FP8 cast of the activation) for given pair ids."""
    xc, xs, idx = _c(x_codes, np.uint8), _c(x_scales, np.uint8), _c(topk_idx, np.int32)
    w1c, w1s = _c(w1_codes, np.uint8), _c(w1_scales, np.uint8)
    T, H = xc.shape
    EL, N, _ = w1c.shape
    pr = _c(pairs, np.int32)
    a = np.zeros((len(pr), N // 2), np.float64)
    rc = _load().oracle_mx_l1_rows(T, H, N // 2, E, e_lo, EL, idx.shape[1], _p(xc), _p(xs), _p(idx), _p(w1c),
                                   _p(w1s), float(clamp), _p(pr), len(pr), _p(a))
    if rc != 0:
        raise MemoryError("oracle_mx_l1_rows failed: %d" % rc)
    return a


def mx_l2_rows(w2_codes, w2_scales, experts, act_codes, act_scales):
    """MX L2 rows o [n, H] (fp64, unweighted) of given FP8 activation rows and their local experts."""
    w2c, w2s = _c(w2_codes, np.uint8), _c(w2_scales, np.uint8)
    EL, H, I = w2c.shape
    ex, ac, as_ = _c(experts, np.int32), _c(act_codes, np.uint8), _c(act_scales, np.uint8)
    o = np.zeros((len(ex), H), np.float64)
    rc = _load().oracle_mx_l2_rows(H, I, EL, _p(w2c), _p(w2s), _p(ex), len(ex), _p(ac), _p(as_), _p(o))
    if rc != 0:
        raise MemoryError("oracle_mx_l2_rows failed: %d" % rc)
    return o
