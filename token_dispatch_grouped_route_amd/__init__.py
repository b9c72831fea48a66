"""MoE expert layer (one GPU's share of the experts) on MI355X / gfx950.

A thin binding over the C ABI of ``libmoe_gfx950.so`` (declared in ``include/moe.h``): every
function here only checks tensor dtypes/devices and passes ``data_ptr()`` values and the HIP
stream to the function of the same name (``moe_`` prefix) in the library.  All arithmetic runs
in the library's HIP kernels; there is no fallback.  PyTorch is used for device memory and
streams only.

Pipeline ("Mega MoE" page, Pipeline): route_prologue -> dispatch_gemm1 (gather + L1 NT +
SwiGLU) -> gemm2_combine (L2 NT + top-k weighted scatter-add), or ``forward`` for all of it;
the backward entry points follow the page's backward (L2 dgrad NN with the routing-weight
gradient, SwiGLU transpose, dW2 and dW1 with a variable K, L1 dgrad NN with its combine to dx).
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that the library then shares (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gfx950.so")
_lib = None

ENTRY_POINTS = (
    "moe_status_string", "moe_workspace_bytes", "moe_workspace_layout", "moe_preferred_block_m",
    "moe_pack_weights", "moe_unpack_weights", "moe_route_prologue", "moe_dispatch_gemm1", "moe_swiglu",
    "moe_gemm2_combine", "moe_forward", "moe_bwd_gemm2_dgrad", "moe_swiglu_bwd",
    "moe_bwd_gemm1_dgrad_combine", "moe_wgrad2", "moe_wgrad1", "moe_backward",
    "moe_mx_cast_fp8", "moe_mx_pack_weights", "moe_forward_mx", "moe_mx_dispatch_gemm1",
    "moe_mx_gemm2_combine", "moe_forward_noalloc",
)
NOALLOC_SCRATCH_BYTES = 256 * 1024 * 1024   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


class MoeError(RuntimeError):
    pass


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "I", "E", "e_lo", "EL", "k", "block_m", "train")]

    def __repr__(self):
        return "Shape(%s)" % ", ".join("%s=%d" % (n, getattr(self, n)) for n, _ in self._fields_)


_LAYOUT_FIELDS = ("counts", "padded_offsets", "row_pair", "pair_row", "tile_expert", "tok_nloc",
                  "meta", "act", "stage", "hgu", "dact", "dhgu", "zeros", "scratch", "tile_sync",
                  "dtw_part", "dhgu_lo", "wact", "wact_lo")


class WsLayout(ctypes.Structure):
    _fields_ = ([("total_bytes", ctypes.c_size_t), ("rows_capacity", ctypes.c_int64),
                 ("num_blocks", ctypes.c_int64)] + [(n, ctypes.c_size_t) for n in _LAYOUT_FIELDS])


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError("HIP library %s is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, S, i32 = ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.c_int32
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [i32]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [S]
        L.moe_workspace_layout.argtypes = [S, ctypes.POINTER(WsLayout)]
        L.moe_preferred_block_m.argtypes = [S]
        L.moe_pack_weights.argtypes = [S, P, P, P, P, P]
        L.moe_unpack_weights.argtypes = [S, P, P, P, P, P]
        L.moe_route_prologue.argtypes = [S, P, P, ctypes.c_size_t, P]
        L.moe_dispatch_gemm1.argtypes = [S, P, P, P, ctypes.c_size_t, P, P, P]
        L.moe_swiglu.argtypes = [S, P, P, ctypes.c_size_t, P, P]
        L.moe_gemm2_combine.argtypes = [S, P, P, P, P, ctypes.c_size_t, P, P]
        L.moe_forward.argtypes = [S, P, P, P, P, P, P, ctypes.c_size_t, P, P]
        L.moe_forward_noalloc.argtypes = [S, P, P, P, P, P, P, P]
        L.moe_bwd_gemm2_dgrad.argtypes = [S, P, P, P, P, ctypes.c_size_t, i32, P, P]
        L.moe_swiglu_bwd.argtypes = [S, P, ctypes.c_size_t, P]
        L.moe_bwd_gemm1_dgrad_combine.argtypes = [S, P, P, ctypes.c_size_t, P, P]
        L.moe_wgrad2.argtypes = [S, P, P, ctypes.c_size_t, P, P]
        L.moe_wgrad1.argtypes = [S, P, P, ctypes.c_size_t, P, P]
        L.moe_backward.argtypes = [S, P, P, P, P, P, P, ctypes.c_size_t, P, P, P, P, P]
        L.moe_mx_cast_fp8.argtypes = [ctypes.c_int64, i32, P, P, P, P]
        L.moe_mx_pack_weights.argtypes = [S, P, P, P, P, P, P, P]
        L.moe_forward_mx.argtypes = [S, P, P, P, P, P, P, P, P, ctypes.c_float, P, ctypes.c_size_t, P, P]
        L.moe_mx_dispatch_gemm1.argtypes = [S, P, P, P, P, ctypes.c_float, P, ctypes.c_size_t, P]
        L.moe_mx_gemm2_combine.argtypes = [S, P, P, P, P, ctypes.c_size_t, P, P]
        for n in ENTRY_POINTS[2:]:
            if n != "moe_workspace_bytes":
                getattr(L, n).restype = i32
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise MoeError("%s: %s (%d)" % (what, lib().moe_status_string(status).decode(), status))


def _ptr(t, dtype, name, numel=None):
    """Device address of t after checking dtype, device, contiguity and (when given) that it
    holds at least ``numel`` elements: an undersized buffer becomes an error here instead of an
    out-of-bounds access in a kernel."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise MoeError("%s must be a contiguous %s tensor on a GPU" % (name, dtype))
    if numel is not None and t.numel() < numel:
        raise MoeError("%s holds %d elements; the shape needs %d" % (name, t.numel(), numel))
    return t.data_ptr()


def _n(shape: Shape):
    """Element counts of every caller buffer of a shape (rows regions use the static bound)."""
    R = _rows_capacity(shape)
    th, tk, w1n, w2n = shape.T * shape.H, shape.T * shape.k, shape.EL * 2 * shape.I * shape.H, \
        shape.EL * shape.H * shape.I
    return {"x": th, "y": th, "dy": th, "dx": th, "topk_idx": tk, "topk_w": tk, "dtopk_w": tk,
            "w1": w1n, "w2": w2n, "w1p": w1n, "w2p": w2n, "dw1p": w1n, "dw2p": w2n,
            "act": R * shape.I, "act_out": R * shape.I, "hgu": R * 2 * shape.I, "hgu_out": R * 2 * shape.I,
            "xq": th, "xs": th // 32, "w1q": w1n // 2, "w1s": w1n // 32, "w2q": w2n // 2, "w2s": w2n // 32}


_ROWS_CAP = {}


def _rows_capacity(shape: Shape) -> int:
    key = tuple(getattr(shape, n) for n, _ in Shape._fields_)
    if key not in _ROWS_CAP:
        L = WsLayout()
        _check(lib().moe_workspace_layout(ctypes.byref(shape), ctypes.byref(L)), "moe_workspace_layout")
        _ROWS_CAP[key] = int(L.rows_capacity)
    return _ROWS_CAP[key]


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ws(ws):
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise MoeError("ws must be a contiguous GPU tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def make_shape(T, H, I, E, EL, k, block_m=None, e_lo=0, train=False) -> Shape:
    s = Shape(T, H, I, E, e_lo, EL, k, 0, int(bool(train)))
    s.block_m = block_m if block_m is not None else preferred_block_m(s)
    return s


def preferred_block_m(shape: Shape) -> int:
    return int(lib().moe_preferred_block_m(ctypes.byref(shape)))


def workspace_bytes(shape: Shape) -> int:
    n = int(lib().moe_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise MoeError("invalid shape %r" % (shape,))
    return n


def workspace_layout(shape: Shape) -> dict:
    L = WsLayout()
    _check(lib().moe_workspace_layout(ctypes.byref(shape), ctypes.byref(L)), "moe_workspace_layout")
    return {n: getattr(L, n) for n, _ in WsLayout._fields_}


def alloc_workspace(shape: Shape, device="cuda") -> torch.Tensor:
    """A workspace tensor for the shape (torch's allocator returns 512-byte aligned blocks)."""
    return torch.empty(workspace_bytes(shape), dtype=torch.uint8, device=device)


_REGION = {  # name -> (dtype, row width in elements or None)
    "counts": (torch.int32, None), "padded_offsets": (torch.int32, None),
    "row_pair": (torch.int32, None), "pair_row": (torch.int32, None),
    "tile_expert": (torch.int32, None), "tok_nloc": (torch.int32, None), "meta": (torch.int32, None),
    "act": (torch.bfloat16, "I"), "stage": (torch.float32, "H"), "hgu": (torch.float32, "2I"),
    "dact": (torch.float32, "I"), "dhgu": (torch.bfloat16, "2I"), "dhgu_lo": (torch.bfloat16, "2I"),
    "wact": (torch.bfloat16, "I"), "wact_lo": (torch.bfloat16, "I"),
    "dtw_part": (torch.float32, "I/128"),
}


def ws_region(ws: torch.Tensor, shape: Shape, name: str) -> torch.Tensor:
    """A typed view of one workspace region (no copy); row regions are [rows_capacity, width]."""
    L = workspace_layout(shape)
    R = L["rows_capacity"]
    sizes = {"counts": shape.EL, "padded_offsets": shape.EL + 1, "row_pair": R,
             "pair_row": shape.T * shape.k, "tile_expert": L["num_blocks"], "tok_nloc": shape.T,
             "meta": 4}
    dtype, width = _REGION[name]
    if width is None:
        n, view = sizes[name], None
    else:
        if name in ("hgu", "dact", "dhgu", "dhgu_lo", "wact", "wact_lo", "dtw_part") and not shape.train:
            raise MoeError("region %s exists only for train shapes" % name)
        cols = {"I": shape.I, "H": shape.H, "2I": 2 * shape.I, "I/128": shape.I // 128}[width]
        n, view = R * cols, (R, cols)
    esz = torch.tensor([], dtype=dtype).element_size()
    t = ws[L[name]:L[name] + n * esz].view(dtype)
    return t.view(*view) if view else t


def packed_sizes(shape: Shape):
    """Tensor sizes of the packed weights W1p (and dW1p) and W2p (and dW2p): one flat row of
    2I*H resp. H*I elements per expert, in the fragment-major order of moe_pack_weights."""
    return ((shape.EL, 2 * shape.I * shape.H), (shape.EL, shape.H * shape.I))


def alloc_packed(shape: Shape, device="cuda"):
    """Uninitialised (W1p, W2p) tensors of the packed sizes."""
    s1, s2 = packed_sizes(shape)
    return (torch.empty(s1, dtype=torch.bfloat16, device=device),
            torch.empty(s2, dtype=torch.bfloat16, device=device))


def pack_weights(shape, w1=None, w2=None, w1p=None, w2p=None, stream=None):
    nn = _n(shape)
    _check(lib().moe_pack_weights(ctypes.byref(shape), _ptr(w1, torch.bfloat16, "w1", nn["w1"]),
                                  _ptr(w2, torch.bfloat16, "w2", nn["w2"]), _ptr(w1p, torch.bfloat16, "w1p", nn["w1p"]),
                                  _ptr(w2p, torch.bfloat16, "w2p", nn["w2p"]), _stream(stream)), "moe_pack_weights")


def route_prologue(shape, topk_idx, ws, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_route_prologue(ctypes.byref(shape), _ptr(topk_idx, torch.int32, "topk_idx", nn["topk_idx"]), p, n,
                                    _stream(stream)), "moe_route_prologue")


def unpack_weights(shape, w1p=None, w2p=None, w1=None, w2=None, stream=None):
    """Packed (w1p, w2p) or weight gradients (dw1p, dw2p) -> logical [EL, H, 2I], [EL, I, H]."""
    nn = _n(shape)
    _check(lib().moe_unpack_weights(ctypes.byref(shape), _ptr(w1p, torch.bfloat16, "w1p", nn["w1p"]),
                                    _ptr(w2p, torch.bfloat16, "w2p", nn["w2p"]), _ptr(w1, torch.bfloat16, "w1", nn["w1"]),
                                    _ptr(w2, torch.bfloat16, "w2", nn["w2"]), _stream(stream)), "moe_unpack_weights")


def dispatch_gemm1(shape, x, w1p, ws, act_out=None, hgu_out=None, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_dispatch_gemm1(ctypes.byref(shape), _ptr(x, torch.bfloat16, "x", nn["x"]),
                                    _ptr(w1p, torch.bfloat16, "w1p", nn["w1p"]), p, n,
                                    _ptr(act_out, torch.bfloat16, "act_out", nn["act_out"]),
                                    _ptr(hgu_out, torch.float32, "hgu_out", nn["hgu_out"]), _stream(stream)),
           "moe_dispatch_gemm1")


def swiglu(shape, hgu, ws, act, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_swiglu(ctypes.byref(shape), _ptr(hgu, torch.float32, "hgu", nn["hgu"]), p, n,
                            _ptr(act, torch.bfloat16, "act", nn["act"]), _stream(stream)), "moe_swiglu")


def gemm2_combine(shape, act, w2p, topk_w, ws, y, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_gemm2_combine(ctypes.byref(shape), _ptr(act, torch.bfloat16, "act", nn["act"]),
                                   _ptr(w2p, torch.bfloat16, "w2p", nn["w2p"]), _ptr(topk_w, torch.float32, "topk_w", nn["topk_w"]),
                                   p, n, _ptr(y, torch.bfloat16, "y", nn["y"]), _stream(stream)), "moe_gemm2_combine")


def forward(shape, x, topk_idx, topk_w, w1p, w2p, ws, y, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_forward(ctypes.byref(shape), _ptr(x, torch.bfloat16, "x", nn["x"]),
                             _ptr(topk_idx, torch.int32, "topk_idx", nn["topk_idx"]), _ptr(topk_w, torch.float32, "topk_w", nn["topk_w"]),
                             _ptr(w1p, torch.bfloat16, "w1p", nn["w1p"]), _ptr(w2p, torch.bfloat16, "w2p", nn["w2p"]), p, n,
                             _ptr(y, torch.bfloat16, "y", nn["y"]), _stream(stream)), "moe_forward")


def forward_noalloc(shape, x, topk_idx, topk_w, w1p, w2p, y, stream=None):
    """moe_forward with the library's fixed device scratch instead of a workspace (allocates
    nothing; shapes whose workspace exceeds NOALLOC_SCRATCH_BYTES raise MoeError)."""
    nn = _n(shape)
    _check(lib().moe_forward_noalloc(ctypes.byref(shape), _ptr(x, torch.bfloat16, "x", nn["x"]),
                                     _ptr(topk_idx, torch.int32, "topk_idx", nn["topk_idx"]),
                                     _ptr(topk_w, torch.float32, "topk_w", nn["topk_w"]),
                                     _ptr(w1p, torch.bfloat16, "w1p", nn["w1p"]),
                                     _ptr(w2p, torch.bfloat16, "w2p", nn["w2p"]),
                                     _ptr(y, torch.bfloat16, "y", nn["y"]), _stream(stream)), "moe_forward_noalloc")


def bwd_gemm2_dgrad(shape, dy, topk_w, w2p, ws, fuse_swiglu_bwd=True, dtopk_w=None, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_bwd_gemm2_dgrad(ctypes.byref(shape), _ptr(dy, torch.bfloat16, "dy", nn["dy"]),
                                     _ptr(topk_w, torch.float32, "topk_w", nn["topk_w"]), _ptr(w2p, torch.bfloat16, "w2p", nn["w2p"]),
                                     p, n, int(bool(fuse_swiglu_bwd)), _ptr(dtopk_w, torch.float32, "dtopk_w", nn["dtopk_w"]),
                                     _stream(stream)), "moe_bwd_gemm2_dgrad")


def bwd_gemm1_dgrad_combine(shape, w1p, ws, dx, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_bwd_gemm1_dgrad_combine(ctypes.byref(shape), _ptr(w1p, torch.bfloat16, "w1p", nn["w1p"]), p, n,
                                             _ptr(dx, torch.bfloat16, "dx", nn["dx"]), _stream(stream)),
           "moe_bwd_gemm1_dgrad_combine")


def swiglu_bwd(shape, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_swiglu_bwd(ctypes.byref(shape), p, n, _stream(stream)), "moe_swiglu_bwd")


def wgrad2(shape, dy, ws, dw2p, stream=None):
    """dW2 from the weighted activation rows that bwd_gemm2_dgrad wrote into ws."""
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_wgrad2(ctypes.byref(shape), _ptr(dy, torch.bfloat16, "dy", nn["dy"]), p, n,
                            _ptr(dw2p, torch.bfloat16, "dw2p", nn["dw2p"]), _stream(stream)), "moe_wgrad2")


def wgrad1(shape, x, ws, dw1p, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_wgrad1(ctypes.byref(shape), _ptr(x, torch.bfloat16, "x", nn["x"]), p, n,
                            _ptr(dw1p, torch.bfloat16, "dw1p", nn["dw1p"]), _stream(stream)), "moe_wgrad1")


def backward(shape, x, dy, topk_w, w2p, ws, dw1p, dw2p, w1p=None, dx=None, dtopk_w=None, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_backward(ctypes.byref(shape), _ptr(x, torch.bfloat16, "x", nn["x"]), _ptr(dy, torch.bfloat16, "dy", nn["dy"]),
                              _ptr(topk_w, torch.float32, "topk_w", nn["topk_w"]), _ptr(w1p, torch.bfloat16, "w1p", nn["w1p"]),
                              _ptr(w2p, torch.bfloat16, "w2p", nn["w2p"]), p, n,
                              _ptr(dw1p, torch.bfloat16, "dw1p", nn["dw1p"]), _ptr(dw2p, torch.bfloat16, "dw2p", nn["dw2p"]),
                              _ptr(dx, torch.bfloat16, "dx", nn["dx"]), _ptr(dtopk_w, torch.float32, "dtopk_w", nn["dtopk_w"]),
                              _stream(stream)), "moe_backward")


# ------------------------------------------------------------------------------------------------
# MX variant: FP8 activations, FP4 weights, power-of-two scales per 32 values along K
# ------------------------------------------------------------------------------------------------
def mx_cast_fp8(x, codes=None, scales=None, stream=None):
    """FP8 E4M3 codes (uint8, x's shape) and UE8M0 scale bytes (uint8, [rows, cols / 32]) of bf16 x."""
    rows, cols = x.shape
    if codes is None:
        codes = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device)
    _check(lib().moe_mx_cast_fp8(rows, cols, _ptr(x, torch.bfloat16, "x"),
                                 _ptr(codes, torch.uint8, "codes", rows * cols),
                                 _ptr(scales, torch.uint8, "scales", rows * (cols // 32)), _stream(stream)),
           "moe_mx_cast_fp8")
    return codes, scales


def mx_packed_sizes(shape: Shape):
    """Byte sizes of (w1q, w1s, w2q, w2s) of moe_mx_pack_weights."""
    n1 = shape.EL * 2 * shape.I * shape.H
    n2 = shape.EL * shape.H * shape.I
    return n1 // 2, n1 // 32, n2 // 2, n2 // 32


def mx_alloc_packed(shape: Shape, device="cuda"):
    return tuple(torch.empty(n, dtype=torch.uint8, device=device) for n in mx_packed_sizes(shape))


def mx_pack_weights(shape, w1, w2, w1q, w1s, w2q, w2s, stream=None):
    nn = _n(shape)
    _check(lib().moe_mx_pack_weights(ctypes.byref(shape), _ptr(w1, torch.bfloat16, "w1", nn["w1"]),
                                     _ptr(w2, torch.bfloat16, "w2", nn["w2"]), _ptr(w1q, torch.uint8, "w1q", nn["w1q"]),
                                     _ptr(w1s, torch.uint8, "w1s", nn["w1s"]), _ptr(w2q, torch.uint8, "w2q", nn["w2q"]),
                                     _ptr(w2s, torch.uint8, "w2s", nn["w2s"]), _stream(stream)), "moe_mx_pack_weights")


def forward_mx(shape, xq, xs, topk_idx, topk_w, w1q, w1s, w2q, w2s, ws, y, clamp=10.0, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_forward_mx(ctypes.byref(shape), _ptr(xq, torch.uint8, "xq", nn["xq"]), _ptr(xs, torch.uint8, "xs", nn["xs"]),
                                _ptr(topk_idx, torch.int32, "topk_idx", nn["topk_idx"]), _ptr(topk_w, torch.float32, "topk_w", nn["topk_w"]),
                                _ptr(w1q, torch.uint8, "w1q", nn["w1q"]), _ptr(w1s, torch.uint8, "w1s", nn["w1s"]),
                                _ptr(w2q, torch.uint8, "w2q", nn["w2q"]), _ptr(w2s, torch.uint8, "w2s", nn["w2s"]), float(clamp), p, n,
                                _ptr(y, torch.bfloat16, "y", nn["y"]), _stream(stream)), "moe_forward_mx")


def mx_dispatch_gemm1(shape, xq, xs, w1q, w1s, ws, clamp=10.0, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_mx_dispatch_gemm1(ctypes.byref(shape), _ptr(xq, torch.uint8, "xq", nn["xq"]), _ptr(xs, torch.uint8, "xs", nn["xs"]),
                                       _ptr(w1q, torch.uint8, "w1q", nn["w1q"]), _ptr(w1s, torch.uint8, "w1s", nn["w1s"]), float(clamp), p,
                                       n, _stream(stream)), "moe_mx_dispatch_gemm1")


def mx_gemm2_combine(shape, w2q, w2s, topk_w, ws, y, stream=None):
    nn = _n(shape)
    p, n = _ws(ws)
    _check(lib().moe_mx_gemm2_combine(ctypes.byref(shape), _ptr(w2q, torch.uint8, "w2q", nn["w2q"]), _ptr(w2s, torch.uint8, "w2s", nn["w2s"]),
                                      _ptr(topk_w, torch.float32, "topk_w", nn["topk_w"]), p, n, _ptr(y, torch.bfloat16, "y", nn["y"]),
                                      _stream(stream)), "moe_mx_gemm2_combine")


# ------------------------------------------------------------------------------------------------
# One autograd op over the C ABI ("Mega MoE" page, Key points: the layer is one differentiable op
# that takes the routing as an input)
# ------------------------------------------------------------------------------------------------
class _MoeLayer(torch.autograd.Function):
    """y = moe_forward(x, topk_idx, topk_w, w1p, w2p) with shape.train set; backward runs
    moe_backward for dx, d(topk_w), dW1p and dW2p.  Only marshalling: every step is a library call."""

    @staticmethod
    def forward(ctx, x, topk_w, w1p, w2p, topk_idx, shape, ws):
        y = torch.empty(shape.T, shape.H, dtype=torch.bfloat16, device=x.device)
        forward(shape, x, topk_idx, topk_w, w1p, w2p, ws, y)
        ctx.save_for_backward(x, topk_w, w1p, w2p)
        ctx.shape, ctx.ws = shape, ws
        return y

    @staticmethod
    def backward(ctx, dy):
        x, topk_w, w1p, w2p = ctx.saved_tensors
        shape, ws = ctx.shape, ctx.ws
        dy = dy.contiguous()
        dw1p, dw2p = torch.empty_like(w1p), torch.empty_like(w2p)
        dx = torch.empty_like(x)
        dtw = torch.empty_like(topk_w)
        backward(shape, x, dy, topk_w, w2p, ws, dw1p, dw2p, w1p=w1p, dx=dx, dtopk_w=dtw)
        return dx, dtw, dw1p, dw2p, None, None, None


def moe_layer(x, topk_idx, topk_w, w1p, w2p, shape, ws=None):
    """The expert layer as one autograd op: y [T, H] bf16 from x [T, H] bf16, external routing
    (topk_idx int32 [T, k], topk_w fp32 [T, k]) and the packed weights (pack_weights).  Gradients
    flow to x, topk_w, w1p and w2p (the last two in the packed layout).  shape.train must be set;
    ws (alloc_workspace(shape)) holds the saved activations until backward runs, so one ws serves
    one layer call at a time."""
    if not shape.train:
        raise MoeError("moe_layer needs a train shape (the backward reads the saved activations)")
    if ws is None:
        ws = alloc_workspace(shape, x.device)
    return _MoeLayer.apply(x, topk_w, w1p, w2p, topk_idx, shape, ws)
