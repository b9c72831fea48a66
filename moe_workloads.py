"""Seeded synthetic inputs for the MoE expert layer (one GPU's share of the experts).

This module is data only: it draws router logits, token activations, expert weights and
output gradients, and turns the logits into external routing (``topk_idx``/``topk_weights``),
which the layer receives as given inputs.  It holds none of the layer's own arithmetic (no
routing tables, no GEMM, no activation, no combine), so both the CPU oracle and the HIP path
can consume the same arrays without sharing any code of the method.

Workloads follow the shapes of the pages' test models:
  * DeepSeek-V3 expert shapes (hidden 7168, intermediate 2048, 256 experts, top-8, 8192 tokens
    per rank): "Mega MoE" page, Performance / Test Configuration; the page-scale share stands in
    for the rows one of its 8 ranks receives from all of them (65 536 tokens' worth).
  * DeepSeek-V2-Lite and DeepSeek-V3 as MoE model presets: "MoE training deep-dive" page,
    section 2 (Representative model configs).
  * 384 experts, top-6, hidden 7168, intermediate 3072, 4096 tokens: the "How Mega MoE Overlaps
    ..." page, code example.
The pages do not state how their tokens were routed; N(0,1) router logits (near-uniform expert
loads) and a Zipf-biased variant (skewed loads with empty experts) stand in for trained routers.

Recipe (numpy PCG64, ``default_rng([seed, stream(, expert)])``):
  stream 0: logits [T, E] fp32 ~ N(0, 1)
  stream 1: expert rank permutation for the Zipf bias (skewed workload only)
  stream 2: x [T, H] ~ N(0, 1)
  stream 3: W1[e] [H, 2I] ~ N(0, std = 1/sqrt(H)), one stream per local expert e
  stream 4: W2[e] [I, H]  ~ N(0, std = 1/sqrt(I)), one stream per local expert e
  stream 5: dy [T, H] ~ N(0, 1)
fp32 draws are rounded to bf16 (round to nearest even) and kept as uint16 bit patterns.
topk_idx = the k largest logits per token (ties to the lower expert id, slots in descending
order); topk_weights = fp32 softmax over the k selected logits.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
import os

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    H: int          # hidden
    I: int          # intermediate (L1 output width is 2*I: [gate | up])
    E: int          # experts in routing
    EL: int         # experts owned by this GPU: ids [e_lo, e_lo + EL)
    k: int          # top-k
    e_lo: int = 0
    zipf_s: float = 0.0   # > 0: per-expert Zipf(s) log-pmf bias added to the logits
    backward: bool = False

    @property
    def pairs(self) -> int:
        return self.T * self.k

    def flops_fwd(self, local_pairs: int) -> float:
        """Algorithmic forward FLOPs on the real (unpadded) rows: L1 + L2."""
        return 2.0 * local_pairs * self.H * (2 * self.I) + 2.0 * local_pairs * self.I * self.H


WORKLOADS = [
    Workload("tiny_fwd", T=256, H=256, I=128, E=8, EL=8, k=2),
    Workload("dsv2lite_fwd", T=4096, H=2048, I=1408, E=64, EL=64, k=6),
    Workload("dsv3_share_fwd", T=8192, H=7168, I=2048, E=256, EL=32, k=8),
    Workload("dsv3_share_skewed_fwd", T=8192, H=7168, I=2048, E=256, EL=32, k=8, zipf_s=1.2),
    Workload("wide_share_fwd_bwd", T=4096, H=7168, I=3072, E=384, EL=48, k=6, backward=True),
    # the rows one GPU of the pages' 8-GPU DeepSeek-V3 run receives: 8 x 8192 tokens routed
    # top-8 over 256 experts, 32 of them local (about 65 536 local rows), all resident here
    Workload("dsv3_page_share_fwd", T=65536, H=7168, I=2048, E=256, EL=32, k=8),
    # the pages' low-precision run (FP8 activations, FP4 weights): 384 experts, top-6, 4096 tokens
    # per GPU, the 48 experts of one GPU of eight
    Workload("wide_share_mx_fwd", T=4096, H=7168, I=3072, E=384, EL=48, k=6),
    # the page-scale share's training step (the pages time its backward legs at this scale)
    Workload("dsv3_page_share_fwd_bwd", T=65536, H=7168, I=2048, E=256, EL=32, k=8, backward=True),
]

_THREADS = max(1, min(16, os.cpu_count() or 1))


def get(i_or_name) -> Workload:
    if isinstance(i_or_name, int):
        return WORKLOADS[i_or_name]
    for w in WORKLOADS:
        if w.name == i_or_name:
            return w
    raise KeyError(i_or_name)


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some sizes replaced (for reduced-size test cases)."""
    return replace(w, **kw)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(seed_seq, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed_seq)
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def zipf_bias(E: int, s: float, seed: int) -> np.ndarray:
    """Per-expert logit bias: log of the finite-E Zipf(s) pmf at a random rank per expert."""
    rng = np.random.default_rng([seed, 1])
    by_rank = rng.permutation(E)              # by_rank[r] = expert holding Zipf rank r + 1
    rank = np.empty(E, dtype=np.float64)
    rank[by_rank] = np.arange(1, E + 1, dtype=np.float64)
    norm = np.sum(np.arange(1, E + 1, dtype=np.float64) ** (-s))
    return np.log(rank ** (-s) / norm).astype(np.float32)


def logits(w: Workload, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng([seed, 0])
    lg = rng.standard_normal((w.T, w.E), dtype=np.float32)
    if w.zipf_s > 0:
        lg = lg + zipf_bias(w.E, w.zipf_s, seed)[None, :]
    return lg


def routing_from_logits(lg: np.ndarray, k: int):
    """External routing input: top-k expert ids per token and softmax weights over them."""
    order = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(lg, order, axis=1).astype(np.float32)
    sel = sel - sel.max(axis=1, keepdims=True)
    ex = np.exp(sel)
    wts = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(order.astype(np.int32)), np.ascontiguousarray(wts)


def routing(w: Workload, seed: int = 0):
    return routing_from_logits(logits(w, seed), w.k)


def activations(w: Workload, seed: int = 0) -> np.ndarray:
    """x [T, H] as bf16 bits."""
    return _normal_bf16([seed, 2], (w.T, w.H), 1.0)


def grad_output(w: Workload, seed: int = 0) -> np.ndarray:
    """dy [T, H] as bf16 bits."""
    return _normal_bf16([seed, 5], (w.T, w.H), 1.0)


def weights(w: Workload, seed: int = 0, experts=None):
    """Local expert weights in the logical x @ W layouts, as bf16 bits.

    W1 [EL, H, 2I] (columns [0, I) = gate, [I, 2I) = up), W2 [EL, I, H].
    Expert e's draws depend only on (seed, e_lo + e), so a shard draws the same weights for a
    global expert id as the all-local workload does.
    """
    ex = list(range(w.EL)) if experts is None else list(experts)
    W1 = np.empty((len(ex), w.H, 2 * w.I), dtype=np.uint16)
    W2 = np.empty((len(ex), w.I, w.H), dtype=np.uint16)
    s1, s2 = 1.0 / np.sqrt(w.H), 1.0 / np.sqrt(w.I)

    def one(i):
        g = w.e_lo + ex[i]
        W1[i] = _normal_bf16([seed, 3, g], (w.H, 2 * w.I), s1)
        W2[i] = _normal_bf16([seed, 4, g], (w.I, w.H), s2)

    with ThreadPoolExecutor(_THREADS) as pool:
        list(pool.map(one, range(len(ex))))
    return W1, W2


def local_pairs(w: Workload, topk_idx: np.ndarray) -> int:
    """Number of (token, slot) pairs whose expert id lies in this GPU's range (a count of the
    input, used only to size reports)."""
    ids = topk_idx.astype(np.int64)
    return int(np.count_nonzero((ids >= w.e_lo) & (ids < w.e_lo + w.EL)))


def inputs(w: Workload, seed: int = 0, with_weights: bool = True):
    idx, wts = routing(w, seed)
    d = {"topk_idx": idx, "topk_weights": wts, "x": activations(w, seed)}
    if with_weights:
        d["W1"], d["W2"] = weights(w, seed)
    if w.backward:
        d["dy"] = grad_output(w, seed)
    return d
