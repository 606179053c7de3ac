"""Seeded synthetic inputs for the MoE forward pass.

This module only draws and stores numbers: it holds none of the layer's
arithmetic (no gate, no softmax, no FFN), so both the oracle side and the HIP
side may take their inputs from it.

The pages measure on real pretraining runs and trained routers, which are not
available; these generators stand in for them with the shapes and the routing
structure of the five workloads:

* tiny top-2 MoE, fp32: T=256, d=128, E=8, k=2, GELU d_ff=256, capacity 1.25
* Mixtral-style slice, bf16: T=4096, d=4096, E=8, k=2, SwiGLU d_ff=14336,
  dropless, softmax over the two chosen logits; and the same layer on a
  decode batch of T=128 tokens (about 32 rows per expert: the expert
  weights are streamed from HBM once per step)
* fine-grained + shared expert, bf16: T=8192, d=2048, E=64, k=6, SwiGLU
  d_ff=1408, shared SwiGLU d_ff=2816, dropless; router std 1/sqrt(d) so the
  logits are about N(0,1)
* Switch-style top-1, bf16: T=16384, d=1024, E=128, GELU d_ff=4096, capacity
  1.0, an additive per-expert logit bias with std 2
* correlated top-2, bf16: T=8192, d=2048, E=64, SwiGLU d_ff=1024, dropless; 16
  hot expert pairs (0.8 % of the 2016 pairs, the share in the Abstract of
  "Expert Coupling in MoE Pretraining") get +8 on both logits for 42 % of the
  tokens, spread round-robin; the same inputs also run ExpertChoice with
  C = 2T/E.

Draw order from ``numpy.random.default_rng(seed)`` (PCG64): x, W_r, bias, W1,
W2, Ws1, Ws2.  Values are drawn in fp32 (``standard_normal(dtype=float32)``
times the std, one fp32 multiply) and rounded to nearest-even bf16 where the
workload is bf16.  bf16 arrays are carried as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

# routing modes
SOFTMAX_ALL = 0
SOFTMAX_TOPK = 1
EXPERT_CHOICE = 2
# activations
GELU = 0
SWIGLU = 1
# dtypes
F32 = 0
BF16 = 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    act: int
    dtype: int
    routing: int
    cf: float = 0.0           # 0 = dropless
    d_ff_shared: int = 0      # 0 = no shared expert
    ec_capacity: int = 0      # ExpertChoice C
    x_std: float = 1.0
    w_std: float = 0.02
    wr_std: float = 0.02
    bias: str = "none"        # none | expert | pairs
    bias_std: float = 2.0
    hot_pairs: int = 16
    hot_share: float = 0.42
    hot_boost: float = 8.0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def n_up(self) -> int:
        return 2 if self.act == SWIGLU else 1

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def assignments(self) -> int:
        return self.E * self.ec_capacity if self.routing == EXPERT_CHOICE else self.T * self.k


WORKLOADS: Dict[str, Workload] = {
    "tiny_top2_fp32": Workload("tiny_top2_fp32", T=256, d=128, E=8, k=2, d_ff=256, act=GELU,
                               dtype=F32, routing=SOFTMAX_ALL, cf=1.25),
    "mixtral_top2_bf16": Workload("mixtral_top2_bf16", T=4096, d=4096, E=8, k=2, d_ff=14336,
                                  act=SWIGLU, dtype=BF16, routing=SOFTMAX_TOPK),
    "mixtral_decode_bf16": Workload("mixtral_decode_bf16", T=128, d=4096, E=8, k=2, d_ff=14336,
                                    act=SWIGLU, dtype=BF16, routing=SOFTMAX_TOPK),
    "finegrained_shared_bf16": Workload("finegrained_shared_bf16", T=8192, d=2048, E=64, k=6,
                                        d_ff=1408, act=SWIGLU, dtype=BF16, routing=SOFTMAX_ALL,
                                        d_ff_shared=2816, wr_std=1.0 / np.sqrt(2048.0)),
    "switch_top1_bf16": Workload("switch_top1_bf16", T=16384, d=1024, E=128, k=1, d_ff=4096,
                                 act=GELU, dtype=BF16, routing=SOFTMAX_ALL, cf=1.0, bias="expert"),
    "correlated_top2_bf16": Workload("correlated_top2_bf16", T=8192, d=2048, E=64, k=2, d_ff=1024,
                                     act=SWIGLU, dtype=BF16, routing=SOFTMAX_ALL, bias="pairs"),
    "correlated_ec_bf16": Workload("correlated_ec_bf16", T=8192, d=2048, E=64, k=2, d_ff=1024,
                                   act=SWIGLU, dtype=BF16, routing=EXPERT_CHOICE,
                                   ec_capacity=8192 * 2 // 64, bias="pairs"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16, ties to even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, dtype: int, chunk_rows: int = 1) -> np.ndarray:
    """std * N(0,1) in fp32, rounded to bf16 bits when dtype is bf16.  Drawn in
    chunks along the first axis (the stream is the same as one big draw)."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, np.float32 if dtype == F32 else np.uint16)
    n0 = shape[0]
    step = max(1, chunk_rows)
    for s in range(0, n0, step):
        e = min(n0, s + step)
        v = rng.standard_normal((e - s,) + shape[1:], dtype=np.float32)
        v *= np.float32(std)
        out[s:e] = v if dtype == F32 else f32_to_bf16_bits(v)
    return out


def hot_pair_list(E: int):
    return [(a, b) for a in range(E) for b in range(a + 1, E)]


def make_inputs(w: Workload, seed: int = 0, with_experts: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """Draw every input of one workload.  Returns x, wr, bias (fp32 or None),
    bias_stride, w1 [E, n_up*d_ff, d], w2 [E, d, d_ff], ws1, ws2 (or None), and
    for the correlated workloads the hot pairs and the boosted tokens."""
    rng = np.random.default_rng(seed)
    out: Dict[str, Optional[np.ndarray]] = {}
    out["x"] = _normal(rng, (w.T, w.d), w.x_std, w.dtype, chunk_rows=4096)
    out["wr"] = _normal(rng, (w.E, w.d), w.wr_std, w.dtype, chunk_rows=w.E)
    out["bias"] = None
    out["bias_stride"] = 0
    if w.bias == "expert":
        out["bias"] = (rng.standard_normal(w.E, dtype=np.float32) * np.float32(w.bias_std)).astype(np.float32)
        out["bias_stride"] = 0
    elif w.bias == "pairs":
        pairs = hot_pair_list(w.E)
        hot = rng.choice(len(pairs), size=w.hot_pairs, replace=False)
        n_hot = int(round(w.hot_share * w.T))
        toks = rng.choice(w.T, size=n_hot, replace=False)
        b = np.zeros((w.T, w.E), np.float32)
        for i, t in enumerate(toks):
            a_, b_ = pairs[hot[i % w.hot_pairs]]
            b[t, a_] += np.float32(w.hot_boost)
            b[t, b_] += np.float32(w.hot_boost)
        out["bias"] = b
        out["bias_stride"] = w.E
        out["hot_pairs"] = np.array([pairs[h] for h in hot], np.int32)
        out["hot_tokens"] = np.asarray(toks, np.int64)
    if with_experts:
        out["w1"] = _normal(rng, (w.E, w.n_up * w.d_ff, w.d), w.w_std, w.dtype, chunk_rows=1)
        out["w2"] = _normal(rng, (w.E, w.d, w.d_ff), w.w_std, w.dtype, chunk_rows=1)
        if w.d_ff_shared:
            out["ws1"] = _normal(rng, (w.n_up * w.d_ff_shared, w.d), w.w_std, w.dtype, chunk_rows=1024)
            out["ws2"] = _normal(rng, (w.d, w.d_ff_shared), w.w_std, w.dtype, chunk_rows=1024)
        else:
            out["ws1"] = None
            out["ws2"] = None
    return out


def make_dy(w: Workload, seed: int = 0) -> np.ndarray:
    """Upstream gradient dL/dy [T, d] for the backward pass: its own stream
    (``default_rng(seed + 1000003)``), standard normal, rounded like x."""
    rng = np.random.default_rng(seed + 1000003)
    return _normal(rng, (w.T, w.d), 1.0, w.dtype, chunk_rows=4096)


def small_variant(w: Workload, **kw) -> Workload:
    """A reduced-size copy of a workload for parity runs the oracle finishes in
    seconds (same routing structure, dtype and activation)."""
    return w.replace(name=w.name + "_small", **kw)
