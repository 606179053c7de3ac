"""Python handle on the fp64 CPU oracle (``oracle/moe_oracle.c``): forward and
backward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It never
imports the HIP library or its binding, and the HIP path never imports it.

Inputs are numpy arrays: ``float32`` for fp32 data, ``uint16`` for bf16 bit
patterns (the C side widens either exactly to fp64).  Everything the oracle
computes is fp64.

Each wrapper names the passage it follows; the readings taken where the pages
are silent are listed at the top of ``moe_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
# a sanitizer build of the same source (tests/test_sanitizers.py) is loaded
# in place of the default one when this names it
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")

SOFTMAX_ALL = 0
SOFTMAX_TOPK = 1
EXPERT_CHOICE = 2
GELU = 0
SWIGLU = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (portable -O2, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_logits.argtypes = [i32, i32, i32, i32, P, P, P, i64, P]
    lib.orc_softmax.argtypes = [i32, i32, P, P]
    lib.orc_topk.argtypes = [i32, i32, i32, P, P]
    lib.orc_gate_weights.argtypes = [i32, i32, i32, i32, P, P, P]
    lib.orc_capacity.argtypes = [f64, i32, i32, i32]
    lib.orc_capacity.restype = i64
    lib.orc_dispatch_topk.argtypes = [i32, i32, i32, i64, P, P, P, P, P, P]
    lib.orc_dispatch_topk.restype = i64
    lib.orc_ec_select.argtypes = [i32, i32, i32, P, P]
    lib.orc_ffn_row.argtypes = [i32, i32, i32, i32, P, i64, P, i64, P, i64, P]
    lib.orc_moe_rows_topk.argtypes = [i32] * 7 + [P] * 8 + [i32, P, P]
    lib.orc_moe_rows_ec.argtypes = [i32] * 8 + [P] * 7 + [i32, P, P]
    lib.orc_ffn_row_bwd.argtypes = [i32, i32, i32, i32, P, i64, P, i64, P, i64, P, P, P, P, P]
    lib.orc_gate_bwd_topk.argtypes = [i32, i32, i32, i32, P, P, P, P]
    lib.orc_gate_bwd_ec.argtypes = [i32, i32, i32, P, P, P, P]
    lib.orc_moe_bwd_topk.argtypes = [i32] * 9 + [P] * 18
    lib.orc_moe_bwd_ec.argtypes = [i32] * 8 + [P] * 17
    lib.orc_moe_bwd_tokens_topk.argtypes = [i32] * 8 + [P] * 10 + [i32] + [P] * 4
    lib.orc_moe_bwd_tokens_ec.argtypes = [i32] * 7 + [P] * 9 + [i32] + [P] * 4
    lib.orc_ffn_dw_elems.argtypes = [i32] * 4 + [P] * 4 + [i32, P, P, i32, i32, P, P, P]
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle input must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dtype=None):
    a = np.asarray(a)
    if dtype is not None:
        a = a.astype(dtype, copy=False)
    return np.ascontiguousarray(a)


# ---------------------------------------------------------------------------
# Steps of the pass, one wrapper each.
# ---------------------------------------------------------------------------

def logits(x, wr, bias=None, bias_stride: int = 0) -> np.ndarray:
    """Router logits in fp64 ("Routing Mechanisms": one trained linear map per token)."""
    x, wr = _c(x), _c(wr)
    assert _dt(x) == _dt(wr)
    T, d = x.shape
    E = wr.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float64)
    _load().orc_logits(T, d, E, _dt(x), _ptr(x), _ptr(wr), _ptr(b), bias_stride, _ptr(out))
    return out


def softmax(lg) -> np.ndarray:
    lg = _c(lg, np.float64)
    T, E = lg.shape
    out = np.empty_like(lg)
    _load().orc_softmax(T, E, _ptr(lg), _ptr(out))
    return out


def topk(lg, k: int) -> np.ndarray:
    """Top-k experts per token by (logit desc, expert asc)."""
    lg = _c(lg, np.float64)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    _load().orc_topk(T, E, k, _ptr(lg), _ptr(idx))
    return idx


def gate_weights(lg, idx, mode: int) -> np.ndarray:
    lg, idx = _c(lg, np.float64), _c(idx, np.int32)
    T, E = lg.shape
    k = idx.shape[1]
    w = np.empty((T, k), np.float64)
    _load().orc_gate_weights(T, E, k, mode, _ptr(lg), _ptr(idx), _ptr(w))
    return w


def capacity(cf: float, T: int, k: int, E: int) -> int:
    """Capacity per expert ("Expert Parallelism > Key Parameters",
    capacity_factor); -1 for dropless."""
    return int(_load().orc_capacity(float(cf), T, k, E))


@dataclass
class Dispatch:
    slot_row: np.ndarray      # [T,k] int32, -1 = dropped
    row_token: np.ndarray     # [N] int32
    expert_count: np.ndarray  # [E] kept rows per expert
    expert_load: np.ndarray   # [E] assignments per expert before dropping
    expert_offset: np.ndarray  # [E+1]

    @property
    def n_rows(self) -> int:
        return int(self.expert_offset[-1])


def dispatch_topk(idx, E: int, cap: int) -> Dispatch:
    """token_permutation with the capacity drop rule."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    slot_row = np.empty((T, k), np.int32)
    row_token = np.full(max(T * k, 1), -1, np.int32)
    cnt = np.empty(E, np.int32)
    load = np.empty(E, np.int32)
    off = np.empty(E + 1, np.int32)
    n = _load().orc_dispatch_topk(T, E, k, cap, _ptr(idx), _ptr(slot_row), _ptr(row_token),
                                  _ptr(cnt), _ptr(load), _ptr(off))
    return Dispatch(slot_row, row_token[:n].copy(), cnt, load, off)


def ec_select(scores, C: int) -> np.ndarray:
    """ExpertChoice: the C best tokens of each expert column, ascending token."""
    s = _c(scores, np.float64)
    T, E = s.shape
    out = np.empty((E, C), np.int32)
    _load().orc_ec_select(T, E, C, _ptr(s), _ptr(out))
    return out


def ffn_row(x_row, w1_e, w2_e, act: int) -> np.ndarray:
    """One expert FFN on one row (fp64)."""
    x_row, w1_e, w2_e = _c(x_row), _c(w1_e), _c(w2_e)
    d = x_row.shape[-1]
    dff = w2_e.shape[-1]
    y = np.empty(d, np.float64)
    _load().orc_ffn_row(d, dff, act, _dt(x_row), _ptr(x_row), 0, _ptr(w1_e), 0, _ptr(w2_e), 0, _ptr(y))
    return y


def moe_rows_topk(x, idx, w, slot_row, w1, w2, act: int, toks, ws1=None, ws2=None) -> np.ndarray:
    """Layer output rows for the listed tokens, top-k routing."""
    x, idx, slot_row = _c(x), _c(idx, np.int32), _c(slot_row, np.int32)
    w = _c(w, np.float64)
    w1, w2 = _c(w1), _c(w2)
    toks = _c(toks, np.int32)
    T, d = x.shape
    E, _, dff = w2.shape
    k = idx.shape[1]
    dffs = 0 if ws2 is None else ws2.shape[-1]
    ws1 = None if ws1 is None else _c(ws1)
    ws2 = None if ws2 is None else _c(ws2)
    y = np.empty((len(toks), d), np.float64)
    _load().orc_moe_rows_topk(d, E, k, dff, dffs, act, _dt(x), _ptr(x), _ptr(idx), _ptr(w),
                              _ptr(slot_row), _ptr(w1), _ptr(w2), _ptr(ws1), _ptr(ws2),
                              len(toks), _ptr(toks), _ptr(y))
    return y


def moe_rows_ec(x, ec_token, scores, w1, w2, act: int, toks, ws1=None, ws2=None) -> np.ndarray:
    """Layer output rows for the listed tokens, ExpertChoice routing."""
    x, ec_token = _c(x), _c(ec_token, np.int32)
    scores = _c(scores, np.float64)
    w1, w2 = _c(w1), _c(w2)
    toks = _c(toks, np.int32)
    T, d = x.shape
    E, C = ec_token.shape
    dff = w2.shape[-1]
    dffs = 0 if ws2 is None else ws2.shape[-1]
    ws1 = None if ws1 is None else _c(ws1)
    ws2 = None if ws2 is None else _c(ws2)
    y = np.empty((len(toks), d), np.float64)
    _load().orc_moe_rows_ec(T, d, E, C, dff, dffs, act, _dt(x), _ptr(x), _ptr(ec_token), _ptr(scores),
                            _ptr(w1), _ptr(w2), _ptr(ws1), _ptr(ws2), len(toks), _ptr(toks), _ptr(y))
    return y


# ---------------------------------------------------------------------------
# The whole pass, composed from the steps above.
# ---------------------------------------------------------------------------

@dataclass
class LayerResult:
    logits: np.ndarray                 # [T,E] fp64 (or the fp32 logits it was given)
    idx: Optional[np.ndarray] = None   # top-k [T,k]
    w: Optional[np.ndarray] = None     # top-k weights [T,k]
    dispatch: Optional[Dispatch] = None
    scores: Optional[np.ndarray] = None  # EC softmax [T,E]
    ec_token: Optional[np.ndarray] = None  # EC [E,C]
    y: Optional[np.ndarray] = None     # [len(toks), d]
    toks: Optional[np.ndarray] = None


def layer(x, wr, w1, w2, *, k: int, routing: int, act: int, cf: float = 0.0, ec_capacity: int = 0,
          bias=None, bias_stride: int = 0, ws1=None, ws2=None, given_logits=None, given_scores=None,
          toks=None) -> LayerResult:
    """The forward pass of one MoE block ("Core MoE Layer Architecture",
    MoELayer / MoELayerExpertChoice), in fp64, for the listed tokens.

    ``given_logits`` (fp32 values) replaces the oracle's own fp64 logits for
    every decision that floating point turns into an integer; ``given_scores``
    does the same for the ExpertChoice scores."""
    T = x.shape[0]
    E = wr.shape[0]
    lg = logits(x, wr, bias, bias_stride) if given_logits is None else _c(given_logits, np.float64)
    if toks is None:
        toks = np.arange(T, dtype=np.int32)
    res = LayerResult(logits=lg, toks=np.asarray(toks, np.int32))
    if routing == EXPERT_CHOICE:
        sc = softmax(lg) if given_scores is None else _c(given_scores, np.float64)
        res.scores = sc
        res.ec_token = ec_select(sc, ec_capacity)
        # weights are the oracle's own fp64 softmax at the chosen entries
        res.y = moe_rows_ec(x, res.ec_token, softmax(lg), w1, w2, act, res.toks, ws1, ws2)
        return res
    res.idx = topk(lg, k)
    res.w = gate_weights(lg, res.idx, routing)
    res.dispatch = dispatch_topk(res.idx, E, capacity(cf, T, k, E))
    res.y = moe_rows_topk(x, res.idx, res.w, res.dispatch.slot_row, w1, w2, act, res.toks, ws1, ws2)
    return res


# ---------------------------------------------------------------------------
# Backward pass ("Activation Checkpointing and Constraints": the layer is
# trained and its forward is re-run inside the backward).  The choice of
# experts is held fixed; gradients flow through the gate weights, the expert
# FFNs and the router's linear layer.
# ---------------------------------------------------------------------------

def ffn_row_bwd(x_row, w1_e, w2_e, act: int, g):
    """Backward of one expert FFN on one row: (dW1, dW2, dx, out)."""
    x_row, w1_e, w2_e = _c(x_row), _c(w1_e), _c(w2_e)
    g = _c(g, np.float64)
    d = x_row.shape[-1]
    dff = w2_e.shape[-1]
    n_up = 2 if act == SWIGLU else 1
    dw1 = np.zeros((n_up * dff, d))
    dw2 = np.zeros((d, dff))
    dx = np.zeros(d)
    out = np.empty(d)
    _load().orc_ffn_row_bwd(d, dff, act, _dt(x_row), _ptr(x_row), 0, _ptr(w1_e), 0, _ptr(w2_e), 0,
                            _ptr(g), _ptr(dw1), _ptr(dw2), _ptr(dx), _ptr(out))
    return dw1, dw2, dx, out


def gate_bwd_topk(lg, idx, dw, mode: int) -> np.ndarray:
    """dL/dlogits from dL/d(gate weight), the expert choice held fixed."""
    lg, idx, dw = _c(lg, np.float64), _c(idx, np.int32), _c(dw, np.float64)
    T, E = lg.shape
    k = idx.shape[1]
    out = np.empty((T, E))
    _load().orc_gate_bwd_topk(T, E, k, mode, _ptr(lg), _ptr(idx), _ptr(dw), _ptr(out))
    return out


def gate_bwd_ec(lg, ec_token, dw_ec) -> np.ndarray:
    lg, ec_token, dw_ec = _c(lg, np.float64), _c(ec_token, np.int32), _c(dw_ec, np.float64)
    T, E = lg.shape
    C = ec_token.shape[1]
    out = np.empty((T, E))
    _load().orc_gate_bwd_ec(T, E, C, _ptr(lg), _ptr(ec_token), _ptr(dw_ec), _ptr(out))
    return out


@dataclass
class Grads:
    dx: np.ndarray
    dwr: np.ndarray
    dlogits: np.ndarray
    dw1: np.ndarray
    dw2: np.ndarray
    dws1: Optional[np.ndarray]
    dws2: Optional[np.ndarray]
    d_slot_w: np.ndarray  # top-k: [T,k]; ExpertChoice: [E,C]


def layer_bwd(x, wr, w1, w2, dy, fwd: LayerResult, *, k: int, routing: int, act: int,
              ws1=None, ws2=None) -> Grads:
    """Every gradient of the layer for upstream gradient dy [T,d], given the
    routing of a forward pass (``layer()``), serial fp64: small problems."""
    x, wr, w1, w2, dy = _c(x), _c(wr), _c(w1), _c(w2), _c(dy)
    T, d = x.shape
    E = wr.shape[0]
    dff = w2.shape[-1]
    n_up = 2 if act == SWIGLU else 1
    dffs = 0 if ws2 is None else ws2.shape[-1]
    ws1 = None if ws1 is None else _c(ws1)
    ws2 = None if ws2 is None else _c(ws2)
    lg = _c(fwd.logits, np.float64)
    g = Grads(dx=np.empty((T, d)), dwr=np.empty((E, d)), dlogits=np.empty((T, E)),
              dw1=np.empty((E, n_up * dff, d)), dw2=np.empty((E, d, dff)),
              dws1=np.empty((n_up * dffs, d)) if dffs else None,
              dws2=np.empty((d, dffs)) if dffs else None, d_slot_w=None)
    lib = _load()
    if routing == EXPERT_CHOICE:
        C = fwd.ec_token.shape[1]
        g.d_slot_w = np.empty((E, C))
        lib.orc_moe_bwd_ec(T, d, E, C, dff, dffs, act, _dt(x), _ptr(x), _ptr(wr), _ptr(lg),
                           _ptr(_c(fwd.ec_token, np.int32)), _ptr(w1), _ptr(w2), _ptr(ws1), _ptr(ws2),
                           _ptr(dy), _ptr(g.dx), _ptr(g.dwr), _ptr(g.dlogits), _ptr(g.dw1), _ptr(g.dw2),
                           _ptr(g.dws1), _ptr(g.dws2), _ptr(g.d_slot_w))
    else:
        g.d_slot_w = np.empty((T, k))
        lib.orc_moe_bwd_topk(T, d, E, k, dff, dffs, act, _dt(x), routing, _ptr(x), _ptr(wr), _ptr(lg),
                             _ptr(_c(fwd.idx, np.int32)), _ptr(_c(fwd.dispatch.slot_row, np.int32)),
                             _ptr(w1), _ptr(w2), _ptr(ws1), _ptr(ws2), _ptr(dy), _ptr(g.dx), _ptr(g.dwr),
                             _ptr(g.dlogits), _ptr(g.dw1), _ptr(g.dw2), _ptr(g.dws1), _ptr(g.dws2),
                             _ptr(g.d_slot_w))
    return g


def layer_bwd_tokens(x, wr, w1, w2, dy, fwd: LayerResult, toks, *, k: int, routing: int, act: int,
                     ws1=None, ws2=None):
    """dx, dlogits and dL/d(gate weight) for the listed tokens only (sampled
    checks of large problems).  ExpertChoice: the weight gradients come as
    [ntok, E] (0 where the expert did not choose the token)."""
    x, wr, w1, w2, dy = _c(x), _c(wr), _c(w1), _c(w2), _c(dy)
    toks = _c(toks, np.int32)
    T, d = x.shape
    E = wr.shape[0]
    dff = w2.shape[-1]
    dffs = 0 if ws2 is None else ws2.shape[-1]
    ws1 = None if ws1 is None else _c(ws1)
    ws2 = None if ws2 is None else _c(ws2)
    lg = _c(fwd.logits, np.float64)
    n = len(toks)
    dx = np.empty((n, d))
    dl = np.empty((n, E))
    lib = _load()
    if routing == EXPERT_CHOICE:
        C = fwd.ec_token.shape[1]
        dw = np.empty((n, E))
        lib.orc_moe_bwd_tokens_ec(d, E, C, dff, dffs, act, _dt(x), _ptr(x), _ptr(wr), _ptr(lg),
                                  _ptr(_c(fwd.ec_token, np.int32)), _ptr(w1), _ptr(w2), _ptr(ws1),
                                  _ptr(ws2), _ptr(dy), n, _ptr(toks), _ptr(dx), _ptr(dl), _ptr(dw))
    else:
        dw = np.empty((n, k))
        lib.orc_moe_bwd_tokens_topk(d, E, k, dff, dffs, act, _dt(x), routing, _ptr(x), _ptr(wr),
                                    _ptr(lg), _ptr(_c(fwd.idx, np.int32)),
                                    _ptr(_c(fwd.dispatch.slot_row, np.int32)), _ptr(w1), _ptr(w2),
                                    _ptr(ws1), _ptr(ws2), _ptr(dy), n, _ptr(toks), _ptr(dx), _ptr(dl),
                                    _ptr(dw))
    return dx, dl, dw


def ffn_dw_elems(x, dy, w1_e, w2_e, row_tok, row_w, act: int, which: int, rr, cc) -> np.ndarray:
    """Sampled elements of one expert's weight gradients (which 1: dW1[rr,cc],
    2: dW2[rr,cc]) over its rows row_tok with gate weights row_w."""
    x, dy, w1_e, w2_e = _c(x), _c(dy), _c(w1_e), _c(w2_e)
    row_tok, row_w = _c(row_tok, np.int32), _c(row_w, np.float64)
    rr, cc = _c(rr, np.int32), _c(cc, np.int32)
    d = x.shape[1]
    dff = w2_e.shape[-1]
    out = np.empty(len(rr))
    _load().orc_ffn_dw_elems(d, dff, act, _dt(x), _ptr(x), _ptr(dy), _ptr(w1_e), _ptr(w2_e), len(row_tok),
                             _ptr(row_tok), _ptr(row_w), which, len(rr), _ptr(rr), _ptr(cc), _ptr(out))
    return out
