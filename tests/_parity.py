"""Shared helpers of the GPU parity tests: seeded inputs, the HIP pipeline run
through the C ABI, the oracle run on the same inputs, and the comparisons.

The oracle is fed the GPU's fp32 logits (and ExpertChoice scores) for every
decision floating point turns into an integer; its own fp64 logits are
compared with the GPU's separately, within tolerance."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
from mixture_experts_layer_topkrouter_amd import moe
from mixture_experts_layer_topkrouter_amd import workloads as W

# Output tolerance: max |y - y_ref| / max |y_ref| per output tensor.
TOL_Y = {W.F32: 1e-4, W.BF16: 2e-2}
# GPU fp32 logits vs fp64 oracle logits, relative to max |logit|.
TOL_LOGITS = {W.F32: 1e-5, W.BF16: 1e-4}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def inputs(w: W.Workload, seed: int = 0):
    return W.make_inputs(w, seed)


def elem_rel_err(y, ref, floor: float = 1e-3) -> float:
    """Largest element-wise relative error, each element's |ref| floored at
    floor * max |ref| (relative error is undefined near zero)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref), floor * max(np.max(np.abs(ref)), 1e-300))
    return float(np.max(np.abs(y - ref) / den))


def tile_cover_tokens(w: W.Workload, layer, bm: int = None) -> np.ndarray:
    """Tokens whose rows include the first and the last row of every
    (expert, row tile) of the grouped GEMM: bm = 256 when the experts average
    at least 192 rows (the 256-row kernel), else 64 (the weight-streaming
    kernel's tiles).  Checking these tokens' full output rows covers every
    tile of both GEMMs, including tiles whose K range is cut into pieces."""
    off = layer.view("expert_offset").cpu().numpy().astype(np.int64)
    rt = layer.view("row_token").cpu().numpy()
    if bm is None:
        bm = 256 if moe.max_rows(layer.cfg) // w.E >= 192 else 64
    rows = []
    for e in range(w.E):
        for r0 in range(off[e], off[e + 1], bm):
            rows += [r0, min(r0 + bm, off[e + 1]) - 1]
    return np.unique(rt[np.asarray(rows, np.int64)]).astype(np.int32) if rows else np.zeros(0, np.int32)


def max_rel_err(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref)) / (den if den > 0 else 1.0))


def host_float(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_layer(w: W.Workload, seed: int = 0):
    """Runs moe_layer_fwd; returns the MoELayer (intermediates in its workspace)."""
    inp = inputs(w, seed)
    cfg = moe.make_config(w)
    dev = moe.upload(inp)
    layer = moe.MoELayer(cfg, dev)
    layer.forward()
    torch.cuda.synchronize()
    return layer, inp


def sample_tokens(w: W.Workload, n: int, extra=(), seed: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    base = {0, w.T - 1, *[int(t) for t in extra]}
    pick = rng.choice(w.T, size=min(n, w.T), replace=False).tolist()
    return np.array(sorted(base | set(pick)), np.int32)


def x_perm_rows(layer, n: int, kblocked: bool = False) -> np.ndarray:
    """The first n rows of the layer's x_perm as bf16 bits; kblocked: the
    buffer holds the K-blocked order ([d/32][rows][32]) of the packed path."""
    xp = moe.to_host_bits(layer.view("x_perm"))
    if kblocked:
        R, K = xp.shape
        xp = xp.reshape(K // 32, R, 32).transpose(1, 0, 2).reshape(R, K)
    return xp[:n]


def check_routing_topk(w: W.Workload, layer, inp, kblocked: bool = False):
    """Bit-exact routing and permutation against the oracle fed the GPU's logits."""
    lg = layer.view("logits").cpu().numpy()
    ref_lg = oracle.logits(inp["x"], inp["wr"], inp["bias"], inp["bias_stride"])
    err = np.max(np.abs(lg - ref_lg)) / max(np.max(np.abs(ref_lg)), 1e-30)
    assert err <= TOL_LOGITS[w.dtype], f"logits rel err {err}"
    idx = layer.view("topk_idx").cpu().numpy()
    ref_idx = oracle.topk(lg.astype(np.float64), w.k)
    assert np.array_equal(idx, ref_idx), "topk_idx differs from the oracle"
    tw = layer.view("topk_w").cpu().numpy()
    ref_w = oracle.gate_weights(lg.astype(np.float64), ref_idx, w.routing)
    np.testing.assert_allclose(tw, ref_w, rtol=2e-6, atol=1e-7)
    cap = oracle.capacity(w.cf, w.T, w.k, w.E)
    d = oracle.dispatch_topk(ref_idx, w.E, cap)
    assert np.array_equal(layer.view("expert_load").cpu().numpy(), d.expert_load)
    assert np.array_equal(layer.view("expert_count").cpu().numpy(), d.expert_count)
    assert np.array_equal(layer.view("expert_offset").cpu().numpy(), d.expert_offset)
    assert np.array_equal(layer.view("slot_row").cpu().numpy(), d.slot_row), "slot_row / drop mask differ"
    n = d.n_rows
    assert np.array_equal(layer.view("row_token").cpu().numpy()[:n], d.row_token)
    # x_perm rows are the token rows, bit for bit
    assert np.array_equal(x_perm_rows(layer, n, kblocked), inp["x"][d.row_token]), "x_perm is not x[row_token]"
    return lg, ref_idx, d


def check_output_topk(w: W.Workload, layer, inp, lg, toks):
    ref = oracle.layer(inp["x"], inp["wr"], inp["w1"], inp["w2"], k=w.k, routing=w.routing, act=w.act, cf=w.cf,
                       bias=inp["bias"], bias_stride=inp["bias_stride"], ws1=inp["ws1"], ws2=inp["ws2"],
                       given_logits=lg, toks=toks)
    y = host_float(layer.y)[toks]
    err = max_rel_err(y, ref.y)
    say(f"  {w.name}: output max rel err {err:.3e} over {len(toks)} tokens (tol {TOL_Y[w.dtype]}); "
        f"element-wise {elem_rel_err(y, ref.y):.3e} (floor 1e-3 max|ref|)")
    assert err <= TOL_Y[w.dtype]
    return err


def check_routing_ec(w: W.Workload, layer, inp, kblocked: bool = False):
    lg = layer.view("logits").cpu().numpy()
    ref_lg = oracle.logits(inp["x"], inp["wr"], inp["bias"], inp["bias_stride"])
    err = np.max(np.abs(lg - ref_lg)) / max(np.max(np.abs(ref_lg)), 1e-30)
    assert err <= TOL_LOGITS[w.dtype], f"logits rel err {err}"
    sc = layer.view("scores").cpu().numpy().T  # stored expert-major [E, T]
    np.testing.assert_allclose(sc, oracle.softmax(lg.astype(np.float64)), rtol=2e-6, atol=1e-9)
    ec = layer.view("ec_token").cpu().numpy()
    ref_ec = oracle.ec_select(sc.astype(np.float64), w.ec_capacity)
    assert np.array_equal(ec, ref_ec), "ec_token differs from the oracle"
    ecw = layer.view("ec_w").cpu().numpy()
    assert np.array_equal(ecw, sc[ref_ec, np.arange(w.E)[:, None]]), "ec_w is not the chosen scores"
    # permutation: row e*C+i holds ec_token[e,i]; CSR lists rows per token, ascending expert
    C = w.ec_capacity
    assert np.array_equal(layer.view("row_token").cpu().numpy(), ref_ec.ravel())
    assert np.array_equal(layer.view("expert_offset").cpu().numpy(), np.arange(w.E + 1) * C)
    tp = layer.view("tok_ptr").cpu().numpy()
    sr = layer.view("slot_row").cpu().numpy()
    sw = layer.view("slot_w").cpu().numpy()
    cnt = np.bincount(ref_ec.ravel(), minlength=w.T)
    assert np.array_equal(tp, np.concatenate([[0], np.cumsum(cnt)]))
    # the CSR lists each token's rows in ascending expert order: the rows
    # e*C+i sorted by (token, expert)
    e_of = np.repeat(np.arange(w.E), C)
    rows = np.arange(w.E * C)
    order = np.lexsort((e_of, ref_ec.ravel()))
    assert np.array_equal(sr, rows[order].astype(np.int32)), "CSR slot rows"
    assert np.array_equal(sw, ecw.ravel()[sr])
    n = w.E * C
    assert np.array_equal(x_perm_rows(layer, n, kblocked), inp["x"][ref_ec.ravel()])
    return lg, sc, ref_ec


def check_output_ec(w: W.Workload, layer, inp, lg, sc, toks):
    ref = oracle.layer(inp["x"], inp["wr"], inp["w1"], inp["w2"], k=0, routing=W.EXPERT_CHOICE, act=w.act,
                       ec_capacity=w.ec_capacity, bias=inp["bias"], bias_stride=inp["bias_stride"],
                       ws1=inp["ws1"], ws2=inp["ws2"], given_logits=lg, given_scores=sc, toks=toks)
    y = host_float(layer.y)[toks]
    err = max_rel_err(y, ref.y)
    say(f"  {w.name}: output max rel err {err:.3e} over {len(toks)} tokens (tol {TOL_Y[w.dtype]}); "
        f"element-wise {elem_rel_err(y, ref.y):.3e} (floor 1e-3 max|ref|)")
    assert err <= TOL_Y[w.dtype]
    return err
