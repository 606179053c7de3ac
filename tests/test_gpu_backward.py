"""GPU parity of the backward pass (moe_layer_bwd through the C ABI) against
the fp64 oracle's backward.

The oracle takes the routing of the GPU's forward (its fp32 logits / scores
decide every expert choice, as in the forward parity tests) and the same dy.
Small problems are compared element by element on every gradient; the full
workloads on sampled tokens and sampled weight-gradient elements the oracle
computes one by one, plus the router's gradients from the GPU's (checked)
dlogits.  Integer outputs (padded offsets, padded row of each slot) and the
rows copied into the padded layout are compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from _parity import TOL_Y, host_float, inputs, max_rel_err, say
from mixture_experts_layer_topkrouter_amd import moe
from mixture_experts_layer_topkrouter_amd import workloads as W

WL = W.WORKLOADS

SMALL = {
    "tiny_top2_fp32": WL["tiny_top2_fp32"],
    "tiny_swiglu_fp32_ragged": W.small_variant(WL["tiny_top2_fp32"], T=203, E=5, k=3, d_ff=200, act=W.SWIGLU,
                                               cf=1.1),
    "mixtral_bwd_small": W.small_variant(WL["mixtral_top2_bf16"], T=300, d=256, d_ff=328),
    "finegrained_bwd_small": W.small_variant(WL["finegrained_shared_bf16"], T=200, d=128, E=12, d_ff=136,
                                             d_ff_shared=264, wr_std=1.0 / np.sqrt(128)),
    "switch_bwd_small": W.small_variant(WL["switch_top1_bf16"], T=500, d=128, E=16, d_ff=192),
    "correlated_ec_bwd_small": W.small_variant(WL["correlated_ec_bf16"], T=400, d=128, E=8, d_ff=160,
                                               ec_capacity=90),
    # bf16 shapes on the 256-row direct-to-LDS kernel with [K][N] operands:
    # every GEMM has partial row / column tiles
    "bwd_dma_partial_tiles": W.small_variant(WL["mixtral_top2_bf16"], T=600, d=384, E=4, d_ff=320),
    # the data-gradient GEMM dx = dz W1 contracts over 2 * 4096 = 8192: its
    # last round is cut along K and reduced in a second pass
    "bwd_ksplit_small": W.small_variant(WL["mixtral_top2_bf16"], T=256, d=128, E=2, d_ff=4096),
    # decode-sized batch: the recomputed forward GEMM runs the skinny kernel
    "bwd_decode_small": W.small_variant(WL["mixtral_top2_bf16"], T=64, d=512, E=8, d_ff=1024),
}


def _run(w: W.Workload, seed: int = 0, recompute: bool = True):
    """Forward, then backward.  recompute=False: the training forward keeps the
    expert pre-activations and the backward reads them instead of re-running
    the expert GEMM1."""
    inp = inputs(w, seed)
    cfg = moe.make_config(w)
    dev = moe.upload(inp)
    layer = moe.MoELayer(cfg, dev)
    layer.forward(train=not recompute)
    dy_np = W.make_dy(w, seed)
    dy = moe.to_device(dy_np)
    layer.backward(dy, recompute=recompute)
    torch.cuda.synchronize()
    return layer, inp, dy_np


def _oracle_fwd(w, layer, inp):
    lg = layer.view("logits").cpu().numpy()
    sc = layer.view("scores").cpu().numpy().T if w.routing == W.EXPERT_CHOICE else None
    return oracle.layer(inp["x"], inp["wr"], inp["w1"], inp["w2"], k=w.k, routing=w.routing, act=w.act, cf=w.cf,
                        ec_capacity=w.ec_capacity, bias=inp["bias"], bias_stride=inp["bias_stride"],
                        ws1=inp["ws1"], ws2=inp["ws2"], given_logits=lg, given_scores=sc, toks=np.zeros(0, np.int32))


def _check(name, got, ref, tol):
    err = max_rel_err(got, ref)
    say(f"    {name}: max rel err {err:.3e} (tol {tol})")
    assert err <= tol, f"{name}: {err}"


def _check_layout(w, layer, inp):
    """Padded offsets, the padded row of each slot, and the copied rows."""
    count = layer.view("expert_count").cpu().numpy().astype(np.int64)
    poff = layer.bwd_view("poff").cpu().numpy()
    want = np.concatenate([[0], np.cumsum((count + 31) // 32 * 32)])
    assert np.array_equal(poff, want), "padded offsets"
    sr = layer.view("slot_row").cpu().numpy().ravel()
    sp = layer.bwd_view("slot_prow").cpu().numpy()
    off = layer.view("expert_offset").cpu().numpy()
    if w.routing == W.EXPERT_CHOICE:
        e_of = sr // w.ec_capacity
        tok = np.repeat(np.arange(w.T), np.diff(layer.view("tok_ptr").cpu().numpy()))
    else:
        e_of = layer.view("topk_idx").cpu().numpy().ravel()
        tok = np.repeat(np.arange(w.T), w.k)
    exp = np.where(sr >= 0, sr - off[e_of] + poff[e_of], -1)
    assert np.array_equal(sp, exp), "slot_prow"
    xp = moe.to_host_bits(layer.bwd_view("xp"))
    kept = sp >= 0
    assert np.array_equal(xp[sp[kept]], inp["x"][tok[kept]]), "xp rows are not the token rows"
    # pad rows are zero
    pad = np.ones(poff[-1], bool)
    pad[sp[kept]] = False
    # only rows [0, poff[E]) are written: slice before converting, so the
    # unwritten tail (uninitialised memory) is never read
    assert not np.any(host_float(layer.bwd_view("xp")[:poff[-1]])[pad]), "xp pad rows"
    assert not np.any(host_float(layer.bwd_view("dyp")[:poff[-1]])[pad]), "dyp pad rows"


def _slot_w_ref(w, layer, g):
    """The oracle's dL/dw in the GPU's slot order."""
    if w.routing != W.EXPERT_CHOICE:
        return g.d_slot_w.ravel()
    sr = layer.view("slot_row").cpu().numpy()
    return g.d_slot_w[sr // w.ec_capacity, sr % w.ec_capacity]


@pytest.mark.gpu
@pytest.mark.parametrize("recompute", [True, False], ids=["recompute", "saved_z"])
@pytest.mark.parametrize("name", list(SMALL))
def test_backward_parity_small(name, recompute):
    w = SMALL[name]
    say(f"[bwd small] {name}: T={w.T} d={w.d} E={w.E} k={w.k} d_ff={w.d_ff} shared={w.d_ff_shared} "
        f"recompute={recompute}")
    layer, inp, dy = _run(w, recompute=recompute)
    if not recompute:
        # the training forward's output is the layer's output too
        ref = oracle.layer(inp["x"], inp["wr"], inp["w1"], inp["w2"], k=w.k, routing=w.routing, act=w.act, cf=w.cf,
                           ec_capacity=w.ec_capacity, bias=inp["bias"], bias_stride=inp["bias_stride"],
                           ws1=inp["ws1"], ws2=inp["ws2"], given_logits=layer.view("logits").cpu().numpy(),
                           given_scores=(layer.view("scores").cpu().numpy().T if w.routing == W.EXPERT_CHOICE
                                         else None))
        _check("y (training forward)", host_float(layer.y), ref.y, TOL_Y[w.dtype])
    _check_layout(w, layer, inp)
    fwd = _oracle_fwd(w, layer, inp)
    g = oracle.layer_bwd(inp["x"], inp["wr"], inp["w1"], inp["w2"], dy, fwd, k=w.k, routing=w.routing, act=w.act,
                         ws1=inp["ws1"], ws2=inp["ws2"])
    tol = TOL_Y[w.dtype]
    _check("d_slot_w", layer.bwd_view("d_slot_w").cpu().numpy(), _slot_w_ref(w, layer, g), tol)
    _check("dlogits", layer.bwd_view("dlogits").cpu().numpy(), g.dlogits, tol)
    _check("dx", host_float(layer.dx), g.dx, tol)
    _check("dw_router", host_float(layer.dwr), g.dwr, tol)
    _check("dw1", host_float(layer.dw1), g.dw1, tol)
    _check("dw2", host_float(layer.dw2), g.dw2, tol)
    if w.d_ff_shared:
        _check("dws1", host_float(layer.dws1), g.dws1, tol)
        _check("dws2", host_float(layer.dws2), g.dws2, tol)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["finegrained_bwd_small", "tiny_swiglu_fp32_ragged", "bwd_decode_small"])
def test_saved_mode_after_plain_forward_recomputes(name):
    """moe_layer_bwd(recompute=0) after a plain moe_layer_fwd: the forward's
    last step stamped the workspace as not holding pre-activations, so the
    device re-runs GEMM1 (routed and shared expert) and every gradient equals
    the recompute mode's bit for bit, although the workspace's pre-activation
    regions hold NaN."""
    w = SMALL[name]
    say(f"[bwd stamp] {name}")
    inp = inputs(w, 0)
    cfg = moe.make_config(w)
    layer = moe.MoELayer(cfg, moe.upload(inp))
    L = layer.layout
    layer.workspace[L["z"]:L["stamp"]].view(torch.uint8).fill_(0xFF)  # NaN bit patterns in z / shared_z
    layer.forward()
    dy = moe.to_device(W.make_dy(w, 0))
    layer.backward(dy, recompute=True)
    torch.cuda.synchronize()
    want = [t.clone() for t in (layer.dx, layer.dwr, layer.dw1, layer.dw2) + ((layer.dws1, layer.dws2)
                                                                              if w.d_ff_shared else ())]
    layer.backward(dy, recompute=False)
    torch.cuda.synchronize()
    got = (layer.dx, layer.dwr, layer.dw1, layer.dw2) + ((layer.dws1, layer.dws2) if w.d_ff_shared else ())
    for a, b in zip(got, want):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    # after a training forward the same call reads the kept pre-activations
    layer.forward(train=True)
    layer.backward(dy, recompute=False)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(t.float()).all()) for t in got)


FULL = ["tiny_top2_fp32", "mixtral_top2_bf16", "mixtral_decode_bf16", "finegrained_shared_bf16",
        "switch_top1_bf16", "correlated_ec_bf16"]


def _expert_rows(w, layer, fwd, e):
    """Tokens and gate weights of expert e's rows (oracle weights)."""
    if w.routing == W.EXPERT_CHOICE:
        rt = fwd.ec_token[e]
        return rt, oracle.softmax(fwd.logits)[rt, e]
    off = fwd.dispatch.expert_offset
    rt = fwd.dispatch.row_token[off[e]:off[e + 1]]
    rw = np.array([fwd.w[t][list(fwd.idx[t]).index(e)] for t in rt])
    return rt, rw


@pytest.mark.gpu
@pytest.mark.parametrize("name", FULL)
def test_backward_parity_full_size(name):
    """Full workloads: dx, dlogits and dL/dw on sampled tokens; sampled
    elements of each weight gradient; the router's gradients (dx term and
    dW_r) from the GPU's dlogits, whose sampled rows are checked first.
    (The bf16 workloads run the training forward and the backward that
    reads its saved pre-activations, the way the benchmark times it.)"""
    w = WL[name]
    say(f"[bwd full] {name}")
    layer, inp, dy = _run(w, recompute=w.dtype != W.BF16)
    tol = TOL_Y[w.dtype]
    _check_layout(w, layer, inp)
    lg = layer.view("logits").cpu().numpy()
    sc = layer.view("scores").cpu().numpy().T if w.routing == W.EXPERT_CHOICE else None
    rng = np.random.default_rng(3)
    toks = np.array(sorted({0, w.T - 1, *rng.choice(w.T, size=min(24, w.T), replace=False).tolist()}), np.int32)
    fwd = oracle.layer(inp["x"], inp["wr"], inp["w1"], inp["w2"], k=w.k, routing=w.routing, act=w.act, cf=w.cf,
                       ec_capacity=w.ec_capacity, bias=inp["bias"], bias_stride=inp["bias_stride"], ws1=inp["ws1"],
                       ws2=inp["ws2"], given_logits=lg, given_scores=sc, toks=np.zeros(0, np.int32))
    dx, dl, dw = oracle.layer_bwd_tokens(inp["x"], inp["wr"], inp["w1"], inp["w2"], dy, fwd, toks, k=w.k,
                                         routing=w.routing, act=w.act, ws1=inp["ws1"], ws2=inp["ws2"])
    _check("dx (sampled tokens)", host_float(layer.dx)[toks], dx, tol)
    gdl = layer.bwd_view("dlogits").cpu().numpy()
    _check("dlogits (sampled tokens)", gdl[toks], dl, tol)
    gsw = layer.bwd_view("d_slot_w").cpu().numpy()
    if w.routing == W.EXPERT_CHOICE:
        tp = layer.view("tok_ptr").cpu().numpy()
        sr = layer.view("slot_row").cpu().numpy()
        got = np.zeros((len(toks), w.E))
        for i, t in enumerate(toks):
            for s in range(tp[t], tp[t + 1]):
                got[i, sr[s] // w.ec_capacity] = gsw[s]
        _check("d_slot_w (sampled tokens)", got, dw, tol)
    else:
        _check("d_slot_w (sampled tokens)", gsw.reshape(w.T, w.k)[toks], dw, tol)
    # router: dW_r = dlogits^T x and the dx term dlogits W_r, from the GPU's dlogits
    x64 = W.bf16_bits_to_f32(inp["x"]).astype(np.float64) if w.dtype == W.BF16 else inp["x"].astype(np.float64)
    _check("dw_router (from GPU dlogits)", host_float(layer.dwr), gdl.astype(np.float64).T @ x64, tol)
    # sampled weight-gradient elements of a few experts
    n_up = 2 if w.act == W.SWIGLU else 1
    counts = layer.view("expert_count").cpu().numpy()
    experts = [int(e) for e in np.argsort(-counts)[:2]] + [int(np.argmin(np.where(counts > 0, counts, 1 << 30)))]
    for e in sorted(set(experts)):
        rt, rw = _expert_rows(w, layer, fwd, e)
        rr1 = rng.integers(0, n_up * w.d_ff, 8).astype(np.int32)
        cc1 = rng.integers(0, w.d, 8).astype(np.int32)
        ref1 = oracle.ffn_dw_elems(inp["x"], dy, inp["w1"][e], inp["w2"][e], rt, rw, w.act, 1, rr1, cc1)
        rr2 = rng.integers(0, w.d, 8).astype(np.int32)
        cc2 = rng.integers(0, w.d_ff, 8).astype(np.int32)
        ref2 = oracle.ffn_dw_elems(inp["x"], dy, inp["w1"][e], inp["w2"][e], rt, rw, w.act, 2, rr2, cc2)
        g1 = host_float(layer.dw1[e])
        g2 = host_float(layer.dw2[e])
        # relative to the largest element of the expert's gradient on the GPU
        for nm, got, ref, full in (("dw1", g1[rr1, cc1], ref1, g1), ("dw2", g2[rr2, cc2], ref2, g2)):
            err = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(full)), 1e-30))
            say(f"    {nm}[expert {e}, {len(rt)} rows] sampled: max err / max|grad| {err:.3e}")
            assert err <= tol
    if w.d_ff_shared:
        allt = np.arange(w.T, dtype=np.int32)
        rr = rng.integers(0, n_up * w.d_ff_shared, 4).astype(np.int32)
        cc = rng.integers(0, w.d, 4).astype(np.int32)
        ref = oracle.ffn_dw_elems(inp["x"], dy, inp["ws1"], inp["ws2"], allt, np.ones(w.T), w.act, 1, rr, cc)
        full = host_float(layer.dws1)
        err = float(np.max(np.abs(full[rr, cc] - ref)) / max(np.max(np.abs(full)), 1e-30))
        say(f"    dws1 sampled: {err:.3e}")
        assert err <= tol


@pytest.mark.gpu
def test_backward_is_deterministic():
    """Two backward passes on the same inputs give the same bits."""
    w = SMALL["finegrained_bwd_small"]
    layer, inp, dy = _run(w)
    first = [t.clone() for t in (layer.dx, layer.dwr, layer.dw1, layer.dw2, layer.dws1, layer.dws2)]
    layer.backward(moe.to_device(dy))
    torch.cuda.synchronize()
    for a, b in zip(first, (layer.dx, layer.dwr, layer.dw1, layer.dw2, layer.dws1, layer.dws2)):
        assert torch.equal(a, b)


@pytest.mark.gpu
def test_backward_empty_batch_zero_grads():
    """T = 0: every weight gradient is written as zero."""
    w = W.small_variant(WL["finegrained_shared_bf16"], T=0, d=128, E=4, k=2, d_ff=64, d_ff_shared=64)
    cfg = moe.make_config(w)
    inp = W.make_inputs(W.small_variant(w, T=1))
    dev = moe.upload(inp)
    x0 = dev.x[:0]
    dwr = torch.full_like(dev.wr, 7.0)
    dw1 = torch.full_like(dev.w1, 7.0)
    dw2 = torch.full_like(dev.w2, 7.0)
    dws1 = torch.full_like(dev.ws1, 7.0)
    dws2 = torch.full_like(dev.ws2, 7.0)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    moe.layer_bwd(cfg, x0, dev.wr, dev.w1, dev.w2, ws, x0, x0, dwr, dw1, dw2, ws, ws1=dev.ws1, ws2=dev.ws2,
                  dws1=dws1, dws2=dws2)
    torch.cuda.synchronize()
    for t in (dwr, dw1, dw2, dws1, dws2):
        assert not torch.any(t != 0)
