"""Pins for the oracle's backward pass, against things other than the oracle's
own backward code:

* central finite differences of the oracle's fp64 FORWARD pass, on inputs
  chosen on a binary grid so that every perturbed value is exact in fp32;
* torch.autograd (fp64, CPU), which derives the gradients of the same forward
  by itself;
* closed forms of the softmax gradient and invariants that hold for any input.

Each test names the mistake it is there to catch.  Throughout, the choice of
experts (top-k, ExpertChoice, capacity drops) is held fixed: it is a
piecewise-constant function of the logits, and every finite-difference test
asserts that its perturbations leave it unchanged."""
import numpy as np
import pytest
import torch

import oracle

H = 2.0 ** -14  # finite-difference step; every perturbed input stays exact in fp32


def _grid(rng, shape, den, lim):
    """fp32 values m/den, |m| <= lim: exact, and still exact after +-H."""
    return (rng.integers(-lim, lim + 1, size=shape) / den).astype(np.float32)


def _problem(seed, *, T=6, d=8, E=4, k=2, dff=8, dffs=0, act=oracle.GELU):
    rng = np.random.default_rng(seed)
    n_up = 2 if act == oracle.SWIGLU else 1
    p = dict(
        x=_grid(rng, (T, d), 64, 96),
        wr=_grid(rng, (E, d), 4096, 2048),
        w1=_grid(rng, (E, n_up * dff, d), 256, 64),
        w2=_grid(rng, (E, d, dff), 256, 64),
        ws1=_grid(rng, (n_up * dffs, d), 256, 64) if dffs else None,
        ws2=_grid(rng, (d, dffs), 256, 64) if dffs else None,
    )
    dy = _grid(rng, (T, d), 64, 64)
    return p, dy


def _fwd(p, *, k, routing, act, cf=0.0, C=0):
    return oracle.layer(p["x"], p["wr"], p["w1"], p["w2"], k=k, routing=routing, act=act, cf=cf,
                        ec_capacity=C, ws1=p["ws1"], ws2=p["ws2"])


def _route_key(r):
    if r.ec_token is not None:
        return ("ec", r.ec_token.tobytes())
    return ("topk", r.idx.tobytes(), r.dispatch.slot_row.tobytes())


def _loss(p, dy, **kw):
    r = _fwd(p, **kw)
    return float(np.sum(r.y * dy.astype(np.float64))), _route_key(r)


def _fd_grad(p, dy, name, **kw):
    base_key = _route_key(_fwd(p, **kw))
    a = p[name]
    g = np.empty(a.shape)
    for i in np.ndindex(a.shape):
        v = a[i]
        a[i] = np.float32(v + H)
        lp, kp = _loss(p, dy, **kw)
        a[i] = np.float32(v - H)
        lm, km = _loss(p, dy, **kw)
        a[i] = v
        assert kp == base_key and km == base_key, f"routing flipped while perturbing {name}{i}"
        g[i] = (lp - lm) / (2 * H)
    return g


CASES = [
    # id, problem kwargs, forward kwargs
    ("gelu_softmax_all", dict(act=oracle.GELU), dict(k=2, routing=oracle.SOFTMAX_ALL, act=oracle.GELU)),
    ("swiglu_softmax_topk", dict(act=oracle.SWIGLU),
     dict(k=2, routing=oracle.SOFTMAX_TOPK, act=oracle.SWIGLU)),
    ("gelu_capacity_drops", dict(T=8, act=oracle.GELU),
     dict(k=2, routing=oracle.SOFTMAX_ALL, act=oracle.GELU, cf=0.5)),
    ("swiglu_shared", dict(act=oracle.SWIGLU, dffs=8),
     dict(k=2, routing=oracle.SOFTMAX_ALL, act=oracle.SWIGLU)),
    ("gelu_expert_choice", dict(T=8, act=oracle.GELU, dffs=8),
     dict(k=1, routing=oracle.EXPERT_CHOICE, act=oracle.GELU, C=3)),
]


@pytest.mark.parametrize("cid,pk,fk", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_finite_differences(cid, pk, fk):
    """Catches any wrong term, sign, transposed operand, wrong activation
    derivative, a gradient through a dropped slot, or a wrong softmax Jacobian:
    every gradient is compared with central differences of the forward."""
    p, dy = _problem(11, **pk)
    fwd = _fwd(p, **fk)
    if fk["routing"] != oracle.EXPERT_CHOICE:
        if fk.get("cf"):
            assert (fwd.dispatch.slot_row < 0).any(), "the capacity case must drop something"
    g = oracle.layer_bwd(p["x"], p["wr"], p["w1"], p["w2"], dy, fwd, k=fk["k"], routing=fk["routing"],
                         act=fk["act"], ws1=p["ws1"], ws2=p["ws2"])
    analytic = dict(x=g.dx, wr=g.dwr, w1=g.dw1, w2=g.dw2, ws1=g.dws1, ws2=g.dws2)
    for name, ga in analytic.items():
        if p[name] is None:
            assert ga is None
            continue
        fd = _fd_grad(p, dy, name, **fk)
        scale = max(np.abs(fd).max(), 1e-3)
        np.testing.assert_allclose(ga, fd, rtol=0, atol=2e-7 * scale, err_msg=f"{cid}: d{name}")


def _torch_layer(p, dy, fwd, *, k, routing, act):
    """The same forward written with torch ops in fp64 (routing from the oracle's
    forward, held fixed); autograd supplies the gradients."""
    t = {n: (torch.tensor(v.astype(np.float64), requires_grad=True) if v is not None else None)
         for n, v in p.items()}
    x, wr = t["x"], t["wr"]
    lg = x @ wr.T
    T, d = x.shape

    def ffn(xr, w1, w2):
        z = xr @ w1.T
        if act == oracle.GELU:
            h = 0.5 * z * (1 + torch.erf(z / np.sqrt(2.0)))
        else:
            dff = w2.shape[-1]
            a, b = z[..., :dff], z[..., dff:]
            h = a * torch.sigmoid(a) * b
        return h @ w2.T

    y = torch.zeros(T, d, dtype=torch.float64)
    if routing == oracle.EXPERT_CHOICE:
        S = torch.softmax(lg, dim=1)
        for e in range(fwd.ec_token.shape[0]):
            for tok in fwd.ec_token[e]:
                y[tok] = y[tok] + S[tok, e] * ffn(x[tok], t["w1"][e], t["w2"][e])
    else:
        for tok in range(T):
            if routing == oracle.SOFTMAX_ALL:
                w = torch.softmax(lg[tok], 0)[torch.tensor(fwd.idx[tok], dtype=torch.long)]
            else:
                w = torch.softmax(lg[tok][torch.tensor(fwd.idx[tok], dtype=torch.long)], 0)
            for j in range(k):
                if fwd.dispatch.slot_row[tok, j] < 0:
                    continue
                e = int(fwd.idx[tok, j])
                y[tok] = y[tok] + w[j] * ffn(x[tok], t["w1"][e], t["w2"][e])
    if t["ws1"] is not None:
        y = y + ffn(x, t["ws1"], t["ws2"])
    (y * torch.tensor(dy.astype(np.float64))).sum().backward()
    return {n: (v.grad.numpy() if v is not None else None) for n, v in t.items()}


@pytest.mark.parametrize("cid,pk,fk", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_torch_autograd(cid, pk, fk):
    """A second, independent derivation of every gradient (torch autograd of the
    same forward in fp64); catches the same mistakes as the finite differences,
    to rounding precision instead of O(H^2)."""
    p, dy = _problem(23, **pk)
    fwd = _fwd(p, **fk)
    g = oracle.layer_bwd(p["x"], p["wr"], p["w1"], p["w2"], dy, fwd, k=fk["k"], routing=fk["routing"],
                         act=fk["act"], ws1=p["ws1"], ws2=p["ws2"])
    ref = _torch_layer(p, dy, fwd, k=fk["k"], routing=fk["routing"], act=fk["act"])
    ours = dict(x=g.dx, wr=g.dwr, w1=g.dw1, w2=g.dw2, ws1=g.dws1, ws2=g.dws2)
    for name, ga in ours.items():
        if ref[name] is None:
            continue
        np.testing.assert_allclose(ga, ref[name], rtol=1e-10, atol=1e-12, err_msg=f"{cid}: d{name}")


def test_gate_bwd_two_experts_closed_form():
    """E = 2, k = 1, SOFTMAX_ALL: w = p_chosen = sigmoid(l_c - l_o), so
    dL/dl_c = dw * p (1 - p) and dL/dl_o = -dL/dl_c.  Catches a wrong sign or a
    missing p(1-p) factor."""
    rng = np.random.default_rng(5)
    lg = rng.normal(size=(16, 2))
    idx = oracle.topk(lg, 1)
    dw = rng.normal(size=(16, 1))
    got = oracle.gate_bwd_topk(lg, idx, dw, oracle.SOFTMAX_ALL)
    for t in range(16):
        c = idx[t, 0]
        pc = 1.0 / (1.0 + np.exp(-(lg[t, c] - lg[t, 1 - c])))
        assert got[t, c] == pytest.approx(dw[t, 0] * pc * (1 - pc), rel=1e-12)
        assert got[t, 1 - c] == pytest.approx(-dw[t, 0] * pc * (1 - pc), rel=1e-12)


@pytest.mark.parametrize("mode", [oracle.SOFTMAX_ALL, oracle.SOFTMAX_TOPK])
def test_gate_bwd_rows_sum_to_zero(mode):
    """Adding a constant to every logit of a token changes no softmax, so each
    row of dL/dlogits sums to 0.  Catches a dropped "- sum p g" term."""
    rng = np.random.default_rng(6)
    lg = rng.normal(size=(32, 8))
    idx = oracle.topk(lg, 3)
    got = oracle.gate_bwd_topk(lg, idx, rng.normal(size=(32, 3)), mode)
    np.testing.assert_allclose(got.sum(axis=1), 0.0, atol=1e-14)


def test_gate_bwd_topk_single_expert_is_zero():
    """SOFTMAX_TOPK with k = 1 gives weight 1 whatever the logits: no gradient."""
    rng = np.random.default_rng(7)
    lg = rng.normal(size=(16, 8))
    got = oracle.gate_bwd_topk(lg, oracle.topk(lg, 1), rng.normal(size=(16, 1)), oracle.SOFTMAX_TOPK)
    assert np.all(got == 0.0)


def test_gate_bwd_topk_touches_only_chosen_logits():
    """SOFTMAX_TOPK weights depend only on the chosen logits."""
    rng = np.random.default_rng(8)
    lg = rng.normal(size=(16, 8))
    idx = oracle.topk(lg, 2)
    got = oracle.gate_bwd_topk(lg, idx, rng.normal(size=(16, 2)), oracle.SOFTMAX_TOPK)
    mask = np.zeros_like(got, bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.all(got[~mask] == 0.0)


def test_gelu_and_silu_derivatives_against_finite_differences():
    """The activation derivatives by themselves, over pre-activations from -6 to
    6: with W1 = I (SwiGLU: [I; I]) and W2 = I the FFN is elementwise, so
    dx = act'(z) is checked against central differences of the forward row.
    Catches, e.g., a tanh-approximate GELU derivative or a missing term of
    silu'."""
    d = dff = 8
    z = (np.arange(-96, 97, 24) / 16.0).astype(np.float32)[:d]  # -6 .. 4.5, exact +-H
    w2 = np.eye(d, dff, dtype=np.float32)
    for act, w1 in ((oracle.GELU, np.eye(dff, d, dtype=np.float32)),
                    (oracle.SWIGLU, np.concatenate([np.eye(dff, d), np.eye(dff, d)]).astype(np.float32))):
        _, _, dx, out = oracle.ffn_row_bwd(z, w1, w2, act, np.ones(d))
        np.testing.assert_allclose(out, oracle.ffn_row(z, w1, w2, act), rtol=1e-15, atol=0)
        fd = np.empty(d)
        for i in range(d):
            zp, zm = z.copy(), z.copy()
            zp[i] += np.float32(H)
            zm[i] -= np.float32(H)
            fd[i] = (oracle.ffn_row(zp, w1, w2, act)[i] - oracle.ffn_row(zm, w1, w2, act)[i]) / (2 * H)
        np.testing.assert_allclose(dx, fd, rtol=0, atol=1e-7)


@pytest.mark.parametrize("cid,pk,fk", CASES, ids=[c[0] for c in CASES])
def test_sampled_oracle_paths_agree_with_full_backward(cid, pk, fk):
    """The token-by-token and element-by-element functions used for large
    problems give what the full backward gives (same oracle, different loop
    order: catches an indexing slip in the sampled paths)."""
    p, dy = _problem(31, **pk)
    fwd = _fwd(p, **fk)
    kw = dict(k=fk["k"], routing=fk["routing"], act=fk["act"], ws1=p["ws1"], ws2=p["ws2"])
    g = oracle.layer_bwd(p["x"], p["wr"], p["w1"], p["w2"], dy, fwd, **kw)
    toks = np.array([0, 2, 5], np.int32)
    dx, dl, dw = oracle.layer_bwd_tokens(p["x"], p["wr"], p["w1"], p["w2"], dy, fwd, toks, **kw)
    np.testing.assert_allclose(dx, g.dx[toks], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dl, g.dlogits[toks], rtol=1e-12, atol=1e-14)
    E = p["wr"].shape[0]
    if fk["routing"] == oracle.EXPERT_CHOICE:
        want = np.zeros((len(toks), E))
        for e in range(E):
            for c, tok in enumerate(fwd.ec_token[e]):
                hit = np.nonzero(toks == tok)[0]
                if len(hit):
                    want[hit[0], e] = g.d_slot_w[e, c]
        np.testing.assert_allclose(dw, want, rtol=1e-12, atol=1e-14)
    else:
        np.testing.assert_allclose(dw, g.d_slot_w[toks], rtol=1e-12, atol=1e-14)
    # weight-gradient elements of expert 1 and of the shared expert
    e = 1
    if fk["routing"] == oracle.EXPERT_CHOICE:
        rt = fwd.ec_token[e]
        rw = oracle.softmax(fwd.logits)[rt, e]
    else:
        off = fwd.dispatch.expert_offset
        rt = fwd.dispatch.row_token[off[e]:off[e + 1]]
        rw = np.array([fwd.w[t][list(fwd.idx[t]).index(e)] for t in rt])
    rr = np.array([0, 3, p["w1"].shape[1] - 1], np.int32)
    cc = np.array([1, 7, 0], np.int32)
    got1 = oracle.ffn_dw_elems(p["x"], dy, p["w1"][e], p["w2"][e], rt, rw, fk["act"], 1, rr, cc)
    np.testing.assert_allclose(got1, g.dw1[e][rr, cc], rtol=1e-12, atol=1e-14)
    rr2 = np.array([0, 5, 7], np.int32)
    cc2 = np.array([2, 0, 7], np.int32)
    got2 = oracle.ffn_dw_elems(p["x"], dy, p["w1"][e], p["w2"][e], rt, rw, fk["act"], 2, rr2, cc2)
    np.testing.assert_allclose(got2, g.dw2[e][rr2, cc2], rtol=1e-12, atol=1e-14)
    if p["ws1"] is not None:
        T = p["x"].shape[0]
        allt = np.arange(T, dtype=np.int32)
        got = oracle.ffn_dw_elems(p["x"], dy, p["ws1"], p["ws2"], allt, np.ones(T), fk["act"], 1, rr, cc)
        np.testing.assert_allclose(got, g.dws1[rr, cc], rtol=1e-12, atol=1e-14)
