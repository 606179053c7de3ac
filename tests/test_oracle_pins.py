"""Pins for the fp64 CPU oracle, against things other than the oracle itself:
hand-worked examples (tests/golden), closed forms, textbook tables, independent
library routines (numpy/scipy), invariants and brute force on tiny inputs.

Each test names the mistake it is there to catch."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- top-k ----

def test_topk_golden_ties_and_signed_zero():
    """Hand-worked cases: tie -> lower index, -0 == +0, slot order descending."""
    for case in _golden("topk_ties.json")["cases"]:
        lg = np.array([case["logits"]], np.float64)
        got = oracle.topk(lg, case["k"])[0].tolist()
        assert got == case["idx"], case["why"]


def _brute_topk(row, k):
    """Brute force over every ordered choice of k experts: the answer is the one
    where every chosen expert beats every unchosen one and the chosen ones are in
    beating order (beat = larger value, or equal value and lower index)."""
    E = len(row)

    def beats(a, b):
        return row[a] > row[b] or (row[a] == row[b] and a < b)

    found = []
    for perm in itertools.permutations(range(E), k):
        rest = [e for e in range(E) if e not in perm]
        if all(beats(perm[i], perm[i + 1]) for i in range(k - 1)) and all(
                beats(p, r) for p in perm for r in rest):
            found.append(list(perm))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_tiny(seed):
    """Catches a wrong comparison direction, a wrong tie rule or a slot-order bug."""
    rng = np.random.default_rng(100 + seed)
    T, E = 8, 6
    # few distinct values so ties are common; include signed zeros
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 2.0], np.float64)
    lg = vals[rng.integers(0, len(vals), size=(T, E))]
    for k in (1, 2, 3, E):
        idx = oracle.topk(lg, k)
        for t in range(T):
            assert idx[t].tolist() == _brute_topk(lg[t].tolist(), k)


def test_topk_matches_stable_argsort():
    """An independent routine: numpy's stable argsort of -logits keeps equal
    keys in index order (and -(-0.0) == -(+0.0) under its comparisons)."""
    rng = np.random.default_rng(7)
    lg = np.round(rng.standard_normal((300, 16)), 1)  # rounding makes ties
    for k in (1, 2, 6):
        ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
        assert np.array_equal(oracle.topk(lg, k), ref)


# -------------------------------------------------------------- softmax ----

def test_softmax_two_experts_closed_form():
    """E = 2: p0 = sigmoid(l0 - l1).  Catches a missing max-shift sign error or
    a normalisation over the wrong axis."""
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((50, 2)) * 3
    p = oracle.softmax(lg)
    np.testing.assert_allclose(p[:, 0], special.expit(lg[:, 0] - lg[:, 1]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-14)


def test_gate_weights_modes_against_library_softmax():
    """SOFTMAX_ALL: weights are scipy's softmax over all E at the chosen
    indices (not renormalised).  SOFTMAX_TOPK: scipy's softmax over the chosen
    logits; sums to 1."""
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((40, 8)) * 2
    idx = oracle.topk(lg, 2)
    p = special.softmax(lg, axis=1)
    w_all = oracle.gate_weights(lg, idx, oracle.SOFTMAX_ALL)
    np.testing.assert_allclose(w_all, np.take_along_axis(p, idx, 1), rtol=1e-13)
    assert np.all(w_all.sum(1) < 1.0)
    w_top = oracle.gate_weights(lg, idx, oracle.SOFTMAX_TOPK)
    np.testing.assert_allclose(w_top, special.softmax(np.take_along_axis(lg, idx, 1), axis=1), rtol=1e-13)
    np.testing.assert_allclose(w_top.sum(1), 1.0, rtol=1e-14)
    # top-2 with softmax over the pair is the logistic of the logit gap
    np.testing.assert_allclose(w_top[:, 0], special.expit(lg[np.arange(40), idx[:, 0]] - lg[np.arange(40), idx[:, 1]]),
                               rtol=1e-13)


def test_softmax_large_logits_do_not_overflow():
    lg = np.array([[1000.0, 999.0, -1000.0]])
    p = oracle.softmax(lg)
    assert np.all(np.isfinite(p))
    np.testing.assert_allclose(p[0, 0], special.expit(1.0), rtol=1e-14)


# ------------------------------------------------------------- capacity ----

def test_capacity_values_from_the_key_parameters_page():
    for c in _golden("capacity_values.json")["cases"]:
        assert oracle.capacity(c["cf"], c["T"], c["k"], c["E"]) == c["C"], c["why"]


# ------------------------------------------------------------- dispatch ----

def test_dispatch_golden_hand_worked():
    g = _golden("capacity_dispatch.json")
    cap = oracle.capacity(g["cf"], g["T"], g["k"], g["E"])
    assert cap == g["capacity"]
    d = oracle.dispatch_topk(np.array(g["idx"]), g["E"], cap)
    assert d.expert_load.tolist() == g["expert_load"]
    assert d.expert_count.tolist() == g["expert_count"]
    assert d.expert_offset.tolist() == g["expert_offset"]
    assert d.slot_row.tolist() == g["slot_row"]
    assert d.row_token.tolist() == g["row_token"]


def _independent_dispatch(idx, E, cap):
    """The same rule written another way: expert e keeps the first C entries of
    the list of positions (in token-major order) that chose it."""
    flat = idx.ravel()
    k = idx.shape[1]
    slot_row = np.full(flat.shape, -1, np.int64)
    row_token = []
    counts = []
    for e in range(E):
        pos = np.flatnonzero(flat == e)
        keep = pos if cap < 0 else pos[:cap]
        base = len(row_token)
        slot_row[keep] = base + np.arange(len(keep))
        row_token.extend((keep // k).tolist())
        counts.append(len(keep))
    return slot_row.reshape(idx.shape), np.array(row_token), np.array(counts)


@pytest.mark.parametrize("cf", [0.0, 0.5, 1.0, 1.25])
def test_dispatch_against_independent_rule_and_invariants(cf):
    rng = np.random.default_rng(3)
    T, E, k = 97, 7, 3
    # skewed routing so the capacity bites
    lg = rng.standard_normal((T, E)) + np.linspace(2, -2, E)
    idx = oracle.topk(lg, k)
    cap = oracle.capacity(cf, T, k, E)
    d = oracle.dispatch_topk(idx, E, cap)
    sr, rt, cnt = _independent_dispatch(idx, E, cap)
    assert np.array_equal(d.slot_row, sr)
    assert np.array_equal(d.row_token, rt)
    assert np.array_equal(d.expert_count, cnt)
    dropped = int((d.slot_row < 0).sum())
    # sum of counts = T*k - dropped; counts bounded by C; loads are the raw histogram
    assert d.expert_count.sum() == T * k - dropped
    assert np.array_equal(d.expert_load, np.bincount(idx.ravel(), minlength=E))
    if cap >= 0:
        assert d.expert_count.max() <= cap
    else:
        assert dropped == 0  # dropless: no -1
    # kept slots <-> rows [0, N) is a bijection; each expert segment ascends
    kept = d.slot_row[d.slot_row >= 0]
    assert np.array_equal(np.sort(kept), np.arange(d.n_rows))
    for e in range(E):
        seg = d.row_token[d.expert_offset[e]:d.expert_offset[e + 1]]
        assert np.all(np.diff(seg) > 0) or len(seg) <= 1


def test_permute_then_unpermute_is_identity_on_kept_tokens():
    """Gather x by row_token, scatter back through slot_row (k = 1, unit
    weight): kept tokens come back bit-exact, dropped ones are absent."""
    rng = np.random.default_rng(4)
    T, E, d = 64, 5, 9
    x = rng.standard_normal((T, d))
    idx = oracle.topk(rng.standard_normal((T, E)) + np.array([3, 0, 0, 0, 0.0]), 1)
    d_ = oracle.dispatch_topk(idx, E, oracle.capacity(1.0, T, 1, E))
    x_perm = x[d_.row_token]
    back = np.zeros_like(x)
    for t in range(T):
        r = d_.slot_row[t, 0]
        if r >= 0:
            back[t] = 1.0 * x_perm[r]
    kept = d_.slot_row[:, 0] >= 0
    assert np.array_equal(back[kept], x[kept])
    assert (~kept).sum() > 0


# ------------------------------------------------------------ FFN pins ----

def _scalar_ffn(z, act, u=None, w2=1.0):
    """One-dimensional FFN through the oracle: d = 1, d_ff = 1, x = [1]."""
    x = np.array([1.0], np.float32)
    w1 = np.array([[z]] if act == oracle.GELU else [[z], [u]], np.float32)
    return oracle.ffn_row(x, w1, np.array([[w2]], np.float32), act)[0]


def test_gelu_against_normal_table():
    """GELU(z)/z = Phi(z).  A tanh approximation misses the table at z = 1."""
    g = _golden("normal_cdf.json")
    tol = 0.5 * 10 ** -g["decimals"] + 1e-12
    for z, phi in g["values"]:
        zz = float(np.float32(z))
        assert abs(_scalar_ffn(zz, oracle.GELU) / zz - phi) <= tol, (z, phi)
    # and against scipy's normal CDF (Cephes ndtr, not the C library's erf)
    for z in np.linspace(-4, 4, 33, dtype=np.float32):
        if z == 0:
            assert _scalar_ffn(0.0, oracle.GELU) == 0.0
            continue
        assert abs(_scalar_ffn(float(z), oracle.GELU) - float(z) * special.ndtr(float(z))) < 1e-14


def test_swiglu_closed_form_and_gate_up_order():
    """silu(ln 3) = (3/4) ln 3 since sigmoid(ln 3) = 3/4.  W1 rows: gate first,
    then up; swapping them gives silu(u)*g, which the value below rejects."""
    z = float(np.float32(math.log(3.0)))
    sig = 1.0 / (1.0 + 1.0 / 3.0 * math.exp(math.log(3.0) - z))  # exact sigmoid(z) around ln 3
    got = _scalar_ffn(z, oracle.SWIGLU, u=2.0, w2=1.0)
    assert abs(got - 2.0 * z * sig) < 1e-12
    assert abs(got - 2.0 * 0.75 * math.log(3.0)) < 1e-6
    # odd-part identity silu(z) - silu(-z) = z
    for zz in (0.3, 1.7, 4.0):
        zz = float(np.float32(zz))
        a = _scalar_ffn(zz, oracle.SWIGLU, u=1.0)
        b = _scalar_ffn(-zz, oracle.SWIGLU, u=1.0)
        assert abs((a - b) - zz) < 1e-14


def _np_mlp(x, w1, w2, act):
    """Dense MLP with numpy fp64 matmul (BLAS) and scipy's erf / expit."""
    h = x @ w1.T
    if act == oracle.GELU:
        a = 0.5 * h * (1.0 + special.erf(h / np.sqrt(2.0)))
    else:
        dff = w1.shape[0] // 2
        g, u = h[:, :dff], h[:, dff:]
        a = g * special.expit(g) * u
    return a @ w2.T


@pytest.mark.parametrize("act", [oracle.GELU, oracle.SWIGLU])
def test_one_expert_top1_is_a_dense_mlp(act):
    """E = 1, k = 1: the layer reduces to one dense MLP (weight 1)."""
    rng = np.random.default_rng(5)
    T, d, dff = 12, 16, 24
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((1, d)).astype(np.float32)
    nup = 2 if act == oracle.SWIGLU else 1
    w1 = (rng.standard_normal((1, nup * dff, d)) * 0.3).astype(np.float32)
    w2 = (rng.standard_normal((1, d, dff)) * 0.3).astype(np.float32)
    for mode in (oracle.SOFTMAX_ALL, oracle.SOFTMAX_TOPK):
        r = oracle.layer(x, wr, w1, w2, k=1, routing=mode, act=act)
        assert np.all(r.w == 1.0)
        ref = _np_mlp(x.astype(np.float64), w1[0].astype(np.float64), w2[0].astype(np.float64), act)
        np.testing.assert_allclose(r.y, ref, rtol=1e-12, atol=1e-12)


def test_two_experts_softmax_topk_mix():
    """E = 2, k = 2, SOFTMAX_TOPK: y = s*MLP_a + (1-s)*MLP_b with s the logistic
    of the logit gap; catches swapped weights or experts."""
    rng = np.random.default_rng(6)
    T, d, dff = 10, 8, 12
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((2, d)).astype(np.float32)
    w1 = (rng.standard_normal((2, 2 * dff, d)) * 0.3).astype(np.float32)
    w2 = (rng.standard_normal((2, d, dff)) * 0.3).astype(np.float32)
    r = oracle.layer(x, wr, w1, w2, k=2, routing=oracle.SOFTMAX_TOPK, act=oracle.SWIGLU)
    x64 = x.astype(np.float64)
    lg = x64 @ wr.astype(np.float64).T
    s = special.expit(lg[:, 0] - lg[:, 1])
    m0 = _np_mlp(x64, w1[0].astype(np.float64), w2[0].astype(np.float64), oracle.SWIGLU)
    m1 = _np_mlp(x64, w1[1].astype(np.float64), w2[1].astype(np.float64), oracle.SWIGLU)
    np.testing.assert_allclose(r.y, s[:, None] * m0 + (1 - s)[:, None] * m1, rtol=1e-11, atol=1e-12)


def test_logits_against_blas_with_both_bias_layouts():
    rng = np.random.default_rng(8)
    T, d, E = 20, 33, 5
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T
    np.testing.assert_allclose(oracle.logits(x, wr), ref, rtol=1e-13, atol=1e-13)
    be = rng.standard_normal(E).astype(np.float32)
    np.testing.assert_allclose(oracle.logits(x, wr, be, 0), ref + be, rtol=1e-13, atol=1e-13)
    bt = rng.standard_normal((T, E)).astype(np.float32)
    np.testing.assert_allclose(oracle.logits(x, wr, bt, E), ref + bt, rtol=1e-13, atol=1e-13)


def test_bf16_inputs_are_widened_exactly():
    """bf16 bit patterns: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3EAB ~ 0.333984375."""
    x = np.array([[0x3F80, 0xC000, 0x3EAB]], np.uint16)
    wr = np.array([[0x3F80, 0x3F80, 0x3F80]], np.uint16)
    assert oracle.logits(x, wr)[0, 0] == 1.0 - 2.0 + 0.333984375


def test_scaling_w2_doubles_output_and_dropped_tokens_are_zero():
    """Linearity in W2 (exact in fp64 for a factor 2); tokens whose every slot
    is dropped give exactly 0 without a shared expert."""
    rng = np.random.default_rng(9)
    T, d, dff, E, k = 40, 8, 16, 4, 1
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = np.zeros((E, d), np.float32)
    bias = np.array([4.0, 0.0, 0.0, 0.0], np.float32)  # everyone picks expert 0
    w1 = (rng.standard_normal((E, dff, d)) * 0.3).astype(np.float32)
    w2 = (rng.standard_normal((E, d, dff)) * 0.3).astype(np.float32)
    r1 = oracle.layer(x, wr, w1, w2, k=k, routing=oracle.SOFTMAX_ALL, act=oracle.GELU, cf=1.0, bias=bias)
    r2 = oracle.layer(x, wr, w1, 2 * w2, k=k, routing=oracle.SOFTMAX_ALL, act=oracle.GELU, cf=1.0, bias=bias)
    assert np.array_equal(r2.y, 2 * r1.y)
    cap = oracle.capacity(1.0, T, k, E)
    assert cap == 10
    dropped = r1.dispatch.slot_row[:, 0] < 0
    assert dropped.sum() == T - cap
    assert np.all(r1.y[dropped] == 0.0)
    assert np.all(np.abs(r1.y[~dropped]).sum(1) > 0)


def test_shared_expert_alone_is_a_dense_mlp():
    """Routed W2 = 0: the output is the shared expert's dense MLP, weight 1."""
    rng = np.random.default_rng(10)
    T, d, dff, dffs, E = 9, 8, 12, 20, 3
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    w1 = rng.standard_normal((E, 2 * dff, d)).astype(np.float32)
    w2 = np.zeros((E, d, dff), np.float32)
    ws1 = (rng.standard_normal((2 * dffs, d)) * 0.3).astype(np.float32)
    ws2 = (rng.standard_normal((d, dffs)) * 0.3).astype(np.float32)
    r = oracle.layer(x, wr, w1, w2, k=2, routing=oracle.SOFTMAX_ALL, act=oracle.SWIGLU, ws1=ws1, ws2=ws2)
    ref = _np_mlp(x.astype(np.float64), ws1.astype(np.float64), ws2.astype(np.float64), oracle.SWIGLU)
    np.testing.assert_allclose(r.y, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- expert choice ----

def test_expert_choice_golden():
    g = _golden("expert_choice.json")
    got = oracle.ec_select(np.array(g["scores"]), g["C"])
    assert got.tolist() == g["ec_token"], g["why"]


def test_expert_choice_brute_force_properties():
    """Every expert takes exactly C distinct tokens, ascending; every chosen
    score beats every unchosen one in its column (ties -> lower token)."""
    rng = np.random.default_rng(11)
    T, E, C = 37, 5, 9
    sc = np.round(rng.random((T, E)), 1)  # many ties
    ec = oracle.ec_select(sc, C)
    for e in range(E):
        ch = ec[e]
        assert len(set(ch.tolist())) == C and np.all(np.diff(ch) > 0)
        un = [t for t in range(T) if t not in set(ch.tolist())]
        for a in ch:
            for b in un:
                assert sc[a, e] > sc[b, e] or (sc[a, e] == sc[b, e] and a < b)
        # independent routine: stable argsort of -score
        ref = np.sort(np.argsort(-sc[:, e], kind="stable")[:C])
        assert np.array_equal(ch, ref)


def test_expert_choice_layer_uncovered_token_is_zero():
    rng = np.random.default_rng(12)
    T, d, dff, E, C = 16, 8, 8, 2, 3
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    w1 = (rng.standard_normal((E, 2 * dff, d)) * 0.3).astype(np.float32)
    w2 = (rng.standard_normal((E, d, dff)) * 0.3).astype(np.float32)
    r = oracle.layer(x, wr, w1, w2, k=0, routing=oracle.EXPERT_CHOICE, act=oracle.SWIGLU, ec_capacity=C)
    covered = np.zeros(T, bool)
    covered[r.ec_token.ravel()] = True
    assert covered.sum() <= E * C < T
    assert np.all(r.y[~covered] == 0.0)
    # a token picked by exactly one expert: y = S[t,e] * MLP_e(x_t)
    x64 = x.astype(np.float64)
    p = special.softmax(x64 @ wr.astype(np.float64).T, axis=1)
    for e in range(E):
        for t in r.ec_token[e]:
            if (r.ec_token == t).sum() == 1:
                ref = p[t, e] * _np_mlp(x64[t:t + 1], w1[e].astype(np.float64), w2[e].astype(np.float64),
                                        oracle.SWIGLU)[0]
                np.testing.assert_allclose(r.y[t], ref, rtol=1e-11, atol=1e-13)
