"""Randomised shapes (hypothesis, derandomised, no shrinking: the first failing
case ends the test): the whole layer through the C ABI on random T, E, k,
d_model, d_ff, capacity factor, activation, dtype, routing (both top-k softmax
placements and ExpertChoice with a random C) and shared-expert width,
compared with the oracle on every token -- routing and
permutation bit-exact given the GPU's fp32 logits, outputs within the
dtype's tolerance.  The sizes hit ragged tails of every tile the kernels use
(token tiles of the router and permute, 64/128/256-row GEMM tiles, 32/64-wide
K stages, column tiles) while the oracle still finishes in seconds."""
import numpy as np
import pytest
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

from _parity import check_output_ec, check_output_topk, check_routing_ec, check_routing_topk, run_layer, say
from mixture_experts_layer_topkrouter_amd import workloads as W


@st.composite
def shapes(draw):
    E = draw(st.integers(1, 48))
    k = draw(st.integers(1, min(E, 8)))
    T = draw(st.integers(1, 900))
    d = 8 * draw(st.integers(1, 64))
    d_ff = 8 * draw(st.integers(1, 96))
    dtype = draw(st.sampled_from([W.F32, W.BF16]))
    act = draw(st.sampled_from([W.GELU, W.SWIGLU]))
    routing = draw(st.sampled_from([W.SOFTMAX_ALL, W.SOFTMAX_TOPK, W.EXPERT_CHOICE]))
    cf = draw(st.sampled_from([0.0, 0.5, 1.0, 1.25, 2.0]))
    shared = draw(st.sampled_from([0, 0, 8 * draw(st.integers(1, 40))]))
    # ExpertChoice: every expert takes C of the T tokens (1 <= C <= T)
    C = draw(st.integers(1, T)) if routing == W.EXPERT_CHOICE else 0
    return W.Workload("sweep", T=T, d=d, E=E, k=k, d_ff=d_ff, act=act, dtype=dtype,
                      routing=routing, cf=0.0 if C else cf, ec_capacity=C, d_ff_shared=shared,
                      wr_std=1.0 / np.sqrt(d))


@pytest.mark.gpu
@settings(max_examples=40, deadline=None, derandomize=True, phases=[Phase.explicit, Phase.generate],
          report_multiple_bugs=False, suppress_health_check=list(HealthCheck))
@given(w=shapes())
def test_random_shapes_match_oracle(w):
    say(f"[sweep] T={w.T} d={w.d} E={w.E} k={w.k} d_ff={w.d_ff} shared={w.d_ff_shared} act={w.act} "
        f"dtype={w.dtype} routing={w.routing} cf={w.cf}")
    layer, inp = run_layer(w)
    toks = np.arange(w.T, dtype=np.int32)
    if w.routing == W.EXPERT_CHOICE:
        lg, sc, _ = check_routing_ec(w, layer, inp)
        check_output_ec(w, layer, inp, lg, sc, toks)
    else:
        lg, _, _ = check_routing_topk(w, layer, inp)
        check_output_topk(w, layer, inp, lg, toks)


@st.composite
def packable_shapes(draw):
    """bf16 shapes the packed path takes: d_model, d_ff, d_ff_shared multiples of 64."""
    E = draw(st.integers(1, 40))
    k = draw(st.integers(1, min(E, 8)))
    T = draw(st.integers(1, 1200))
    d = 64 * draw(st.integers(1, 10))
    d_ff = 64 * draw(st.integers(1, 14))
    act = draw(st.sampled_from([W.GELU, W.SWIGLU]))
    routing = draw(st.sampled_from([W.SOFTMAX_ALL, W.SOFTMAX_TOPK, W.EXPERT_CHOICE]))
    cf = draw(st.sampled_from([0.0, 0.5, 1.0, 1.25]))
    shared = draw(st.sampled_from([0, 64 * draw(st.integers(1, 6))]))
    C = draw(st.integers(1, T)) if routing == W.EXPERT_CHOICE else 0
    return W.Workload("sweep_packed", T=T, d=d, E=E, k=k, d_ff=d_ff, act=act, dtype=W.BF16,
                      routing=routing, cf=0.0 if C else cf, ec_capacity=C, d_ff_shared=shared,
                      wr_std=1.0 / np.sqrt(d))


@pytest.mark.gpu
@settings(max_examples=30, deadline=None, derandomize=True, phases=[Phase.explicit, Phase.generate],
          report_multiple_bugs=False, suppress_health_check=list(HealthCheck))
@given(w=packable_shapes())
def test_random_shapes_packed_path(w):
    """moe_layer_fwd_packed on random packable shapes: routing, K-blocked
    permutation and every token's output against the oracle, and the bits of
    moe_layer_fwd wherever both orders run the same GEMM kernel (at most 128
    or at least 192 rows per expert on average)."""
    import torch
    from mixture_experts_layer_topkrouter_amd import moe
    say(f"[sweep packed] T={w.T} d={w.d} E={w.E} k={w.k} d_ff={w.d_ff} shared={w.d_ff_shared} act={w.act} "
        f"routing={w.routing} cf={w.cf} C={w.ec_capacity}")
    layer, inp = run_layer(w)
    y_plain = layer.y.clone()
    layer.pack()
    layer.y.fill_(7.0)
    layer.forward(packed=True)
    torch.cuda.synchronize()
    avg = moe.max_rows(layer.cfg) // w.E
    if not 128 < avg < 192:
        assert torch.equal(layer.y.view(torch.int16), y_plain.view(torch.int16)), "packed layer differs"
    toks = np.arange(w.T, dtype=np.int32)
    if w.routing == W.EXPERT_CHOICE:
        lg, sc, _ = check_routing_ec(w, layer, inp, kblocked=True)
        check_output_ec(w, layer, inp, lg, sc, toks)
    else:
        lg, _, _ = check_routing_topk(w, layer, inp, kblocked=True)
        check_output_topk(w, layer, inp, lg, toks)
