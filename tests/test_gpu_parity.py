"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Routing indices, permutation order, counts, offsets and drop masks must match
bit for bit (the oracle routes on the GPU's fp32 logits / scores); outputs must
be within max relative error 1e-4 (fp32) or 2e-2 (bf16) of the fp64 oracle.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from _parity import (TOL_Y, check_output_ec, check_output_topk, check_routing_ec, check_routing_topk, host_float,
                     inputs, max_rel_err, run_layer, sample_tokens, say, tile_cover_tokens)
from mixture_experts_layer_topkrouter_amd import moe
from mixture_experts_layer_topkrouter_amd import workloads as W

WL = W.WORKLOADS
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# Reduced sizes the oracle finishes in seconds; several tiles per expert and
# ragged tails (T, E, d_ff not multiples of the tiles; d_ff % 64 != 0).
SMALL = {
    "tiny_top2_fp32": WL["tiny_top2_fp32"],
    "tiny_swiglu_fp32_ragged": W.small_variant(WL["tiny_top2_fp32"], T=203, E=5, k=3, d_ff=200, act=W.SWIGLU,
                                               cf=1.1),
    "mixtral_small": W.small_variant(WL["mixtral_top2_bf16"], T=1600, d=384, d_ff=520),
    "finegrained_small": W.small_variant(WL["finegrained_shared_bf16"], T=700, d=256, E=12, d_ff=136,
                                         d_ff_shared=264, wr_std=1.0 / 16.0),
    # >= 192 rows per expert and a reduction length of 8192: the bf16
    # 256 x 256 GEMM cuts its last round of tiles along K (8 pieces each) and
    # a second pass adds them: down projection (plain epilogue), up
    # projection with SwiGLU (gate and up pieces paired), up projection with
    # GELU
    "ksplit_down_small": W.small_variant(WL["mixtral_top2_bf16"], T=400, d=256, E=2, d_ff=8192),
    "ksplit_up_swiglu_small": W.small_variant(WL["mixtral_top2_bf16"], T=400, d=8192, E=2, d_ff=256),
    "ksplit_up_gelu_small": W.small_variant(WL["switch_top1_bf16"], T=800, d=8192, E=2, d_ff=264, cf=0.0),
    # few rows per expert (the weight-streaming kernel, 64-row tiles): GELU;
    # decode-sized SwiGLU batches whose K is cut into pieces (2-4 and up to 8
    # per tile) that a second pass adds
    "skinny_gelu_small": W.small_variant(WL["switch_top1_bf16"], T=1200, d=256, E=16, d_ff=512, cf=0.0),
    "skinny_decode_small": W.small_variant(WL["mixtral_top2_bf16"], T=64, d=512, E=8, d_ff=1024),
    "skinny_decode_longk_small": W.small_variant(WL["mixtral_top2_bf16"], T=32, d=256, E=4, d_ff=4096),
    "switch_small": W.small_variant(WL["switch_top1_bf16"], T=2000, d=192, E=16, d_ff=328),
    "correlated_small": W.small_variant(WL["correlated_top2_bf16"], T=1500, d=256, E=16, d_ff=200),
    "correlated_ec_small": W.small_variant(WL["correlated_ec_bf16"], T=1500, d=256, E=16, d_ff=200,
                                           ec_capacity=187),
    # fp32 with 200 experts (the router's widest tile: 16 logits per thread,
    # the router rows staged 64 columns at a time) and d_model 136 (a partial
    # last column chunk), capacity drops
    "fp32_many_experts_small": W.small_variant(WL["tiny_top2_fp32"], T=300, d=136, E=200, k=4, d_ff=72),
    # d_model not a multiple of the router's 64-wide K stages (its last stage
    # holds 8 columns), 24 experts padded to 32, 6 slots, 333 tokens (a
    # partial token tile)
    "route_ktail_small": W.small_variant(WL["finegrained_shared_bf16"], T=333, d=200, E=24, d_ff=136,
                                         d_ff_shared=0, wr_std=1.0 / np.sqrt(200.0)),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity_small(name):
    w = SMALL[name]
    say(f"[parity small] {name}: T={w.T} d={w.d} E={w.E} k={w.k} d_ff={w.d_ff}")
    layer, inp = run_layer(w)
    toks = np.arange(w.T, dtype=np.int32)
    if w.routing == W.EXPERT_CHOICE:
        lg, sc, _ = check_routing_ec(w, layer, inp)
        check_output_ec(w, layer, inp, lg, sc, toks)
    else:
        lg, _, d = check_routing_topk(w, layer, inp)
        if w.cf > 0:
            say(f"  dropped {int((d.slot_row < 0).sum())} of {w.T * w.k} assignments")
        check_output_topk(w, layer, inp, lg, toks)


FULL = ["tiny_top2_fp32", "mixtral_top2_bf16", "mixtral_decode_bf16", "finegrained_shared_bf16",
        "switch_top1_bf16", "correlated_top2_bf16", "correlated_ec_bf16"]


@pytest.mark.gpu
@pytest.mark.parametrize("name", FULL)
def test_layer_parity_full_size(name):
    """The workloads at full size, in the launch configuration the benchmark
    times: routing and permutation bit-exact over every token; outputs on a
    sample of tokens the oracle computes one by one."""
    w = WL[name]
    say(f"[parity full] {name}: T={w.T} d={w.d} E={w.E} d_ff={w.d_ff}")
    layer, inp = run_layer(w)
    # sampled tokens: random ones, plus the tokens of the first and last row
    # of every (expert, row tile), so every tile of both GEMMs is checked
    cover = tile_cover_tokens(w, layer)
    if w.routing == W.EXPERT_CHOICE:
        lg, sc, ec = check_routing_ec(w, layer, inp)
        uncovered = np.setdiff1d(np.arange(w.T), ec.ravel())[:2]
        toks = sample_tokens(w, 12, extra=list(uncovered) + list(cover))
        check_output_ec(w, layer, inp, lg, sc, toks)
        if len(uncovered):
            y = host_float(layer.y)[uncovered]
            assert np.all(y == 0.0)
    else:
        lg, _, d = check_routing_topk(w, layer, inp)
        dropped = np.flatnonzero((d.slot_row < 0).any(1))[:3]
        hot = int(np.argmax(d.expert_count))
        on_hot = d.row_token[d.expert_offset[hot]:d.expert_offset[hot] + 2]
        toks = sample_tokens(w, 12, extra=list(dropped) + list(on_hot) + list(cover))
        check_output_topk(w, layer, inp, lg, toks)


@pytest.mark.gpu
def test_entry_points_step_by_step_match_layer_fwd():
    """moe_route, moe_permute, moe_expert_ffn (routed and shared) and
    moe_unpermute called one by one give the same bits as moe_layer_fwd."""
    w = SMALL["finegrained_small"]
    layer, inp = run_layer(w)
    cfg = moe.make_config(w)
    dev = layer.dev
    dev_ = "cuda"
    T, E, k, d = w.T, w.E, w.k, w.d
    rows = moe.max_rows(cfg)
    dt = moe.torch_dtype(cfg)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev_)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev_)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev_)
    moe.route(cfg, dev.x, dev.wr, logits, idx, tw, bias=dev.bias, bias_stride=dev.bias_stride)
    x_perm = torch.empty((rows, d), dtype=dt, device=dev_)
    row_token = torch.empty(rows, dtype=torch.int32, device=dev_)
    slot_row = torch.empty((T, k), dtype=torch.int32, device=dev_)
    cnt = torch.empty(E, dtype=torch.int32, device=dev_)
    load = torch.empty(E, dtype=torch.int32, device=dev_)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev_)
    scratch = torch.empty(moe.permute_scratch_bytes(cfg), dtype=torch.uint8, device=dev_)
    moe.permute(cfg, dev.x, x_perm, row_token, slot_row, cnt, load, off, topk_idx=idx, scratch=scratch)
    h = torch.empty((rows, w.d_ff), dtype=dt, device=dev_)
    y_perm = torch.empty((rows, d), dtype=dt, device=dev_)
    moe.expert_ffn(cfg, x_perm, off, dev.w1, dev.w2, h, y_perm, moe.alloc_ffn_workspace(cfg))
    scfg = moe.MoeConfig(T, d, 1, 1, w.d_ff_shared, 0, 0.0, 0, w.dtype, w.act, W.SOFTMAX_ALL)
    soff = torch.tensor([0, T], dtype=torch.int32, device=dev_)
    hs = torch.empty((T, w.d_ff_shared), dtype=dt, device=dev_)
    ys = torch.empty((T, d), dtype=dt, device=dev_)
    moe.expert_ffn(scfg, dev.x, soff, dev.ws1, dev.ws2, hs, ys, moe.alloc_ffn_workspace(scfg))
    y = torch.empty((T, d), dtype=dt, device=dev_)
    moe.unpermute(cfg, y_perm, slot_row, tw, y, y_shared=ys)
    torch.cuda.synchronize()
    assert torch.equal(logits, layer.view("logits"))
    assert torch.equal(idx, layer.view("topk_idx"))
    assert torch.equal(slot_row, layer.view("slot_row"))
    assert torch.equal(ys, layer.view("shared_y"))
    assert torch.equal(y.view(torch.int16), layer.y.view(torch.int16))


@pytest.mark.gpu
def test_gate_on_given_logits_golden_ties():
    """x = NULL: the gate runs on given fp32 logits.  Hand-worked tie cases
    (lower index wins, -0 == +0)."""
    with open(os.path.join(GOLDEN, "topk_ties.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        E, k = len(c["logits"]), c["k"]
        cfg = moe.MoeConfig(1, 8, E, k, 8, 0, 0.0, 0, W.F32, W.GELU, W.SOFTMAX_ALL)
        lg = torch.tensor([c["logits"]], dtype=torch.float32, device="cuda")
        idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
        tw = torch.empty((1, k), dtype=torch.float32, device="cuda")
        moe.route(cfg, None, None, lg, idx, tw)
        torch.cuda.synchronize()
        assert idx.cpu().numpy()[0].tolist() == c["idx"], c["why"]


@pytest.mark.gpu
@pytest.mark.parametrize("E,k,mode", [(8, 2, W.SOFTMAX_ALL), (64, 6, W.SOFTMAX_ALL), (128, 1, W.SOFTMAX_ALL),
                                      (200, 16, W.SOFTMAX_TOPK), (256, 3, W.SOFTMAX_TOPK), (1, 1, W.SOFTMAX_TOPK),
                                      (7, 7, W.SOFTMAX_ALL)])
def test_gate_tie_heavy_logits_match_oracle(E, k, mode):
    """Logits from a handful of values (many exact ties, signed zeros):
    indices bit-exact, weights within fp32 rounding."""
    rng = np.random.default_rng(E * 31 + k)
    T = 777
    vals = np.array([-2.0, -0.0, 0.0, 0.5, 1.0, 3.0], np.float32)
    lg = vals[rng.integers(0, len(vals), size=(T, E))]
    cfg = moe.MoeConfig(T, 8, E, k, 8, 0, 0.0, 0, W.F32, W.GELU, mode)
    d_lg = torch.from_numpy(lg).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.route(cfg, None, None, d_lg, idx, tw)
    torch.cuda.synchronize()
    ref = oracle.topk(lg.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), ref)
    np.testing.assert_allclose(tw.cpu().numpy(), oracle.gate_weights(lg.astype(np.float64), ref, mode),
                               rtol=2e-6, atol=1e-7)


@pytest.mark.gpu
@pytest.mark.parametrize("T,E,C,vals", [
    (777, 8, 100, (-2.0, -0.0, 0.0, 0.5, 1.0, 3.0)),   # many exact score ties across tokens
    (2048, 64, 32, (0.0,)),                             # every score equal: the lowest C tokens
    (4000, 16, 4000, (-1.0, 0.0, 1.0)),                 # C = T: every token
    (16384, 128, 2, (0.0, 0.25, 0.5)),                  # the largest T, tiny C
    (300, 5, 299, (-3.0, 2.0)),                         # two score levels, C one short of T
    (16384, 2, 8000, (-5.0, 0.0)),                      # > 4096 keys share the first digit's threshold bin
    (4096, 48, 100, (0.0, 1e-3, 2e-3, 3e-3)),           # keys share their top 15 bits: digits start lower
])
def test_expert_choice_selection_ties_match_oracle(T, E, C, vals):
    """ExpertChoice selection on given fp32 logits with heavy ties: the
    softmax scores repeat exactly, so the C-th largest score is shared by many
    tokens and the lowest of them must be taken; selections bit-exact against
    the oracle run on the GPU's scores, weights equal the chosen scores."""
    rng = np.random.default_rng(T + E * 7 + C)
    lg = np.asarray(vals, np.float32)[rng.integers(0, len(vals), size=(T, E))]
    cfg = moe.MoeConfig(T, 8, E, 0, 8, 0, 0.0, C, W.F32, W.GELU, W.EXPERT_CHOICE)
    d_lg = torch.from_numpy(lg).cuda()
    sc = torch.empty((E, T), dtype=torch.float32, device="cuda")
    ect = torch.empty((E, C), dtype=torch.int32, device="cuda")
    ecw = torch.empty((E, C), dtype=torch.float32, device="cuda")
    moe.route(cfg, None, None, d_lg, scores=sc, ec_token=ect, ec_w=ecw)
    torch.cuda.synchronize()
    scores = sc.cpu().numpy().T
    np.testing.assert_allclose(scores, oracle.softmax(lg.astype(np.float64)), rtol=2e-6, atol=1e-9)
    ref = oracle.ec_select(scores.astype(np.float64), C)
    got = ect.cpu().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(ecw.cpu().numpy(), scores[ref, np.arange(E)[:, None]])


@pytest.mark.gpu
def test_all_tokens_on_one_expert_capacity_edge():
    """Every token prefers expert 0: exactly C are kept (the lowest tokens),
    the rest are dropped and give 0."""
    base = W.small_variant(WL["switch_top1_bf16"], T=1000, d=64, E=8, d_ff=64, cf=1.0)
    inp = dict(inputs(base))
    inp["bias"] = np.array([50.0] + [0.0] * 7, np.float32)
    cfg = moe.make_config(base)
    layer = moe.MoELayer(cfg, moe.upload(inp))
    layer.forward()
    torch.cuda.synchronize()
    C = oracle.capacity(1.0, 1000, 1, 8)
    assert C == 125
    sr = layer.view("slot_row").cpu().numpy()[:, 0]
    assert np.array_equal(sr[:C], np.arange(C)) and np.all(sr[C:] == -1)
    assert layer.view("expert_count").cpu().numpy().tolist() == [C] + [0] * 7
    y = host_float(layer.y)
    assert np.all(y[C:] == 0.0) and np.all(np.abs(y[:C]).sum(1) > 0)


@pytest.mark.gpu
def test_deterministic_bitwise():
    """No atomics on floating point: two runs give identical bits."""
    w = SMALL["correlated_small"]
    layer, _ = run_layer(w)
    y1 = layer.y.clone()
    xp1 = layer.view("x_perm").clone()
    layer.forward()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), layer.y.view(torch.int16))
    assert torch.equal(xp1.view(torch.int16), layer.view("x_perm").view(torch.int16))


@pytest.mark.gpu
def test_k_split_tiles_deterministic_bitwise():
    """Tiles cut along K are summed in piece order by whichever piece
    finishes last: repeated runs give identical bits."""
    w = SMALL["ksplit_down_small"]
    cfg = moe.make_config(w)
    assert moe.expert_ffn_workspace_bytes(cfg) > 0
    layer, _ = run_layer(w)
    y1 = layer.y.clone()
    h1 = layer.view("h").clone()
    for _ in range(3):
        layer.forward()
        torch.cuda.synchronize()
        assert torch.equal(h1.view(torch.int16), layer.view("h").view(torch.int16))
        assert torch.equal(y1.view(torch.int16), layer.y.view(torch.int16))


@pytest.mark.gpu
def test_skinny_split_deterministic_bitwise():
    """The weight-streaming kernel's K pieces are added in piece order:
    repeated runs give identical bits."""
    w = SMALL["skinny_decode_longk_small"]
    layer, _ = run_layer(w)
    y1 = layer.y.clone()
    for _ in range(3):
        layer.forward()
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), layer.y.view(torch.int16))


@pytest.mark.gpu
def test_empty_token_batch_is_a_noop():
    """T = 0: every entry point accepts empty (NULL) buffers; permute still
    writes zero counts and offsets."""
    w = W.small_variant(WL["mixtral_top2_bf16"], T=0, d=64, d_ff=64)
    cfg = moe.make_config(w)
    ws = moe.alloc_workspace(cfg)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    w1 = torch.zeros((8, 128, 64), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((8, 64, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    moe.layer_fwd(cfg, x, wr, w1, w2, y, ws)
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    f32 = torch.empty(0, dtype=torch.float32, device="cuda")
    moe.route(cfg, x, wr, f32, e32, f32)
    cnt = torch.full((8,), 7, dtype=torch.int32, device="cuda")
    load = torch.full((8,), 7, dtype=torch.int32, device="cuda")
    off = torch.full((9,), 7, dtype=torch.int32, device="cuda")
    moe.permute(cfg, x, x, e32, e32, cnt, load, off, topk_idx=e32)
    moe.expert_ffn(cfg, x, off, w1, w2, x, x)
    moe.unpermute(cfg, x, e32, f32, y)
    torch.cuda.synchronize()
    assert cnt.cpu().tolist() == [0] * 8 and load.cpu().tolist() == [0] * 8 and off.cpu().tolist() == [0] * 9


@pytest.mark.gpu
def test_one_expert_top1_is_a_dense_mlp_on_gpu():
    """E = 1, k = 1: the layer is one dense MLP; compared with the oracle and
    with torch's own fp32 matmul of the same bf16 values."""
    w = W.Workload("dense", T=300, d=256, E=1, k=1, d_ff=264, act=W.SWIGLU, dtype=W.BF16, routing=W.SOFTMAX_ALL)
    layer, inp = run_layer(w)
    x = moe.to_device(inp["x"]).float()
    w1 = moe.to_device(inp["w1"]).float()[0]
    w2 = moe.to_device(inp["w2"]).float()[0]
    hh = x @ w1.t()
    ref = (torch.nn.functional.silu(hh[:, :264]) * hh[:, 264:]) @ w2.t()
    err = max_rel_err(host_float(layer.y), ref.cpu().numpy())
    assert err <= TOL_Y[W.BF16]
