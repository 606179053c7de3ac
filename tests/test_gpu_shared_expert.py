"""The shared expert beside the routed experts, on the 256 x 256 GEMM.

moe_layer_fwd runs the shared expert ("How MegaDLMs Implements Mixture of
Experts (MoE) Architectures", Core MoE Layer Architecture: an always-on
expert that every token passes through, added to the routed output) as one
expert over all T tokens on a side stream beside the routed path, and the
combine adds its row with weight 1.  The layer must give exactly the bits of
the entry points called one by one (moe_expert_ffn for the routed experts,
again for the shared expert, then moe_unpermute), and the packed weights
(moe_layer_fwd_packed) the bits of the unpacked ones; every token is also
checked against the fp64 oracle.

The shapes put both FFNs on the 256-row kernel (bf16, every width a multiple
of 64, at least 192 routed rows per expert on average, more than 128 tokens,
no contraction long enough to be cut along K): a shared expert wider than the
routed ones, a narrower one, an equal one with GELU, and ragged token counts
(partial row tiles in both FFNs).
"""
import numpy as np
import pytest
import torch

from _parity import check_output_topk, check_routing_topk, inputs, say
from mixture_experts_layer_topkrouter_amd import moe
from mixture_experts_layer_topkrouter_amd import workloads as W

WL = W.WORKLOADS
BASE = WL["finegrained_shared_bf16"]

CASES = {
    "wide_shared_swiglu": BASE.replace(name="wide_shared_swiglu", T=1000, d=256, E=8, k=2, d_ff=256,
                                       d_ff_shared=512, wr_std=1.0 / 16.0),
    "narrow_shared_swiglu": BASE.replace(name="narrow_shared_swiglu", T=901, d=320, E=6, k=3, d_ff=384,
                                         d_ff_shared=128, wr_std=1.0 / np.sqrt(320.0)),
    "equal_shared_gelu": BASE.replace(name="equal_shared_gelu", T=1300, d=192, E=5, k=1, d_ff=320,
                                      d_ff_shared=320, act=W.GELU, wr_std=1.0 / np.sqrt(192.0)),
}


def _on_256_row_kernel(w: W.Workload) -> bool:
    """Both FFNs of the layer on the 256 x 256 kernel without a K split
    (the host's kernel choice, restated for the test shapes)."""
    cfg = moe.make_config(w)
    avg = moe.max_rows(cfg) // w.E
    stages_ok = all(n % 32 == 0 and n // 32 < 256 for n in (w.d, w.d_ff, w.d_ff_shared))
    packable = all(n % 64 == 0 for n in (w.d, w.d_ff, w.d_ff_shared))
    return w.dtype == W.BF16 and stages_ok and packable and avg >= 192 and w.T > 128


def _step_by_step(w: W.Workload, layer):
    """moe_route .. moe_unpermute one by one, the shared expert's FFN as its
    own moe_expert_ffn call (unpacked weights)."""
    cfg = layer.cfg
    dev = layer.dev
    T, E, k, d = w.T, w.E, w.k, w.d
    rows = moe.max_rows(cfg)
    dt = moe.torch_dtype(cfg)
    c = "cuda"
    logits = torch.empty((T, E), dtype=torch.float32, device=c)
    idx = torch.empty((T, k), dtype=torch.int32, device=c)
    tw = torch.empty((T, k), dtype=torch.float32, device=c)
    moe.route(cfg, dev.x, dev.wr, logits, idx, tw, bias=dev.bias, bias_stride=dev.bias_stride)
    x_perm = torch.empty((rows, d), dtype=dt, device=c)
    row_token = torch.empty(rows, dtype=torch.int32, device=c)
    slot_row = torch.empty((T, k), dtype=torch.int32, device=c)
    cnt = torch.empty(E, dtype=torch.int32, device=c)
    load = torch.empty(E, dtype=torch.int32, device=c)
    off = torch.empty(E + 1, dtype=torch.int32, device=c)
    scratch = torch.empty(moe.permute_scratch_bytes(cfg), dtype=torch.uint8, device=c)
    moe.permute(cfg, dev.x, x_perm, row_token, slot_row, cnt, load, off, topk_idx=idx, scratch=scratch)
    h = torch.empty((rows, w.d_ff), dtype=dt, device=c)
    y_perm = torch.empty((rows, d), dtype=dt, device=c)
    moe.expert_ffn(cfg, x_perm, off, dev.w1, dev.w2, h, y_perm, moe.alloc_ffn_workspace(cfg))
    scfg = moe.MoeConfig(T, d, 1, 1, w.d_ff_shared, 0, 0.0, 0, w.dtype, w.act, W.SOFTMAX_ALL)
    soff = torch.tensor([0, T], dtype=torch.int32, device=c)
    hs = torch.empty((T, w.d_ff_shared), dtype=dt, device=c)
    ys = torch.empty((T, d), dtype=dt, device=c)
    moe.expert_ffn(scfg, dev.x, soff, dev.ws1, dev.ws2, hs, ys, moe.alloc_ffn_workspace(scfg))
    y = torch.empty((T, d), dtype=dt, device=c)
    moe.unpermute(cfg, y_perm, slot_row, tw, y, y_shared=ys)
    torch.cuda.synchronize()
    return y, ys


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_shared_expert_layer_matches_separate_launches(name):
    w = CASES[name]
    assert _on_256_row_kernel(w), "test shape off the 256-row kernel"
    say(f"[shared expert] {name}: T={w.T} d={w.d} E={w.E} k={w.k} d_ff={w.d_ff} shared={w.d_ff_shared} act={w.act}")
    inp = inputs(w)
    cfg = moe.make_config(w)
    layer = moe.MoELayer(cfg, moe.upload(inp))
    layer.forward()
    torch.cuda.synchronize()
    y_layer = layer.y.clone()
    ys_layer = layer.view("shared_y").clone()
    y_steps, ys_steps = _step_by_step(w, layer)
    assert torch.equal(_bits(ys_layer), _bits(ys_steps)), "shared expert output differs from its own call"
    assert torch.equal(_bits(y_layer), _bits(y_steps)), "layer output differs from the entry points one by one"
    # packed weights: the same kernels on the packed orders, same bits
    layer.y.fill_(3.0)
    layer.pack()
    layer.forward(packed=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(layer.y), _bits(y_layer)), "packed layer differs"
    # and the oracle, every token
    lg, _, _ = check_routing_topk(w, layer, inp, kblocked=True)
    check_output_topk(w, layer, inp, lg, np.arange(w.T, dtype=np.int32))
