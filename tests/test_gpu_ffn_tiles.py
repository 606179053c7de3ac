"""GPU parity of the grouped expert FFN (moe_expert_ffn) on chosen per-expert
row counts: every row against the fp64 oracle's one-row FFN.

The counts put experts on both sides of the 128- and 256-row boundaries of
the 256-row kernel's row tiles, with empty and one-row experts among them,
and the output widths end in a partial column tile.
"""
import numpy as np
import pytest
import torch

import oracle
from _parity import TOL_Y, elem_rel_err, max_rel_err, say
from mixture_experts_layer_topkrouter_amd import moe
from mixture_experts_layer_topkrouter_amd import workloads as W

COUNTS = [0, 1, 127, 128, 129, 255, 256, 257, 383, 384, 385, 640, 700, 130]


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("act,d,d_ff", [(W.SWIGLU, 320, 288), (W.GELU, 256, 416)])
def test_expert_ffn_tile_heights_match_oracle(act, d, d_ff):
    counts = np.array(COUNTS, np.int64)
    E, rows = len(counts), int(counts.sum())
    assert rows // E >= 192  # the 256-row kernel's range
    rng = np.random.default_rng(7)
    n_up = 2 if act == W.SWIGLU else 1
    x = _bf16(rng.standard_normal((rows, d)))
    w1 = _bf16(rng.standard_normal((E, n_up * d_ff, d)) / np.sqrt(d))
    w2 = _bf16(rng.standard_normal((E, d, d_ff)) / np.sqrt(d_ff))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    # one token per row, top-1, no capacity: rows = T * k = the rows given
    cfg = moe.MoeConfig(rows, d, E, 1, d_ff, 0, 0.0, 0, W.BF16, act, W.SOFTMAX_TOPK)
    ws = moe.alloc_ffn_workspace(cfg)
    h = torch.empty((rows, d_ff), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    moe.expert_ffn(cfg, x.cuda(), torch.from_numpy(off).cuda(), w1.cuda(), w2.cuda(), h, y, ws)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    xb, w1b, w2b = _bits(x), _bits(w1), _bits(w2)
    ref = np.empty((rows, d))
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            ref[r] = oracle.ffn_row(xb[r], w1b[e], w2b[e], act)
    err = max_rel_err(got, ref)
    say(f"  expert FFN act={act} d={d} d_ff={d_ff} counts={COUNTS}: max rel err {err:.3e}, "
        f"element-wise {elem_rel_err(got, ref):.3e} (floor 1e-3 max|ref|)")
    assert err <= TOL_Y[W.BF16]
    for e in range(E):  # per expert too: a wrong tile would show in its own rows
        if counts[e]:
            assert max_rel_err(got[off[e]:off[e + 1]], ref[off[e]:off[e + 1]]) <= TOL_Y[W.BF16], e
