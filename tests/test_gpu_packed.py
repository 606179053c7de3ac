"""Packed expert weights on the GPU (moe_pack_weights, moe_expert_ffn_packed,
moe_layer_fwd_packed), through the C ABI.

* The packed buffer holds exactly the order include/moe.h documents, rebuilt
  here on the host from that description.
* The packed FFN gives the unpacked FFN's bits wherever both run the same
  kernel (>= 192 or <= 128 rows per expert on average), with ragged column
  tiles, empty and one-row experts, and K-split tiles; every case (also the
  129-191-row range, where the two orders run different kernels) is checked
  row by row against the fp64 oracle.
* The packed layer forward gives moe_layer_fwd's bits on small variants
  (shared expert, ExpertChoice) and on every bf16 workload at full size,
  whose sampled outputs are also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from _parity import (TOL_Y, check_output_ec, check_output_topk, check_routing_ec, check_routing_topk,
                     elem_rel_err, host_float, inputs, max_rel_err, sample_tokens, say, tile_cover_tokens)
from mixture_experts_layer_topkrouter_amd import moe
from mixture_experts_layer_topkrouter_amd import workloads as W

WL = W.WORKLOADS
# Small layers with packable widths (d_model, d_ff, d_ff_shared multiples of
# 64, column tiles still ragged): 256-row kernel, weight-streaming kernel
# (decode batches, capacity drops), a shared expert in both regimes,
# ExpertChoice, and 129-191 rows per expert (a different kernel than the
# unpacked order's: checked against the oracle only).
WL_SMALL_PACKED = {
    "mixtral_small": W.small_variant(WL["mixtral_top2_bf16"], T=1600, d=384, d_ff=576),
    "finegrained_small": W.small_variant(WL["finegrained_shared_bf16"], T=700, d=256, E=12, d_ff=192,
                                         d_ff_shared=320, wr_std=1.0 / 16.0),
    "decode_small": W.small_variant(WL["mixtral_top2_bf16"], T=64, d=512, E=8, d_ff=1024),
    "decode_shared_small": W.small_variant(WL["finegrained_shared_bf16"], T=48, d=256, E=12, d_ff=192,
                                           d_ff_shared=320, wr_std=1.0 / 16.0),
    "switch_small": W.small_variant(WL["switch_top1_bf16"], T=2000, d=192, E=16, d_ff=320),
    "correlated_ec_small": W.small_variant(WL["correlated_ec_bf16"], T=1500, d=256, E=16, d_ff=320,
                                           ec_capacity=200),
    "mid_rows_small": W.small_variant(WL["correlated_top2_bf16"], T=1200, d=256, E=16, d_ff=320),
}


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def kblock(a: np.ndarray) -> np.ndarray:
    """[rows, K] -> the K-blocked order [K/32][rows][32] include/moe.h describes."""
    R, K = a.shape
    return np.ascontiguousarray(a.reshape(R, K // 32, 32).transpose(1, 0, 2)).reshape(R, K)


def unkblock(a: np.ndarray) -> np.ndarray:
    R, K = a.shape
    return np.ascontiguousarray(a.reshape(K // 32, R, 32).transpose(1, 0, 2)).reshape(R, K)


def expected_packed(w: np.ndarray, n_out: int, swiglu: bool) -> np.ndarray:
    """The packed order of include/moe.h, from its description: column tiles
    of 256 weight rows (SwiGLU: 128 gate rows, then the matching up rows), K
    slices of 32, and in each 16 KB block 16-B chunk q = row q/4 at K chunk
    (q%4) ^ ((q/16)%4); rows past n_out are zero."""
    E, n_rows, K = w.shape
    tw = 128 if swiglu else 256
    tiles = -(-n_out // tw)
    out = np.zeros((E, tiles, K // 32, 256, 4, 8), np.uint16)
    for j in range(tiles):
        for r in range(256):
            col = j * 128 + r % 128 if swiglu else j * 256 + r
            if col >= n_out:
                continue
            src = col + (n_out if swiglu and r >= 128 else 0)
            for cs in range(4):
                c = cs ^ ((r >> 2) & 3)
                out[:, j, :, r, cs, :] = w[:, src, :].reshape(E, K // 32, 4, 8)[:, :, c, :]
    return out.reshape(-1)


@pytest.mark.gpu
@pytest.mark.parametrize("act,d,d_ff", [(W.SWIGLU, 128, 320), (W.GELU, 192, 448)])
def test_packed_order_is_the_documented_one(act, d, d_ff):
    say(f"[packed order] act={act} d={d} d_ff={d_ff}")
    rng = np.random.default_rng(3)
    E = 3
    n_up = 2 if act == W.SWIGLU else 1
    cfg = moe.MoeConfig(64, d, E, 1, d_ff, 0, 0.0, 0, W.BF16, act, W.SOFTMAX_TOPK)
    w1 = _bf16(rng.standard_normal((E, n_up * d_ff, d)))
    w2 = _bf16(rng.standard_normal((E, d, d_ff)))
    for which, w, n_out, sw in ((moe.PACK_W1, w1, d_ff, act == W.SWIGLU), (moe.PACK_W2, w2, d, False)):
        p = moe.pack_weights(cfg, which, w.cuda())
        torch.cuda.synchronize()
        got = p.cpu().numpy().view(np.uint16)
        ref = expected_packed(_bits(w), n_out, sw)
        assert got.size == ref.size == moe.packed_weight_bytes(cfg, which) // 2
        assert np.array_equal(got, ref), which
    # the shared expert's weights: one expert of width d_ff_shared
    cfg_s = moe.MoeConfig(64, d, E, 1, d_ff, 192, 0.0, 0, W.BF16, act, W.SOFTMAX_TOPK)
    ws1 = _bf16(rng.standard_normal((n_up * 192, d)))
    p = moe.pack_weights(cfg_s, moe.PACK_SHARED_W1, ws1.cuda())
    torch.cuda.synchronize()
    ref = expected_packed(_bits(ws1)[None], 192, act == W.SWIGLU)
    assert np.array_equal(p.cpu().numpy().view(np.uint16), ref)


# per-expert row counts: average >= 192 (256-row kernel in both orders),
# 129..191 (packed: 256-row kernel; unpacked: 128-row kernel), <= 128
# (weight-streaming kernel in both orders); empty and one-row experts, and
# counts on both sides of the row-tile boundaries
BIG = [0, 1, 127, 128, 129, 255, 256, 257, 383, 384, 385, 640, 700, 130]
MID = [150, 0, 1, 200, 190, 129, 257, 160, 140]
SMALL = [0, 1, 3, 63, 64, 65, 127, 128, 200, 17]


@pytest.mark.gpu
@pytest.mark.parametrize("act,d,d_ff,counts,tag", [
    (W.SWIGLU, 320, 320, BIG, "256-row"),
    (W.GELU, 192, 448, BIG, "256-row"),
    (W.SWIGLU, 320, 320, MID, "mid"),
    (W.SWIGLU, 320, 320, SMALL, "skinny"),
    (W.GELU, 192, 448, SMALL, "skinny"),
    (W.SWIGLU, 256, 8192, [300, 520, 0, 700], "256-row K-split"),
    (W.GELU, 128, 4096, [5, 40, 1, 90], "skinny K-split"),
    (W.GELU, 128, 8192, MID, "mid K-split"),
])
def test_packed_ffn_matches_unpacked_and_oracle(act, d, d_ff, counts, tag):
    counts = np.array(counts, np.int64)
    E, rows = len(counts), int(counts.sum())
    say(f"[packed ffn] {tag}: act={act} d={d} d_ff={d_ff} counts={counts.tolist()} (avg {rows // E})")
    rng = np.random.default_rng(11)
    n_up = 2 if act == W.SWIGLU else 1
    x = _bf16(rng.standard_normal((rows, d)))
    w1 = _bf16(rng.standard_normal((E, n_up * d_ff, d)) / np.sqrt(d))
    w2 = _bf16(rng.standard_normal((E, d, d_ff)) / np.sqrt(d_ff))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    cfg = moe.MoeConfig(rows, d, E, 1, d_ff, 0, 0.0, 0, W.BF16, act, W.SOFTMAX_TOPK)
    ws = moe.alloc_ffn_workspace(cfg)
    xd, offd, w1d, w2d = x.cuda(), torch.from_numpy(off).cuda(), w1.cuda(), w2.cuda()
    h0 = torch.empty((rows, d_ff), dtype=torch.bfloat16, device="cuda")
    y0 = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    moe.expert_ffn(cfg, xd, offd, w1d, w2d, h0, y0, ws)
    w1p = moe.pack_weights(cfg, moe.PACK_W1, w1d)
    w2p = moe.pack_weights(cfg, moe.PACK_W2, w2d)
    # x_perm row-major, then K-blocked (as moe_permute_packed writes it): the
    # same bits; h comes out K-blocked
    xkb = torch.from_numpy(kblock(_bits(x)).view(np.int16)).view(torch.bfloat16).cuda()
    outs = []
    for x_in, kb in ((xd, False), (xkb, True)):
        h1 = torch.full((rows, d_ff), 7.0, dtype=torch.bfloat16, device="cuda")
        y1 = torch.full((rows, d), 7.0, dtype=torch.bfloat16, device="cuda")
        moe.expert_ffn_packed(cfg, x_in, offd, w1p, w2p, h1, y1, ws, x_kblocked=kb)
        torch.cuda.synchronize()
        outs.append((h1, y1))
    (h1, y1), (h2, y2) = outs
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "K-blocked x_perm changes y"
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16)), "K-blocked x_perm changes h"
    # h rows of the kept rows (the rest of the buffer is not written)
    h1_rows = unkblock(_bits(h1))[:rows]
    if not tag.startswith("mid"):
        assert np.array_equal(h1_rows, _bits(h0)[:rows]), "h differs from the unpacked FFN"
        assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), "y differs from the unpacked FFN"
    got = host_float(y1)
    xb, w1b, w2b = _bits(x), _bits(w1), _bits(w2)
    # every row, or (large cases) every 4th row and each expert's first and
    # last rows of every 64-row tile
    step = 1 if rows * d * d_ff < 2e9 else 4
    for e in range(E):
        chk = set(range(off[e], off[e + 1], step))
        for r0 in range(off[e], off[e + 1], 64):
            chk |= {r0, min(r0 + 64, off[e + 1]) - 1}
        chk = sorted(chk)
        if not chk:
            continue
        ref = np.stack([oracle.ffn_row(xb[r], w1b[e], w2b[e], act) for r in chk])
        err = max_rel_err(got[chk], ref)
        if e == int(np.argmax(counts)):
            say(f"  expert {e}: max rel err {err:.3e}, element-wise {elem_rel_err(got[chk], ref):.3e} "
                f"over {len(chk)} rows")
        assert err <= TOL_Y[W.BF16], e


@pytest.mark.gpu
@pytest.mark.parametrize("T,d,E,k,cf,routing,path", [
    (700, 256, 12, 6, 0.0, W.SOFTMAX_ALL, "one launch"),
    (3000, 8192, 8, 2, 0.0, W.SOFTMAX_TOPK, "one launch, two passes per row"),
    (6000, 512, 16, 2, 1.0, W.SOFTMAX_ALL, "scan in every workgroup, capacity drops"),
    (40000, 128, 256, 2, 0.0, W.SOFTMAX_ALL, "separate scan launch"),
    (1500, 320, 16, 2, 0.0, W.EXPERT_CHOICE, "ExpertChoice"),
])
def test_permute_packed_is_permute_kblocked(T, d, E, k, cf, routing, path):
    """moe_permute_packed: every output of moe_permute, with x_perm in the
    K-blocked order (bit for bit once reordered on the host)."""
    say(f"[permute packed] {path}: T={T} d={d} E={E} k={k} cf={cf}")
    rng = np.random.default_rng(5)
    ec = routing == W.EXPERT_CHOICE
    C = 200 if ec else 0
    cfg = moe.MoeConfig(T, d, E, 0 if ec else k, 128, 0, cf, C, W.BF16, W.SWIGLU, routing)
    rows = moe.max_rows(cfg)
    x = _bf16(rng.standard_normal((T, d))).cuda()
    kw = {}
    if ec:
        tok = np.sort(np.stack([rng.choice(T, C, replace=False) for _ in range(E)]), axis=1).astype(np.int32)
        kw = dict(ec_token=torch.from_numpy(tok).cuda(), ec_w=torch.rand(E, C, device="cuda"),
                  slot_w=torch.empty(E * C, device="cuda"), tok_ptr=torch.empty(T + 1, dtype=torch.int32,
                                                                                  device="cuda"))
    else:
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        kw = dict(topk_idx=torch.from_numpy(idx).cuda(),
                  scratch=torch.empty(max(moe.permute_scratch_bytes(cfg), 16), dtype=torch.uint8, device="cuda"))
    outs = []
    for kb in (False, True):
        o = dict(x_perm=torch.zeros((rows, d), dtype=torch.bfloat16, device="cuda"),
                 row_token=torch.full((rows,), -7, dtype=torch.int32, device="cuda"),
                 slot_row=torch.empty(E * C if ec else T * k, dtype=torch.int32, device="cuda"),
                 cnt=torch.empty(E, dtype=torch.int32, device="cuda"),
                 load=torch.empty(E, dtype=torch.int32, device="cuda"),
                 off=torch.empty(E + 1, dtype=torch.int32, device="cuda"))
        moe.permute(cfg, x, o["x_perm"], o["row_token"], o["slot_row"], o["cnt"], o["load"], o["off"],
                    kblocked=kb, **kw)
        torch.cuda.synchronize()
        if ec:
            o["slot_w"], o["tok_ptr"] = kw["slot_w"].clone(), kw["tok_ptr"].clone()
        outs.append({n: t.cpu() for n, t in o.items()})
    plain, packed = outs
    for n in plain:
        if n != "x_perm":
            assert torch.equal(plain[n], packed[n]), n
    used = int(plain["off"][-1])
    xp = plain["x_perm"].view(torch.int16).numpy().view(np.uint16)
    xk = unkblock(packed["x_perm"].view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(xp[:used], xk[:used]), "K-blocked x_perm differs"


def _run_both(w: W.Workload):
    inp = inputs(w)
    cfg = moe.make_config(w)
    dev = moe.upload(inp)
    layer = moe.MoELayer(cfg, dev)
    layer.forward()
    torch.cuda.synchronize()
    y_plain = layer.y.clone()
    layer.y.fill_(7.0)
    layer.pack()
    layer.forward(packed=True)
    torch.cuda.synchronize()
    return layer, inp, y_plain


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(WL_SMALL_PACKED))
def test_packed_layer_matches_layer_fwd_small(name):
    w = WL_SMALL_PACKED[name]
    say(f"[packed layer small] {name}: T={w.T} d={w.d} E={w.E} d_ff={w.d_ff} shared={w.d_ff_shared}")
    layer, inp, y_plain = _run_both(w)
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


FULL_BF16 = ["mixtral_top2_bf16", "mixtral_decode_bf16", "finegrained_shared_bf16", "switch_top1_bf16",
             "correlated_top2_bf16", "correlated_ec_bf16"]


@pytest.mark.gpu
@pytest.mark.parametrize("name", FULL_BF16)
def test_packed_layer_full_size(name):
    """Full size, as the benchmark runs it: the packed forward's output is
    moe_layer_fwd's bit for bit, and sampled tokens (every row tile's first
    and last row among them) match the oracle."""
    w = W.WORKLOADS[name]
    say(f"[packed layer full] {name}: T={w.T} d={w.d} E={w.E} d_ff={w.d_ff}")
    layer, inp, y_plain = _run_both(w)
    assert torch.equal(layer.y.view(torch.int16), y_plain.view(torch.int16)), "packed layer differs"
    cover = tile_cover_tokens(w, layer)
    if w.routing == W.EXPERT_CHOICE:
        lg, sc, _ = check_routing_ec(w, layer, inp, kblocked=True)
        check_output_ec(w, layer, inp, lg, sc, sample_tokens(w, 8, extra=list(cover)))
    else:
        lg, _, _ = check_routing_topk(w, layer, inp, kblocked=True)
        check_output_topk(w, layer, inp, lg, sample_tokens(w, 8, extra=list(cover)))
