#!/usr/bin/env python3
"""Benchmark: MoE layer forward tokens/s on one MI355X.

One step = the whole forward pass of one MoE block (route, permute, grouped
expert FFN, shared expert when present, unpermute) over one batch of seeded
synthetic tokens already resident in HBM: one moe_layer_fwd_packed call
(the shared expert runs beside the rest on its side stream).  The expert
weights are packed once, before any timed region (moe_pack_weights: the
tile-major order in which the expert GEMMs stream them); the same layer on
the unpacked weights (moe_layer_fwd) is timed beside it and must give the
same bits (``weights``).  ``--unpacked`` times moe_layer_fwd instead; a
workload whose widths cannot be packed (fp32, or not multiples of 64) runs
unpacked.  ``value`` is the
wall-clock rate over the back-to-back calls; the same calls timed one by one
with HIP events give ``layer_fwd_median_ms``, and the layer captured once
into a HIP graph and replayed gives ``graph_replay``.  A second timed
region calls the individual entry points back to back on one stream (the
same kernels) with a HIP event between the stages, which gives each stage's
average duration; its output is checked to match moe_layer_fwd bit for bit.

Prints one JSON line.  ``roofline`` reports the grouped expert FFN (the
dominant stage: the kernels of one moe_expert_ffn call) against the bf16
MFMA peak, or against HBM bandwidth when its flops per byte of expert
weights and activations fall below the ridge (decode batches, few rows per
expert);
``stages`` gives every stage's time and its algorithmic HBM rate or FLOP rate;
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on the host cores.  ``backward`` times moe_layer_bwd (the layer's
backward pass for a seeded upstream gradient) in a region of its own after
the forward regions, in both modes: after a plain forward with the expert
pre-activations recomputed, and after the training forward that keeps them
(whose time is reported as ``train_fwd_ms``).  ``hbm_probe`` gives the
device's read, write and copy rates from the library's own stream kernels, and
the bf16 MFMA rate of a register-only loop (random and constant operands).
``workloads`` then measures every other workload the same way (median layer
time, tokens/s, stage medians with their algorithmic rates, the FFN's
roofline fraction), after the headline's timed regions.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DEFAULT_WORKLOAD = "mixtral_top2_bf16"
METRIC = "MoE layer fwd tokens/sec at 1 GPU; grouped-GEMM % MFMA peak; permute GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-sample", type=int, default=768, help="tokens the oracle computes for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-steps", type=int, default=20,
                    help="moe_layer_bwd calls timed after the forward regions (0: skip the backward)")
    ap.add_argument("--cold-iters", type=int, default=50,
                    help="per-stage cold timings: calls of each stage, each after a 512-MiB write that evicts "
                         "L2 and MALL; the median is reported (0: skip)")
    ap.add_argument("--no-hbm-probe", dest="hbm_probe", action="store_false",
                    help="skip the read / write / copy rate measurement of the device's HBM")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the HIP-graph replay timing of the layer")
    ap.add_argument("--no-workloads", dest="workloads", action="store_false",
                    help="skip the other workloads (each: median layer time and stage breakdown, "
                         "after the headline's timed regions)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (calibrates HBM byte counters)")
    ap.add_argument("--unpacked", dest="packed", action="store_false",
                    help="run the layer on the unpacked expert weights (moe_layer_fwd)")
    ap.add_argument("--traffic-run", action="store_true",
                    help="only the launches a profiler's HBM byte counters are read from: one step through the "
                         "stage entry points, then each stage again (3 calls of each in all, 5 of the shared "
                         "expert FFN), then one 1-GiB copy through the library's copy kernel for calibration")
    return ap.parse_args()


# Calls of each stage in a --traffic-run (the first within one whole step);
# the routed and the shared expert FFN run the same kernels, so their counts
# differ (3 against 5) to tell their dispatches apart.
TRAFFIC_CALLS = {"route": 3, "permute": 3, "expert_ffn": 3, "shared_ffn": 5, "unpermute": 3}
TRAFFIC_COPY_BYTES = 1 << 30


def algorithmic(w, n_rows: int, n_active: int, t_used: int = None):
    """Algorithmic work per stage (bytes or flops), from the kept rows N, the
    number of experts that received rows and the number of tokens with at
    least one kept row (t_used; default every token)."""
    s = w.elem_bytes
    T, d, E = w.T, w.d, w.E
    k = w.k if w.routing != 2 else 0
    A = w.assignments
    t_used = T if t_used is None else t_used
    n_mat = 3 if w.act == 1 else 2
    out = {}
    # x and W_r read, logits written, the bias read (per expert or per token),
    # then top-k indices and weights, or scores and the per-expert choice
    bias_b = {"none": 0, "expert": E * 4, "pairs": T * E * 4}[w.bias]
    route_b = T * d * s + E * d * s + T * E * 4 + bias_b + (T * k * 8 if k else T * E * 4 + E * w.ec_capacity * 8)
    out["route"] = ("bytes", route_b)
    # rows of tokens with a kept slot read once, kept rows written, indices
    out["permute"] = ("bytes", t_used * d * s + n_rows * d * s + A * 12)
    ffn_flops = n_rows * 2 * n_mat * d * w.d_ff
    w_bytes = n_active * n_mat * d * w.d_ff * s
    out["expert_ffn"] = ("flops", ffn_flops, w_bytes + n_rows * d * s * 2 + n_rows * w.d_ff * s * 2)
    if w.d_ff_shared:
        out["shared_ffn"] = ("flops", T * 2 * n_mat * d * w.d_ff_shared)
    out["unpermute"] = ("bytes", n_rows * d * s + T * d * s + (T * d * s if w.d_ff_shared else 0) + A * 8)
    return out


def measured_traffic(workload: str, stage: str = "expert_ffn"):
    """HBM bytes (read + written) per call of a stage from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (each scaled by a plain-copy
    calibration), or None when no such measurement exists or the stage's
    kernel sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("stages", {}).get(stage)
    if rec is None or stage_sources_sha256(stage) != rec.get("sources_sha256"):
        return None
    return int(rec["read_bytes"] + rec["write_bytes"])


# The kernel sources of each stage (with the shared device helpers).
COMMON_SOURCES = ("common.h", "kernels.h")
STAGE_SOURCES = {
    "route": ("route.hip",),
    "permute": ("permute.hip",),
    "expert_ffn": ("gemm_common.h", "gemm.hip", "gemm_skinny.hip"),
    "shared_ffn": ("gemm_common.h", "gemm.hip", "gemm_skinny.hip"),
    "unpermute": ("combine.hip",),
}


def stage_sources_sha256(stage: str) -> str:
    """One hash over a stage's kernel sources and the shared helpers, in a
    fixed order."""
    import hashlib
    h = hashlib.sha256()
    for name in STAGE_SOURCES[stage] + COMMON_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_topkrouter_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def packable(w, W) -> bool:
    """Expert weights the packed entry points take: bf16, widths multiples of 64."""
    return w.dtype == W.BF16 and w.d % 64 == 0 and w.d_ff % 64 == 0 and w.d_ff_shared % 64 == 0


def stage_functions(w, cfg, dev, layer, moe, W, torch, packed=False):
    """One callable per stage of the step-by-step path (route, permute, routed
    FFN, shared FFN, unpermute), on the intermediates of `layer`'s workspace;
    each rewrites only its own outputs, so any stage can be re-run on its own
    once a whole step has run.  packed: the steps of moe_layer_fwd_packed
    (moe_permute_packed writes x_perm K-blocked; the FFNs read the weights
    layer.pack() prepared, moe_expert_ffn_packed)."""
    T, E, d = w.T, w.E, w.d
    ec = w.routing == W.EXPERT_CHOICE
    V = layer.view
    logits = V("logits")
    x_perm, row_token, slot_row = V("x_perm"), V("row_token"), V("slot_row")
    cnt, load, off = V("expert_count"), V("expert_load"), V("expert_offset")
    h, y_perm = V("h"), V("y_perm")
    L = layer.layout
    scratch = layer.workspace[L["scratch"]:L["scratch"] + max(L["scratch_bytes"], 1)]
    ffn_ws = layer.workspace[L["ffn_scratch"]:L["ffn_scratch"] + L["ffn_scratch_bytes"]] if L["ffn_scratch_bytes"] else None
    sffn_ws = (layer.workspace[L["shared_ffn_scratch"]:L["shared_ffn_scratch"] + L["shared_ffn_scratch_bytes"]]
               if L["shared_ffn_scratch_bytes"] else None)
    if ec:
        scores, ec_token, ec_w = V("scores"), V("ec_token"), V("ec_w")
        slot_w, tok_ptr = V("slot_w"), V("tok_ptr")
    else:
        topk_idx, topk_w = V("topk_idx"), V("topk_w")
    if w.d_ff_shared:
        scfg = moe.MoeConfig(T, d, 1, 1, w.d_ff_shared, 0, 0.0, 0, w.dtype, w.act, W.SOFTMAX_ALL)
        soff = torch.tensor([0, T], dtype=torch.int32, device="cuda")
        hs, ys = V("shared_h"), V("shared_y")
    stream = torch.cuda.current_stream()
    names = ["route", "permute", "expert_ffn"] + (["shared_ffn"] if w.d_ff_shared else []) + ["unpermute"]

    def stage_fns():
        """One callable per stage, in order (each rewrites only its own outputs,
        so any stage can be re-run on its own once a whole step has run)."""
        fns = []
        if ec:
            fns.append(lambda: moe.route(cfg, dev.x, dev.wr, logits, bias=dev.bias, bias_stride=dev.bias_stride,
                                         scores=scores, ec_token=ec_token, ec_w=ec_w))
            fns.append(lambda: moe.permute(cfg, dev.x, x_perm, row_token, slot_row, cnt, load, off,
                                           ec_token=ec_token, ec_w=ec_w, slot_w=slot_w, tok_ptr=tok_ptr,
                                           kblocked=packed))
        else:
            fns.append(lambda: moe.route(cfg, dev.x, dev.wr, logits, topk_idx, topk_w, bias=dev.bias,
                                         bias_stride=dev.bias_stride))
            fns.append(lambda: moe.permute(cfg, dev.x, x_perm, row_token, slot_row, cnt, load, off,
                                           topk_idx=topk_idx, scratch=scratch, kblocked=packed))
        if packed:
            fns.append(lambda: moe.expert_ffn_packed(cfg, x_perm, off, layer.w1p, layer.w2p, h, y_perm, ffn_ws,
                                                     x_kblocked=True))
            if w.d_ff_shared:
                fns.append(lambda: moe.expert_ffn_packed(scfg, dev.x, soff, layer.ws1p, layer.ws2p, hs, ys, sffn_ws))
        else:
            fns.append(lambda: moe.expert_ffn(cfg, x_perm, off, dev.w1, dev.w2, h, y_perm, ffn_ws))
            if w.d_ff_shared:
                fns.append(lambda: moe.expert_ffn(scfg, dev.x, soff, dev.ws1, dev.ws2, hs, ys, sffn_ws))
        if ec:
            fns.append(lambda: moe.unpermute(cfg, y_perm, slot_row, slot_w, layer.y, tok_ptr=tok_ptr,
                                             y_shared=ys if w.d_ff_shared else None))
        else:
            fns.append(lambda: moe.unpermute(cfg, y_perm, slot_row, topk_w, layer.y,
                                             y_shared=ys if w.d_ff_shared else None))
        return fns

    return names, stage_fns()


def kept_counts(w, layer, W):
    """Kept rows N, experts with rows, and tokens with at least one kept row
    (read from the device after a step)."""
    V = layer.view
    n_rows = int(V("expert_offset")[-1].item())
    n_active = int((V("expert_count").cpu().numpy() > 0).sum())
    if w.routing == W.EXPERT_CHOICE:
        t_used = int((V("tok_ptr").diff() > 0).sum().item())
    else:
        t_used = int((V("slot_row") >= 0).any(dim=1).sum().item())
    return n_rows, n_active, t_used


def add_traffic(ent, w, n, work, sec):
    """The stage's measured HBM bytes per call (profiler counters, while its
    sources are unchanged), their rate and their ratio to the algorithmic
    bytes."""
    tb = measured_traffic(w.name, n)
    if tb is None:
        return
    alg = work[n][1] if work[n][0] == "bytes" else (work[n][2] if len(work[n]) > 2 else None)
    ent["traffic_bytes"] = tb
    ent["traffic_GB/s"] = round(tb / sec / 1e9, 1)
    if alg:
        ent["traffic_vs_algorithmic"] = round(tb / alg, 3)


def stage_rates(w, work, ms, peak_flops, peak_hbm):
    """Per-stage algorithmic rates from stage durations (ms)."""
    out = {}
    for n, t in ms.items():
        kind = work[n][0]
        sec = t / 1e3
        ent = {"median_ms": round(t, 4)}
        if kind == "bytes":
            ent["GB/s"] = round(work[n][1] / sec / 1e9, 1)
            ent["hbm_frac"] = round(work[n][1] / sec / 1e9 / peak_hbm, 4)
        else:
            ent["TFLOP/s"] = round(work[n][1] / sec / 1e12, 1)
            ent["mfma_frac"] = round(work[n][1] / sec / 1e12 / peak_flops, 4)
            if len(work[n]) > 2:
                ent["GB/s"] = round(work[n][2] / sec / 1e9, 1)
                ent["hbm_frac"] = round(work[n][2] / sec / 1e9 / peak_hbm, 4)
        add_traffic(ent, w, n, work, sec)
        out[n] = ent
    return out


def measure_workload(name, steps, warmup, moe, W, torch, packed=True):
    """One workload besides the headline one: the median layer forward time
    (HIP events around each of `steps` calls; packed weights where the
    workload allows, the unpacked forward's median beside it), tokens/s at
    that median, the median of every stage of the step-by-step path, and the
    FFN's roofline fraction (MFMA or HBM, by its intensity).  Outputs of all
    paths must agree bit for bit."""
    w = W.WORKLOADS[name]
    t_gen = time.time()
    inp = W.make_inputs(w, seed=0)
    t_gen = time.time() - t_gen
    cfg = moe.make_config(w)
    dev = moe.upload(inp)
    del inp
    layer = moe.MoELayer(cfg, dev)
    stream = torch.cuda.current_stream()
    packed = packed and packable(w, W)
    if packed:
        layer.pack()

    def median_fwd(pk):
        for _ in range(warmup):
            layer.forward(packed=pk)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            layer.forward(packed=pk)
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    bits = (lambda t: t.view(torch.int16)) if w.dtype == W.BF16 else (lambda t: t)
    unpacked_ms, unpacked_same = None, None
    if packed:
        unpacked_ms = median_fwd(False)
        y_unpacked = layer.y.clone()
    layer_ms = median_fwd(packed)
    y_layer = layer.y.clone()
    if packed:
        unpacked_same = bool(torch.equal(bits(y_unpacked), bits(y_layer)))
        del y_unpacked
    names, fns = stage_functions(w, cfg, dev, layer, moe, W, torch, packed)
    for _ in range(min(warmup, 3)):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for i in range(steps):
        for j, fn in enumerate(fns):
            evs[i][j].record(stream)
            fn()
        evs[i][len(fns)].record(stream)
    torch.cuda.synchronize()
    med = {n: float(np.median([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
           for j, n in enumerate(names)}
    same = bool(torch.equal(bits(y_layer), bits(layer.y)))
    n_rows, n_active, t_used = kept_counts(w, layer, W)
    work = algorithmic(w, n_rows, n_active, t_used)
    peak = PEAK_BF16_TFLOPS if w.dtype == W.BF16 else PEAK_F32_TFLOPS
    st = stage_rates(w, work, med, peak, PEAK_HBM_GBS)
    flops, fbytes = work["expert_ffn"][1], work["expert_ffn"][2]
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    ffn = st["expert_ffn"]
    out = {"T": w.T, "d_model": w.d, "num_experts": w.E, "top_k": w.k, "d_ff": w.d_ff, "d_ff_shared": w.d_ff_shared,
           "routing": w.routing, "dtype": "bf16" if w.dtype == W.BF16 else "f32", "kept_rows": n_rows,
           "active_experts": n_active, "tokens_with_kept_rows": t_used,
           "layer_fwd_median_ms": round(layer_ms, 4), "tokens_per_s": round(w.T / (layer_ms / 1e3), 1),
           "ffn_roofline": ({"bound": "mfma", "frac": ffn["mfma_frac"]} if flops / fbytes >= ridge
                            else {"bound": "hbm", "frac": ffn["hbm_frac"]}),
           "stages": st, "layer_fwd_matches_steps": same, "input_gen_s": round(t_gen, 1),
           "weights": {"order": "packed" if packed else "unpacked",
                       "unpacked_layer_fwd_median_ms": None if unpacked_ms is None else round(unpacked_ms, 4),
                       "unpacked_matches": unpacked_same}}
    del layer, dev
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU exchange is not built",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_layer_topkrouter_amd import moe
    from mixture_experts_layer_topkrouter_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)
    t_gen = time.time()
    inp = W.make_inputs(w, seed=0)
    t_gen = time.time() - t_gen
    cfg = moe.make_config(w)
    dev = moe.upload(inp)
    layer = moe.MoELayer(cfg, dev)  # owns the workspace and y; its views are the intermediates
    T, E, d = w.T, w.E, w.d
    ec = w.routing == W.EXPERT_CHOICE
    k = 0 if ec else w.k
    # packed expert weights: rearranged once, here, outside every timed region
    use_packed = args.packed and packable(w, W)
    pack_ms = None
    if use_packed:
        torch.cuda.synchronize()
        tp = time.perf_counter()
        layer.pack()
        torch.cuda.synchronize()
        pack_ms = (time.perf_counter() - tp) * 1e3
    fwd = lambda: layer.forward(packed=use_packed)
    names, fns = stage_functions(w, cfg, dev, layer, moe, W, torch, use_packed)
    stream = torch.cuda.current_stream()
    ec = w.routing == W.EXPERT_CHOICE
    V = layer.view
    off, cnt = V("expert_offset"), V("expert_count")

    def step(ev=None):
        for i, fn in enumerate(fns):
            if ev is not None:
                ev[i].record(stream)
            fn()
        if ev is not None:
            ev[len(fns)].record(stream)

    if args.traffic_run:
        # launches for a profiler's HBM byte counters: one step, then every
        # stage on its own until it has run TRAFFIC_CALLS times, then a known
        # copy through the library's stream kernel
        step()
        for n, fn in zip(names, fns):
            for _ in range(TRAFFIC_CALLS[n] - 1):
                fn()
        a = torch.ones(TRAFFIC_COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        moe.stream_probe("copy", a, b, TRAFFIC_COPY_BYTES)
        torch.cuda.synchronize()
        n_rows, n_active, t_used = kept_counts(w, layer, W)
        work = algorithmic(w, n_rows, n_active, t_used)
        print(json.dumps({"traffic_run": w.name, "calls": {n: TRAFFIC_CALLS[n] for n in names},
                          "copy_bytes": TRAFFIC_COPY_BYTES,
                          "algorithmic_bytes": {n: int(work[n][2] if work[n][0] == "flops" and len(work[n]) > 2
                                                       else work[n][1]) for n in names if
                                                work[n][0] == "bytes" or len(work[n]) > 2},
                          "sources_sha256": {n: stage_sources_sha256(n) for n in names}}), flush=True)
        return

    # The headline: K calls of moe_layer_fwd_packed (moe_layer_fwd with
    # --unpacked; the whole layer, shared expert overlapped on its side
    # stream), between two synchronisations.
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    y_layer = layer.y.clone()
    # the same calls one at a time between HIP events on the stream: the
    # median layer time (tokens/s at the median is reported beside `value`)
    lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in lev:
        a.record(stream)
        fwd()
        b.record(stream)
    torch.cuda.synchronize()
    layer_med_ms = float(np.median([a.elapsed_time(b) for a, b in lev]))
    bits = (lambda t: t.view(torch.int16)) if y_layer.dtype == torch.bfloat16 else (lambda t: t)
    # the same layer on the unpacked weights (moe_layer_fwd), timed the same
    # way: what packing saves, and the same bits
    weights = {"order": "packed" if use_packed else "unpacked"}
    if use_packed:
        for _ in range(min(args.warmup, 3)):
            layer.forward()
        torch.cuda.synchronize()
        uev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in uev:
            a.record(stream)
            layer.forward()
            b.record(stream)
        torch.cuda.synchronize()
        weights.update({"pack_ms_untimed": round(pack_ms, 2),
                        "unpacked_layer_fwd_median_ms": round(float(np.median([a.elapsed_time(b) for a, b in uev])), 4),
                        "unpacked_matches": bool(torch.equal(bits(y_layer), bits(layer.y)))})
    # the same layer captured once into a HIP graph and replayed K times (the
    # launches of one step become one graph launch; the outputs must match)
    graph = None
    if args.graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            fwd()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fwd()
        torch.cuda.synchronize()
        for _ in range(min(args.warmup, 3)):
            g.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter() - tg
        gsame = bool(torch.equal(y_layer.view(torch.int16) if y_layer.dtype == torch.bfloat16 else y_layer,
                                 layer.y.view(torch.int16) if layer.y.dtype == torch.bfloat16 else layer.y))
        graph = {"ms_per_step": round(tg * 1e3 / args.steps, 4), "tokens_per_s": round(T * args.steps / tg, 1),
                 "matches_eager": gsame}
        del g

    # Stage breakdown: the same kernels through the individual entry points,
    # one stream, HIP events between the stages (a second timed region).
    for _ in range(min(args.warmup, 3)):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(names)}
    stage_med = {n: float(np.median([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                 for j, n in enumerate(names)}
    ev_total_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][-1]) for i in range(args.steps)]))
    # the step-by-step path and moe_layer_fwd give the same bits
    same = bool(torch.equal(y_layer.view(torch.int16) if y_layer.dtype == torch.bfloat16 else y_layer,
                            layer.y.view(torch.int16) if layer.y.dtype == torch.bfloat16 else layer.y))

    # Cold stage timings: each stage alone, after a 512-MiB write on the same
    # stream that leaves neither L2 nor the 256-MB MALL holding its inputs;
    # median over the calls.
    cold_ms = None
    if args.cold_iters > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold_ms = {}
        for n, fn in zip(names, fns):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.cold_iters)]
            for a, b in ev:
                flush.fill_(1)
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            cold_ms[n] = float(np.median([a.elapsed_time(b) for a, b in ev]))
        del flush
        cold_same = bool(torch.equal(y_layer.view(torch.int16) if y_layer.dtype == torch.bfloat16 else y_layer,
                                     layer.y.view(torch.int16) if layer.y.dtype == torch.bfloat16 else layer.y))
        same = same and cold_same

    # Backward: moe_layer_bwd (recomputed expert pre-activations, data and
    # weight gradients, router and shared expert) for a seeded dy, after one
    # forward on the same inputs; HIP events on the stream around each call.
    bwd = None
    if args.bwd_steps > 0:
        dy = moe.to_device(W.make_dy(w, 0))

        def timed(fn, n):
            for _ in range(min(args.warmup, 3)):
                fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for a, b in ev:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            return float(np.mean([a.elapsed_time(b) for a, b in ev]))

        # recompute mode: after a plain forward, the backward re-runs GEMM1
        fwd()
        ms_re = timed(lambda: layer.backward(dy, recompute=True), args.bwd_steps)
        # training mode: the forward keeps the pre-activations, the backward
        # reads them
        ms_train_fwd = timed(lambda: layer.forward(train=True), args.bwd_steps)
        ms_saved = timed(lambda: layer.backward(dy, recompute=False), args.bwd_steps)
        bwd = {"recompute": {"ms": round(ms_re, 4)}, "saved_z": {"ms": round(ms_saved, 4)},
               "train_fwd_ms": round(ms_train_fwd, 4),
               "train_step_tokens_per_s": round(T / ((ms_train_fwd + ms_saved) / 1e3), 1)}

    # Practical HBM stream rates of this device, for reading the HBM-bound
    # stages against: the library's own read, write and copy kernels
    # (moe_stream_probe: 16-B accesses, one 16-KB run per 256-thread workgroup), plain and
    # non-temporal, each over 1 GiB, median of 5 event-timed runs.
    hbm_probe = None
    if args.hbm_probe:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")

        def rate(kind, nt, moved):
            fn = lambda: moe.stream_probe(kind, src, dst, nbytes, nontemporal=nt, sink=sink)
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return round(moved / (float(np.median(ts)) / 1e3) / 1e9, 1)

        hbm_probe = {"bytes": nbytes, "kernel": "moe_stream_probe (16-B accesses, one 16-KB run per 256-thread workgroup)"}
        for nt in (False, True):
            tag = "_nt" if nt else ""
            hbm_probe["read" + tag + "_GB/s"] = rate("read", nt, nbytes)
            hbm_probe["write" + tag + "_GB/s"] = rate("write", nt, nbytes)
            hbm_probe["copy" + tag + "_GB/s"] = rate("copy", nt, 2 * nbytes)
        del src, dst
        # the bf16 MFMA rate of a register-only loop (moe_mfma_probe: no
        # memory traffic), on random operands and on constant ones: the
        # matrix core's power, and so the clock it holds, depends on the data
        blocks, iters = 512, 4096
        flops = blocks * 4 * iters * 8 * 32768
        g = torch.Generator(device="cuda").manual_seed(7)
        ops = {"random": torch.randn(blocks * 16384, device="cuda", generator=g).to(torch.bfloat16),
               "constant": torch.full((blocks * 16384,), 0.5, dtype=torch.bfloat16, device="cuda")}
        mfma = {"kernel": "moe_mfma_probe (8 independent 32x32x16 bf16 MFMA accumulators per wave, 4 waves x "
                          f"{blocks} workgroups, {iters} rounds)", "flops": flops}
        for name, op in ops.items():
            moe.mfma_probe(blocks, iters, op)
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                moe.mfma_probe(blocks, iters, op)
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            tf = flops / (float(np.median(ts)) / 1e3) / 1e12
            mfma[name + "_TFLOP/s"] = round(tf, 1)
            mfma[name + "_frac_of_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
        hbm_probe["mfma"] = mfma
        del ops

    if args.copy_probe_mib:
        # one known-size copy through the library's copy kernel (calibrates
        # the HBM byte counters of a profiler run)
        a = torch.ones((args.copy_probe_mib << 20) // 2, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        moe.stream_probe("copy", a, b, args.copy_probe_mib << 20)
        torch.cuda.synchronize()
        del a, b

    n_rows, n_active, t_used = kept_counts(w, layer, W)
    work = algorithmic(w, n_rows, n_active, t_used)
    stages = {}
    for n in names:
        kind = work[n][0]
        sec = stage_ms[n] / 1e3
        ent = {"ms": round(stage_ms[n], 4), "median_ms": round(stage_med[n], 4)}
        if kind == "bytes":
            ent["GB/s"] = round(work[n][1] / sec / 1e9, 1)
            ent["hbm_frac"] = round(work[n][1] / sec / 1e9 / PEAK_HBM_GBS, 4)
            ent["bytes"] = int(work[n][1])
            if cold_ms is not None:
                ent["cold_median_ms"] = round(cold_ms[n], 4)
                ent["cold_GB/s"] = round(work[n][1] / (cold_ms[n] / 1e3) / 1e9, 1)
                ent["cold_hbm_frac"] = round(work[n][1] / (cold_ms[n] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)
        else:
            tf = work[n][1] / sec / 1e12
            peak = PEAK_BF16_TFLOPS if w.dtype == W.BF16 else PEAK_F32_TFLOPS
            ent["TFLOP/s"] = round(tf, 1)
            ent["mfma_frac" if w.dtype == W.BF16 else "fp32_frac"] = round(tf / peak, 4)
            ent["flops"] = int(work[n][1])
            if cold_ms is not None:
                ent["cold_median_ms"] = round(cold_ms[n], 4)
                ent["cold_TFLOP/s"] = round(work[n][1] / (cold_ms[n] / 1e3) / 1e12, 1)
            if len(work[n]) > 2:
                ent["min_bytes"] = int(work[n][2])
                ent["GB/s"] = round(work[n][2] / sec / 1e9, 1)
                ent["hbm_frac"] = round(work[n][2] / sec / 1e9 / PEAK_HBM_GBS, 4)
        add_traffic(ent, w, n, work, sec)
        stages[n] = ent

    if bwd is not None:
        # expert GEMM flops of the backward on the kept rows (no pad rows):
        # recomputed z (n_up*d_ff x d; recompute mode only), dh (d_ff x d),
        # dx (n_up*d_ff x d), dW2 (d x d_ff), dW1 (n_up*d_ff x d), and the same
        # over all T tokens for the shared expert
        n_up = 2 if w.act == 1 else 1
        peak_b = PEAK_BF16_TFLOPS if w.dtype == W.BF16 else PEAK_F32_TFLOPS
        for mode, units in (("recompute", 3 * n_up + 2), ("saved_z", 2 * n_up + 2)):
            gflops = 2 * (n_rows * w.d_ff + T * w.d_ff_shared) * d * units
            tf = gflops / (bwd[mode]["ms"] / 1e3) / 1e12
            bwd[mode].update({"expert_gemm_flops": int(gflops), "TFLOP/s_whole_pass": round(tf, 1),
                              "frac_of_peak_whole_pass": round(tf / peak_b, 4)})

    # The dominant kernel is the grouped expert FFN (every kernel of one
    # moe_expert_ffn call).  Its bound follows from its arithmetic intensity:
    # at or above the ridge (peak flops / peak bytes) the matrix core, below
    # it the stream of expert weights from HBM.
    ffn_flops, ffn_bytes = work["expert_ffn"][1], work["expert_ffn"][2]
    ffn_s = stage_ms["expert_ffn"] / 1e3
    peak = PEAK_BF16_TFLOPS if w.dtype == W.BF16 else PEAK_F32_TFLOPS
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    common = {"traffic": measured_traffic(w.name),
              "kernel": "grouped expert FFN: every kernel of one moe_expert_ffn" + ("_packed" if use_packed else "")
                        + " call",
              "avg_ms": round(stage_ms["expert_ffn"], 4), "flops_per_launch": int(ffn_flops),
              "bytes_per_launch": int(ffn_bytes), "intensity_flop_per_byte": round(ffn_flops / ffn_bytes, 1)}
    if ffn_flops / ffn_bytes >= ridge:
        achieved = ffn_flops / ffn_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), **common}
    else:
        achieved = ffn_bytes / ffn_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), **common}

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        rng = np.random.default_rng(123)
        toks = np.sort(rng.choice(T, size=min(args.cpu_sample, T), replace=False)).astype(np.int32)
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        tc = time.perf_counter()
        ref = oracle.layer(inp["x"], inp["wr"], inp["w1"], inp["w2"], k=w.k, routing=w.routing, act=w.act, cf=w.cf,
                           ec_capacity=w.ec_capacity, bias=inp["bias"], bias_stride=inp["bias_stride"],
                           ws1=inp["ws1"], ws2=inp["ws2"], toks=toks)
        tc = time.perf_counter() - tc
        cpu_model = None
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
        except OSError:
            pass
        cpu = {"value": round(len(toks) / tc, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model,
               "sample": f"fp64 oracle: router logits, gate and dispatch of all {T} tokens plus the expert FFN "
                         f"and combine of {len(toks)} sampled tokens; value = sampled tokens / wall time "
                         f"({tc:.1f} s)"}
        y = layer.y.float().cpu().numpy().astype(np.float64)[toks]
        parity = float(np.max(np.abs(y - ref.y)) / np.max(np.abs(ref.y)))

    # Every other workload, measured after the headline's timed regions: the
    # layer at its median, the stage breakdown and the FFN's roofline.
    others = None
    if args.workloads:
        others = {}
        for name in W.WORKLOADS:
            if name != w.name:
                others[name] = measure_workload(name, args.steps, args.warmup, moe, W, torch, args.packed)

    out = {
        "metric": METRIC,
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == W.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "d_model": d, "num_experts": E, "top_k": w.k, "d_ff": w.d_ff,
                   "d_ff_shared": w.d_ff_shared, "capacity_factor": w.cf, "routing": w.routing, "act": w.act,
                   "kept_rows": n_rows, "active_experts": n_active, "tokens_with_kept_rows": t_used},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": stages,
        "backward": bwd,
        "event_ms_per_step": round(ev_total_ms, 4),
        "layer_fwd_median_ms": round(layer_med_ms, 4),
        "weights": weights,
        "graph_replay": graph,
        "hbm_probe": hbm_probe,
        "tokens_per_s_at_median": round(T / (layer_med_ms / 1e3), 1),
        "layer_fwd_matches_steps": same,
        "parity_max_rel_err_sampled": parity,
        "device": dev_name,
        "input_gen_s": round(t_gen, 1),
        "workloads": others,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
