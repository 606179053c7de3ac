"""The C-ABI library: it loads, exports every function include/moe.h declares,
and rejects invalid arguments on the host before anything reaches a GPU
(these calls enqueue nothing, so they run without one)."""
import ctypes

import pytest
import torch

from mixture_experts_layer_topkrouter_amd import moe
from mixture_experts_layer_topkrouter_amd import workloads as W


def test_library_exports_every_header_symbol():
    lib = moe.load_library()
    syms = moe.header_symbols()
    assert len(syms) >= 11
    for s in syms:
        assert hasattr(lib, s), s
    for s in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_unpermute", "moe_layer_fwd", "moe_layer_bwd",
              "moe_layer_bwd_workspace"):
        assert s in syms


def test_status_strings_and_version():
    lib = moe.load_library()
    assert lib.moe_abi_version() == 7
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(3) == b"workspace too small"


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_rows_capacity_and_workspace_sizes(name):
    w = W.WORKLOADS[name]
    cfg = moe.make_config(w)
    cap = moe.capacity(cfg)
    if w.routing == W.EXPERT_CHOICE:
        assert cap == -1 and moe.max_rows(cfg) == w.E * w.ec_capacity
    elif w.cf == 0:
        assert cap == -1 and moe.max_rows(cfg) == w.T * w.k
    else:
        assert cap == {"tiny_top2_fp32": 80, "switch_top1_bf16": 128}[name]
        assert moe.max_rows(cfg) == min(w.T * w.k, cap * w.E)
    L = moe.layer_workspace(cfg)
    assert L["total"] >= L["y_perm"] + moe.max_rows(cfg) * w.d * w.elem_bytes
    offs = [L[n] for n in ("logits", "x_perm", "h", "y_perm", "ffn_scratch", "total")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    ffn = moe.expert_ffn_workspace_bytes(cfg)
    assert L["ffn_scratch_bytes"] >= ffn and L["ffn_scratch"] + L["ffn_scratch_bytes"] <= L["total"]
    assert ffn == expected_ffn_workspace(w.dtype, moe.max_rows(cfg) // w.E, w.d, w.d_ff)


def expected_ffn_workspace(dtype, avg_rows, d, d_ff):
    """K-split partial tiles: 256 of 256 x 256 fp32 for the 256-row kernel
    (>= 192 rows per expert on average, a reduction length >= 8192); 512 of
    64 x 256 fp32 for the weight-streaming kernel (<= 128 rows per expert on
    average, K a multiple of 64).  With packable widths (d and d_ff multiples
    of 64) the packed FFN's need counts too: it runs the 256-row kernel from
    129 rows per expert on."""
    if dtype == W.F32:
        return 0
    need = 0
    if avg_rows >= 192 and max(d, d_ff) >= 8192:
        need = 256 * 256 * 256 * 4
    if avg_rows <= 128 and (d % 64 == 0 or d_ff % 64 == 0):
        need = max(need, 512 * 64 * 256 * 4)
    if d % 64 == 0 and d_ff % 64 == 0 and avg_rows > 128 and max(d, d_ff) >= 8192:
        need = max(need, 256 * 256 * 256 * 4)
    return need


def _ceil(a, b):
    return -(-a // b)


@pytest.mark.parametrize("act,d,d_ff,dffs,E", [(1, 4096, 14336, 0, 8), (0, 192, 448, 320, 3), (1, 128, 320, 192, 5),
                                               (0, 64, 64, 64, 1)])
def test_packed_weight_bytes(act, d, d_ff, dffs, E):
    """E * column tiles * (K / 32) * 16 KB; SwiGLU's W1 has tiles of 128
    d_ff columns (gate and up rows together), every other weight tiles of
    256 output rows."""
    cfg = _cfg(d_model=d, num_experts=E, top_k=1, d_ff=d_ff, d_ff_shared=dffs, act=act)
    tw = 128 if act == 1 else 256
    assert moe.packed_weight_bytes(cfg, moe.PACK_W1) == E * _ceil(d_ff, tw) * (d // 32) * 16384
    assert moe.packed_weight_bytes(cfg, moe.PACK_W2) == E * _ceil(d, 256) * (d_ff // 32) * 16384
    if dffs:
        assert moe.packed_weight_bytes(cfg, moe.PACK_SHARED_W1) == _ceil(dffs, tw) * (d // 32) * 16384
        assert moe.packed_weight_bytes(cfg, moe.PACK_SHARED_W2) == _ceil(d, 256) * (dffs // 32) * 16384


def test_packed_argument_errors():
    lib = moe.load_library()
    fake = ctypes.c_void_p(256)
    n = ctypes.c_size_t(0)
    cfg = _cfg(d_ff_shared=128)
    assert lib.moe_packed_weight_bytes(ctypes.byref(cfg), 4, ctypes.byref(n)) == 1  # unknown weight
    assert lib.moe_packed_weight_bytes(ctypes.byref(_cfg()), moe.PACK_SHARED_W1, ctypes.byref(n)) == 1  # no shared
    assert lib.moe_packed_weight_bytes(ctypes.byref(cfg), 0, None) == 1
    # fp32, or a width that is not a multiple of 64: not packable
    assert lib.moe_packed_weight_bytes(ctypes.byref(_cfg(dtype=0)), 0, ctypes.byref(n)) == 2
    assert lib.moe_packed_weight_bytes(ctypes.byref(_cfg(d_ff=72)), 0, ctypes.byref(n)) == 2
    assert lib.moe_packed_weight_bytes(ctypes.byref(_cfg(d_model=96)), 1, ctypes.byref(n)) == 2
    assert lib.moe_packed_weight_bytes(ctypes.byref(_cfg(d_ff_shared=72)), 2, ctypes.byref(n)) == 2
    assert lib.moe_packed_weight_bytes(ctypes.byref(_cfg(d_ff_shared=72)), 0, ctypes.byref(n)) == 0
    # packing: null, aliased or misaligned buffers
    assert lib.moe_pack_weights(ctypes.byref(cfg), 0, None, fake, None) == 1
    assert lib.moe_pack_weights(ctypes.byref(cfg), 0, fake, None, None) == 1
    assert lib.moe_pack_weights(ctypes.byref(cfg), 0, fake, fake, None) == 1
    assert lib.moe_pack_weights(ctypes.byref(cfg), 0, ctypes.c_void_p(264), ctypes.c_void_p(4096), None) == 1
    assert lib.moe_pack_weights(ctypes.byref(_cfg(dtype=0)), 0, fake, ctypes.c_void_p(4096), None) == 2
    # the packed FFN and layer refuse configurations they cannot run
    st = lib.moe_expert_ffn_packed(ctypes.byref(_cfg(dtype=0)), fake, 0, fake, fake, fake, fake, fake, fake,
                                   1 << 30, None)
    assert st == 2
    st = lib.moe_expert_ffn_packed(ctypes.byref(_cfg(d_ff=200)), fake, 1, fake, fake, fake, fake, fake, fake,
                                   1 << 30, None)
    assert st == 2
    st = lib.moe_expert_ffn_packed(ctypes.byref(cfg), fake, 2, fake, fake, fake, fake, fake, fake, 1 << 30, None)
    assert st == 1  # x_perm order neither row-major nor K-blocked
    # the K-blocked permutation: packable configurations only
    st = lib.moe_permute_packed(ctypes.byref(_cfg(dtype=0)), fake, fake, None, None, fake, fake, fake, None, None,
                                fake, fake, fake, fake, 1 << 20, None)
    assert st == 2
    st = lib.moe_layer_fwd_packed(ctypes.byref(_cfg(d_ff_shared=72)), fake, fake, None, 0, fake, fake, fake, fake,
                                  fake, fake, 1 << 30, None)
    assert st == 2
    # missing shared-expert weights
    st = lib.moe_layer_fwd_packed(ctypes.byref(cfg), fake, fake, None, 0, fake, fake, None, None, fake, fake,
                                  1 << 30, None)
    assert st == 1
    # an empty batch is a no-op on the packed path too (nothing is enqueued;
    # empty buffers may be NULL)
    empty = _cfg(num_tokens=0, d_ff_shared=128)
    assert lib.moe_layer_fwd_packed(ctypes.byref(empty), None, None, None, 0, None, None, None, None, None, None, 0,
                                    None) == 0
    assert lib.moe_expert_ffn_packed(ctypes.byref(empty), None, 1, None, None, None, None, None, None, 0, None) == 0
    # the binding checks the packed buffer's size before the call
    small = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="needs at least"):
        moe.expert_ffn_packed(cfg, None, None, small, small, None, None)
    with pytest.raises(TypeError):
        moe.pack_weights(cfg, moe.PACK_W1, torch.empty(64 * 128, dtype=torch.float32), small)


@pytest.mark.parametrize("T,d,E,k,d_ff", [(64, 512, 8, 2, 1024), (1200, 256, 16, 1, 512), (4096, 256, 8, 2, 8192),
                                          (700, 264, 4, 2, 264), (16, 64, 4, 1, 64), (2400, 256, 16, 1, 8192),
                                          (2400, 264, 16, 1, 8192)])
def test_ffn_workspace_rule(T, d, E, k, d_ff):
    cfg = _cfg(num_tokens=T, d_model=d, num_experts=E, top_k=k, d_ff=d_ff)
    assert moe.expert_ffn_workspace_bytes(cfg) == expected_ffn_workspace(W.BF16, T * k // E, d, d_ff)


def _cfg(**kw):
    base = dict(num_tokens=64, d_model=64, num_experts=8, top_k=2, d_ff=64, d_ff_shared=0, capacity_factor=0.0,
                ec_capacity=0, dtype=1, act=1, routing=0)
    base.update(kw)
    return moe.MoeConfig(**base)


@pytest.mark.parametrize("bad", [dict(top_k=0), dict(top_k=9), dict(num_tokens=-1), dict(d_model=60),
                                 dict(d_ff=100), dict(capacity_factor=-1.0), dict(capacity_factor=float("nan")),
                                 dict(routing=7), dict(dtype=5), dict(act=3), dict(num_experts=0),
                                 dict(routing=2, ec_capacity=0), dict(routing=2, ec_capacity=65)])
def test_invalid_configs_are_rejected_before_launch(bad):
    lib = moe.load_library()
    cfg = _cfg(**bad)
    n = ctypes.c_size_t(0)
    assert lib.moe_permute_scratch_bytes(ctypes.byref(cfg), ctypes.byref(n)) == 1
    L = moe.WorkspaceLayout()
    assert lib.moe_layer_workspace(ctypes.byref(cfg), ctypes.byref(L)) == 1
    # compute entry points refuse too, without touching (fake) pointers
    fake = ctypes.c_void_p(16)
    st = lib.moe_layer_fwd(ctypes.byref(cfg), fake, fake, None, 0, fake, fake, None, None, fake, ctypes.c_void_p(256),
                           1 << 30, None)
    assert st == 1


def test_unsupported_and_workspace_errors():
    lib = moe.load_library()
    assert lib.moe_max_rows(ctypes.byref(_cfg(num_experts=300, top_k=2))) == -1
    L = moe.WorkspaceLayout()
    assert lib.moe_layer_workspace(ctypes.byref(_cfg(num_experts=300)), ctypes.byref(L)) == 2
    assert lib.moe_layer_workspace(ctypes.byref(_cfg(routing=2, ec_capacity=4, num_tokens=20000)),
                                   ctypes.byref(L)) == 2
    cfg = _cfg()
    fake = ctypes.c_void_p(256)
    # workspace too small -> MOE_ERR_WORKSPACE, nothing enqueued
    st = lib.moe_layer_fwd(ctypes.byref(cfg), fake, fake, None, 0, fake, fake, None, None, fake, fake, 16, None)
    assert st == 3
    # misaligned pointer -> invalid argument
    st = lib.moe_layer_fwd(ctypes.byref(cfg), ctypes.c_void_p(8), fake, None, 0, fake, fake, None, None, fake, fake,
                           1 << 30, None)
    assert st == 1
    # expert FFN without the workspace its configuration needs -> MOE_ERR_WORKSPACE
    big = _cfg(num_tokens=4096, d_model=256, d_ff=8192)
    need = moe.expert_ffn_workspace_bytes(big)
    assert need > 0
    st = lib.moe_expert_ffn(ctypes.byref(big), fake, fake, fake, fake, fake, fake, None, 0, None)
    assert st == 3
    st = lib.moe_expert_ffn(ctypes.byref(big), fake, fake, fake, fake, fake, fake, fake, need - 1, None)
    assert st == 3
    # misaligned workspace -> invalid argument
    st = lib.moe_expert_ffn(ctypes.byref(big), fake, fake, fake, fake, fake, fake, ctypes.c_void_p(272), need, None)
    assert st == 1
    # null output -> invalid argument
    st = lib.moe_unpermute(ctypes.byref(cfg), fake, None, fake, fake, None, None, None)
    assert st == 1


@pytest.mark.parametrize("kw", [dict(d_model=1 << 22), dict(d_ff=1 << 22), dict(d_ff_shared=1 << 22)])
def test_widths_past_the_range_checked_loads_are_unsupported(kw):
    """A GEMM tile's A rows are loaded through range-checked buffer loads
    (pad rows past an expert's last row come in as zeros), whose byte
    offsets must stay below 2^31: a width of 2^22 or more is refused on the
    host, before anything is enqueued (the fake pointers are never used)."""
    lib = moe.load_library()
    fake = ctypes.c_void_p(256)
    cfg = _cfg(num_tokens=1, num_experts=1, top_k=1, act=0, **kw)
    st = lib.moe_layer_fwd(ctypes.byref(cfg), fake, fake, None, 0, fake, fake, fake, fake, fake, fake, 1 << 62,
                           None)
    assert st == 2
    if "d_ff_shared" not in kw:
        st = lib.moe_expert_ffn(ctypes.byref(cfg), fake, fake, fake, fake, fake, fake, fake, 1 << 62, None)
        assert st == 2


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_backward_workspace_layout(name):
    """Rows of the backward's padded layout: each expert's block rounded up to
    32 rows, so at most 31 pad rows per expert; the shared expert's T rows
    rounded up to 32; every region 256-B aligned and inside the total."""
    w = W.WORKLOADS[name]
    cfg = moe.make_config(w)
    L = moe.layer_bwd_workspace(cfg)
    assert L["padded_rows"] == moe.max_rows(cfg) + 31 * w.E
    assert L["shared_rows"] == ((w.T + 31) // 32 * 32 if w.d_ff_shared else 0)
    n_up = 2 if w.act == W.SWIGLU else 1
    P, s = L["padded_rows"], w.elem_bytes
    sizes = {"xp": P * w.d * s, "dyp": P * w.d * s, "z": P * n_up * w.d_ff * s, "dh": P * w.d_ff * s,
             "dxp": P * w.d * s, "dlogits": w.T * w.E * 4, "dx_router": w.T * w.d * 4}
    regions = sorted((L[n], L[n] + b) for n, b in sizes.items())
    for (a0, a1), (b0, _) in zip(regions, regions[1:]):
        assert a1 <= b0
    assert all(L[n] % 256 == 0 for n in sizes) and regions[-1][1] <= L["total"]


def test_backward_argument_errors():
    lib = moe.load_library()
    cfg = _cfg()
    fake = ctypes.c_void_p(256)
    F = moe.layer_workspace(cfg)["total"]
    B = moe.layer_bwd_workspace(cfg)["total"]
    args = lambda fwd_bytes, ws_bytes, dx=fake: (ctypes.byref(cfg), fake, fake, fake, fake, None, None, fake,
                                                 fwd_bytes, fake, dx, fake, fake, fake, None, None, 1, fake,
                                                 ws_bytes, None)
    assert lib.moe_layer_bwd(*args(F - 1, B)) == 3      # forward workspace too small
    assert lib.moe_layer_bwd(*args(F, B - 1)) == 3      # backward workspace too small
    assert lib.moe_layer_bwd(*args(F, B, dx=None)) == 1  # missing output
    sh = _cfg(d_ff_shared=64)
    assert lib.moe_layer_bwd(ctypes.byref(sh), fake, fake, fake, fake, None, None, fake, 1 << 30, fake, fake, fake,
                             fake, fake, None, None, 1, fake, 1 << 30, None) == 1  # shared expert without its weights


@pytest.mark.parametrize("cf", [0.3, 0.5, 1.0, 1.1, 1.2, 1.25, 1.6, 2.2, 3.7])
def test_capacity_agrees_with_oracle(cf):
    """moe_capacity and the oracle's capacity evaluate ceil(cf*T*k/E) the same
    way (cf travels as a double), including shapes where cf*T*k/E is an
    integer that a float32 factor would have pushed over (1.2 * 100 / 4)."""
    import oracle
    for T in (1, 7, 100, 256, 1000, 4096, 16384):
        for k in (1, 2, 6):
            for E in (4, 8, 10, 64, 128):
                if k > E:
                    continue
                cfg = _cfg(num_tokens=T, num_experts=E, top_k=k, capacity_factor=cf)
                assert moe.capacity(cfg) == oracle.capacity(cf, T, k, E), (cf, T, k, E)


def test_capacity_of_factors_float32_cannot_hold():
    """Factors whose float32 value sits above the decimal one: the capacity is
    still cf times the average load, rounded up (P3's capacity_factor)."""
    for cf, T, k, E, want in ((1.2, 100, 1, 4, 30), (1.1, 1000, 1, 4, 275), (0.3, 100, 1, 10, 3),
                              (1.25, 256, 2, 8, 80), (1.0, 16384, 1, 128, 128)):
        assert moe.capacity(_cfg(num_tokens=T, num_experts=E, top_k=k, capacity_factor=cf)) == want


@pytest.mark.parametrize("case", ["dtype", "contiguity", "size", "device"])
def test_binding_checks_tensors_before_the_call(case):
    """The binding rejects a tensor of the wrong element type, a strided view,
    a buffer too short for the configuration, or a host tensor, before it
    hands a pointer to the library (CPU tensors: no GPU is involved)."""
    import torch
    cfg = _cfg(num_tokens=16, d_model=64, num_experts=8, top_k=2, dtype=W.F32)
    T, E, d, k = 16, 8, 64, 2
    x = torch.zeros(T, d)
    wr = torch.zeros(E, d)
    logits = torch.zeros(T, E)
    idx = torch.zeros(T, k, dtype=torch.int32)
    tw = torch.zeros(T, k)
    if case == "dtype":
        bad = dict(x=x.to(torch.float64))
        err = TypeError
    elif case == "contiguity":
        bad = dict(x=torch.zeros(d, T).t())
        err = ValueError
    elif case == "size":
        bad = dict(x=torch.zeros(T - 1, d))
        err = ValueError
    else:
        bad = {}
        err = ValueError
    args = dict(x=x, w_router=wr, logits=logits, topk_idx=idx, topk_w=tw)
    args.update(bad)
    with pytest.raises(err):
        moe.route(cfg, args["x"], args["w_router"], args["logits"], args["topk_idx"], args["topk_w"],
                  stream=_NoStream())
    # the other entry points check their tensors the same way
    with pytest.raises(ValueError):
        moe.unpermute(cfg, torch.zeros(T * k, d), torch.zeros(T, k, dtype=torch.int32), torch.zeros(T, k),
                      torch.zeros(T - 1, d), stream=_NoStream())


class _NoStream:
    """Stands in for a stream: the checks fail before it is read."""
    @property
    def cuda_stream(self):
        raise AssertionError("the binding reached the library call")


def test_probe_arguments_are_checked_before_launch():
    """The measurement probes reject bad kinds, sizes, counts and alignments
    on the host (MOE_ERR_INVALID_ARG = 1), so nothing is launched; zero
    bytes is a no-op."""
    lib = moe.load_library()
    p16, p8 = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x100008)
    assert lib.moe_stream_probe(3, 0, p16, p16, 16, None, None) == 1        # no such kind
    assert lib.moe_stream_probe(2, 0, p16, p16, 24, None, None) == 1        # not a multiple of 16
    assert lib.moe_stream_probe(2, 0, p8, p16, 16, None, None) == 1         # misaligned source
    assert lib.moe_stream_probe(2, 0, None, p16, 16, None, None) == 1       # copy without a source
    assert lib.moe_stream_probe(0, 0, p16, None, 0, None, None) == 0        # nothing to read
    assert lib.moe_mfma_probe(0, 1, p16, None, None) == 1
    assert lib.moe_mfma_probe(1, 0, p16, None, None) == 1
    assert lib.moe_mfma_probe(1, 1, p8, None, None) == 1
    assert lib.moe_mfma_probe(1, 1, None, None, None) == 1


def test_probe_binding_checks_sizes():
    """The probe wrappers refuse buffers smaller than the bytes asked for
    before calling the library (CPU tensors: the checks come first)."""
    small = torch.empty(8, dtype=torch.uint8)
    with pytest.raises(ValueError):
        moe.stream_probe("copy", small, small, 16)
    with pytest.raises(ValueError):
        moe.stream_probe("write", None, small, 16)
    with pytest.raises(ValueError):
        moe.mfma_probe(2, 1, torch.empty(16384, dtype=torch.bfloat16))
