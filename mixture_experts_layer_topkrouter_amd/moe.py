"""Thin ctypes binding of ``libmoe_mi355x.so`` (the C ABI in ``include/moe.h``).

Argument marshalling only: every step of the forward and backward passes runs
in the HIP kernels behind the C ABI.  torch is used for device memory and streams; the
functions take torch tensors, pass their device pointers and torch's current
HIP stream, and raise :class:`MoeError` on a non-OK status.  There is no CPU
fallback: when the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import workloads as W

_HERE = os.path.dirname(os.path.abspath(__file__))
# a sanitizer build of the same sources (tests/test_sanitizers.py) is loaded
# in place of the in-tree one when MOE_HIP_LIB names it
LIB_PATH = os.environ.get("MOE_HIP_LIB") or os.path.join(_HERE, "libmoe_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

F32, BF16 = 0, 1
# moe_pack_which: the weight moe_pack_weights rearranges
PACK_W1, PACK_W2, PACK_SHARED_W1, PACK_SHARED_W2 = 0, 1, 2, 3
GELU, SWIGLU = 0, 1
SOFTMAX_ALL, SOFTMAX_TOPK, EXPERT_CHOICE = 0, 1, 2

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_HIP", 5: "MOE_ERR_NOALLOC_LIMIT"}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("d_ff_shared", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
        ("ec_capacity", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("routing", ctypes.c_int32),
    ]


_LAYOUT_FIELDS = ["logits", "topk_idx", "topk_w", "scores", "ec_token", "ec_w", "x_perm", "row_token",
                  "slot_row", "slot_w", "tok_ptr", "expert_count", "expert_load", "expert_offset",
                  "shared_offset", "h", "y_perm", "shared_h", "shared_y", "scratch", "scratch_bytes",
                  "ffn_scratch", "ffn_scratch_bytes", "shared_ffn_scratch", "shared_ffn_scratch_bytes", "z",
                  "shared_z", "stamp", "total"]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _LAYOUT_FIELDS]


_BWD_LAYOUT_FIELDS = ["poff", "roff", "slot_prow", "prow_src", "d_slot_w", "dlogits", "dx_router", "router_offset", "router_part",
                      "xp", "dyp", "z",
                      "dh", "dxp", "shared_offset", "shared_roff", "xs", "dys", "zs", "dhs", "dxs", "scratch", "scratch_bytes",
                      "shared_scratch", "shared_scratch_bytes", "padded_rows", "shared_rows", "total"]


class BwdLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _BWD_LAYOUT_FIELDS]


_lib = None


def load_library() -> ctypes.CDLL:
    """Loads the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run `python -m mixture_experts_layer_topkrouter_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    CP = ctypes.POINTER(MoeConfig)
    i64 = ctypes.c_int64
    sz = ctypes.c_size_t
    sig = {
        "moe_abi_version": ([], ctypes.c_int32),
        "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "moe_max_rows": ([CP], i64),
        "moe_capacity": ([CP], i64),
        "moe_route": ([CP, P, P, P, i64, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_permute_scratch_bytes": ([CP, ctypes.POINTER(sz)], ctypes.c_int),
        "moe_permute": ([CP, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_permute_noalloc": ([CP, P, P, P, P, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_expert_ffn_workspace_bytes": ([CP, ctypes.POINTER(sz)], ctypes.c_int),
        "moe_expert_ffn": ([CP, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_unpermute": ([CP, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_layer_workspace": ([CP, ctypes.POINTER(WorkspaceLayout)], ctypes.c_int),
        "moe_layer_fwd": ([CP, P, P, P, i64, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_packed_weight_bytes": ([CP, ctypes.c_int32, ctypes.POINTER(sz)], ctypes.c_int),
        "moe_pack_weights": ([CP, ctypes.c_int32, P, P, P], ctypes.c_int),
        "moe_permute_packed": ([CP, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_expert_ffn_packed": ([CP, P, ctypes.c_int32, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_layer_fwd_packed": ([CP, P, P, P, i64, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_layer_bwd_workspace": ([CP, ctypes.POINTER(BwdLayout)], ctypes.c_int),
        "moe_layer_fwd_train": ([CP, P, P, P, i64, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_layer_bwd": ([CP, P, P, P, P, P, P, P, sz, P, P, P, P, P, P, P, ctypes.c_int32, P, sz, P], ctypes.c_int),
        "moe_stream_probe": ([ctypes.c_int32, ctypes.c_int32, P, P, sz, P, P], ctypes.c_int),
        "moe_mfma_probe": ([ctypes.c_int32, ctypes.c_int32, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def header_symbols() -> list:
    """Names of the functions declared in include/*.h."""
    import glob
    names = set()
    for path in sorted(glob.glob(os.path.join(os.path.dirname(HEADER_PATH), "*.h"))):
        with open(path) as f:
            text = f.read()
        names |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(moe_\w+)\s*\(", text, re.M))
    return sorted(names)


# ----------------------------------------------------------------- helpers --

def make_config(w: W.Workload) -> MoeConfig:
    return MoeConfig(w.T, w.d, w.E, w.k if w.routing != W.EXPERT_CHOICE else 0, w.d_ff, w.d_ff_shared,
                     float(w.cf), w.ec_capacity, w.dtype, w.act, w.routing)


def torch_dtype(cfg: MoeConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == F32 else torch.bfloat16


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _arg(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype], numel: int):
    """Device pointer of `t` after the checks the C ABI cannot make from a bare
    pointer: the element type (None: any, e.g. byte workspaces), a dense
    layout, at least `numel` elements, and a GPU tensor.  None passes NULL
    (the library decides whether that argument may be NULL)."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: holds {t.numel()} elements, needs at least {numel}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got device {t.device}")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


_I32, _F32 = torch.int32, torch.float32


def _dims(cfg: MoeConfig) -> dict:
    """Element counts of every buffer the entry points take, for this config."""
    T, E, d = cfg.num_tokens, cfg.num_experts, cfg.d_model
    ec = cfg.routing == EXPERT_CHOICE
    C = cfg.ec_capacity if ec else 0
    k = 0 if ec else cfg.top_k
    n_up = 2 if cfg.act == SWIGLU else 1
    rows = max(max_rows(cfg), 0)
    return {"T": T, "E": E, "d": d, "C": C, "k": k, "rows": rows, "slots": E * C if ec else T * k,
            "w1": E * n_up * cfg.d_ff * d, "w2": E * d * cfg.d_ff, "ws1": n_up * cfg.d_ff_shared * d,
            "ws2": d * cfg.d_ff_shared}


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise MoeError(status, where)


def max_rows(cfg: MoeConfig) -> int:
    return int(load_library().moe_max_rows(ctypes.byref(cfg)))


def capacity(cfg: MoeConfig) -> int:
    return int(load_library().moe_capacity(ctypes.byref(cfg)))


# --------------------------------------------------------- the entry points --

def route(cfg: MoeConfig, x: Optional[torch.Tensor], w_router: Optional[torch.Tensor], logits: torch.Tensor,
          topk_idx=None, topk_w=None, bias=None, bias_stride: int = 0, scores=None, ec_token=None, ec_w=None,
          stream=None):
    n, dt = _dims(cfg), torch_dtype(cfg)
    T, E = n["T"], n["E"]
    _check(load_library().moe_route(
        ctypes.byref(cfg), _arg(x, "x", dt, T * n["d"]), _arg(w_router, "w_router", dt, E * n["d"]),
        _arg(bias, "logit_bias", _F32, E if bias_stride == 0 else T * E), bias_stride,
        _arg(logits, "logits", _F32, T * E), _arg(topk_idx, "topk_idx", _I32, T * n["k"]),
        _arg(topk_w, "topk_w", _F32, T * n["k"]), _arg(scores, "scores", _F32, T * E),
        _arg(ec_token, "ec_token", _I32, E * n["C"]), _arg(ec_w, "ec_w", _F32, E * n["C"]), _stream(stream)),
        "moe_route")


def permute_scratch_bytes(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_permute_scratch_bytes(ctypes.byref(cfg), ctypes.byref(n)), "moe_permute_scratch_bytes")
    return int(n.value)


def permute(cfg: MoeConfig, x, x_perm, row_token, slot_row, expert_count, expert_load, expert_offset, *,
            topk_idx=None, ec_token=None, ec_w=None, slot_w=None, tok_ptr=None, scratch=None, stream=None,
            kblocked: bool = False):
    """moe_permute, or moe_permute_packed (x_perm written K-blocked,
    [d/32][rows][32]) when kblocked is set."""
    n, dt = _dims(cfg), torch_dtype(cfg)
    T, E, d, rows = n["T"], n["E"], n["d"], n["rows"]
    lib = load_library()
    fn = lib.moe_permute_packed if kblocked else lib.moe_permute
    _check(fn(
        ctypes.byref(cfg), _arg(x, "x", dt, T * d), _arg(topk_idx, "topk_idx", _I32, T * n["k"]),
        _arg(ec_token, "ec_token", _I32, E * n["C"]), _arg(ec_w, "ec_w", _F32, E * n["C"]),
        _arg(x_perm, "x_perm", dt, rows * d), _arg(row_token, "row_token", _I32, rows),
        _arg(slot_row, "slot_row", _I32, n["slots"]), _arg(slot_w, "slot_w", _F32, n["slots"]),
        _arg(tok_ptr, "tok_ptr", _I32, T + 1), _arg(expert_count, "expert_count", _I32, E),
        _arg(expert_load, "expert_load", _I32, E), _arg(expert_offset, "expert_offset", _I32, E + 1),
        _arg(scratch, "scratch", None, 0), _nbytes(scratch), _stream(stream)),
        "moe_permute_packed" if kblocked else "moe_permute")


def permute_noalloc(cfg: MoeConfig, x, x_perm, row_token, slot_row, expert_count, expert_load, expert_offset, *,
                    topk_idx=None, ec_token=None, ec_w=None, slot_w=None, tok_ptr=None, stream=None):
    """moe_permute_noalloc: moe_permute with its scratch in the library's
    static device array (nothing is allocated per call)."""
    n, dt = _dims(cfg), torch_dtype(cfg)
    T, E, d, rows = n["T"], n["E"], n["d"], n["rows"]
    _check(load_library().moe_permute_noalloc(
        ctypes.byref(cfg), _arg(x, "x", dt, T * d), _arg(topk_idx, "topk_idx", _I32, T * n["k"]),
        _arg(ec_token, "ec_token", _I32, E * n["C"]), _arg(ec_w, "ec_w", _F32, E * n["C"]),
        _arg(x_perm, "x_perm", dt, rows * d), _arg(row_token, "row_token", _I32, rows),
        _arg(slot_row, "slot_row", _I32, n["slots"]), _arg(slot_w, "slot_w", _F32, n["slots"]),
        _arg(tok_ptr, "tok_ptr", _I32, T + 1), _arg(expert_count, "expert_count", _I32, E),
        _arg(expert_load, "expert_load", _I32, E), _arg(expert_offset, "expert_offset", _I32, E + 1),
        _stream(stream)), "moe_permute_noalloc")


def expert_ffn_workspace_bytes(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_expert_ffn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "moe_expert_ffn_workspace_bytes")
    return int(n.value)


def alloc_ffn_workspace(cfg: MoeConfig, device="cuda") -> Optional[torch.Tensor]:
    n = expert_ffn_workspace_bytes(cfg)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def expert_ffn(cfg: MoeConfig, x_perm, expert_offset, w1, w2, h, y_perm, workspace=None, stream=None):
    """moe_expert_ffn.  `workspace` is a uint8 device tensor of
    expert_ffn_workspace_bytes(cfg) bytes (see alloc_ffn_workspace); None
    passes NULL, which the library rejects when the configuration needs one."""
    n, dt = _dims(cfg), torch_dtype(cfg)
    rows, d = n["rows"], n["d"]
    _check(load_library().moe_expert_ffn(
        ctypes.byref(cfg), _arg(x_perm, "x_perm", dt, rows * d), _arg(expert_offset, "expert_offset", _I32, n["E"] + 1),
        _arg(w1, "w1", dt, n["w1"]), _arg(w2, "w2", dt, n["w2"]), _arg(h, "h", dt, rows * cfg.d_ff),
        _arg(y_perm, "y_perm", dt, rows * d), _arg(workspace, "workspace", None, 0), _nbytes(workspace),
        _stream(stream)), "moe_expert_ffn")


_PACK_NAMES = {PACK_W1: "w1", PACK_W2: "w2", PACK_SHARED_W1: "ws1", PACK_SHARED_W2: "ws2"}


def packed_weight_bytes(cfg: MoeConfig, which: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_packed_weight_bytes(ctypes.byref(cfg), which, ctypes.byref(n)),
           "moe_packed_weight_bytes")
    return int(n.value)


def _packed_arg(cfg: MoeConfig, t, which: int):
    """A packed weight: a uint8 device tensor of packed_weight_bytes() bytes."""
    if t is None:
        return None
    return _arg(t, "packed " + _PACK_NAMES[which], torch.uint8, packed_weight_bytes(cfg, which))


def pack_weights(cfg: MoeConfig, which: int, w, packed=None, stream=None) -> torch.Tensor:
    """moe_pack_weights: rearranges weight `which` (PACK_W1, PACK_W2,
    PACK_SHARED_W1, PACK_SHARED_W2) into `packed` (a uint8 device tensor of
    packed_weight_bytes(cfg, which) bytes, allocated on w's device when
    None) and returns it."""
    if which not in _PACK_NAMES:
        raise ValueError(f"unknown packed weight {which}")
    nbytes = packed_weight_bytes(cfg, which)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    n = _dims(cfg)
    name = _PACK_NAMES[which]
    _check(load_library().moe_pack_weights(
        ctypes.byref(cfg), which, _arg(w, name, torch_dtype(cfg), n[name]), _packed_arg(cfg, packed, which),
        _stream(stream)), "moe_pack_weights")
    return packed


def expert_ffn_packed(cfg: MoeConfig, x_perm, expert_offset, w1_packed, w2_packed, h, y_perm, workspace=None,
                      stream=None, x_kblocked: bool = False):
    """moe_expert_ffn_packed: expert_ffn on weights packed by pack_weights;
    x_kblocked says x_perm is K-blocked (permute(kblocked=True)); h is
    written K-blocked."""
    n, dt = _dims(cfg), torch_dtype(cfg)
    rows, d = n["rows"], n["d"]
    _check(load_library().moe_expert_ffn_packed(
        ctypes.byref(cfg), _arg(x_perm, "x_perm", dt, rows * d), 1 if x_kblocked else 0,
        _arg(expert_offset, "expert_offset", _I32, n["E"] + 1),
        _packed_arg(cfg, w1_packed, PACK_W1), _packed_arg(cfg, w2_packed, PACK_W2), _arg(h, "h", dt, rows * cfg.d_ff),
        _arg(y_perm, "y_perm", dt, rows * d), _arg(workspace, "workspace", None, 0), _nbytes(workspace),
        _stream(stream)), "moe_expert_ffn_packed")


def unpermute(cfg: MoeConfig, y_perm, slot_row, slot_w, y, *, tok_ptr=None, y_shared=None, stream=None):
    n, dt = _dims(cfg), torch_dtype(cfg)
    T, d = n["T"], n["d"]
    _check(load_library().moe_unpermute(
        ctypes.byref(cfg), _arg(y_perm, "y_perm", dt, n["rows"] * d), _arg(tok_ptr, "tok_ptr", _I32, T + 1),
        _arg(slot_row, "slot_row", _I32, n["slots"]), _arg(slot_w, "slot_w", _F32, n["slots"]),
        _arg(y_shared, "y_shared", dt, T * d), _arg(y, "y", dt, T * d), _stream(stream)), "moe_unpermute")


def layer_workspace(cfg: MoeConfig) -> Dict[str, int]:
    L = WorkspaceLayout()
    _check(load_library().moe_layer_workspace(ctypes.byref(cfg), ctypes.byref(L)), "moe_layer_workspace")
    return {n: int(getattr(L, n)) for n in _LAYOUT_FIELDS}


def layer_fwd(cfg: MoeConfig, x, w_router, w1, w2, y, workspace, *, bias=None, bias_stride: int = 0, ws1=None,
              ws2=None, train: bool = False, stream=None):
    """moe_layer_fwd, or moe_layer_fwd_train (keeps the expert
    pre-activations for a backward without recompute) when train is set."""
    n, dt = _dims(cfg), torch_dtype(cfg)
    T, E, d = n["T"], n["E"], n["d"]
    lib = load_library()
    fn = lib.moe_layer_fwd_train if train else lib.moe_layer_fwd
    _check(fn(ctypes.byref(cfg), _arg(x, "x", dt, T * d), _arg(w_router, "w_router", dt, E * d),
              _arg(bias, "logit_bias", _F32, E if bias_stride == 0 else T * E), bias_stride,
              _arg(w1, "w1", dt, n["w1"]), _arg(w2, "w2", dt, n["w2"]), _arg(ws1, "ws1", dt, n["ws1"]),
              _arg(ws2, "ws2", dt, n["ws2"]), _arg(y, "y", dt, T * d), _arg(workspace, "workspace", None, 0),
              _nbytes(workspace), _stream(stream)), "moe_layer_fwd_train" if train else "moe_layer_fwd")


def layer_fwd_packed(cfg: MoeConfig, x, w_router, w1_packed, w2_packed, y, workspace, *, bias=None,
                     bias_stride: int = 0, ws1_packed=None, ws2_packed=None, stream=None):
    """moe_layer_fwd_packed: layer_fwd on expert weights packed by
    pack_weights (the router weights stay as they are)."""
    n, dt = _dims(cfg), torch_dtype(cfg)
    T, E, d = n["T"], n["E"], n["d"]
    _check(load_library().moe_layer_fwd_packed(
        ctypes.byref(cfg), _arg(x, "x", dt, T * d), _arg(w_router, "w_router", dt, E * d),
        _arg(bias, "logit_bias", _F32, E if bias_stride == 0 else T * E), bias_stride,
        _packed_arg(cfg, w1_packed, PACK_W1), _packed_arg(cfg, w2_packed, PACK_W2),
        _packed_arg(cfg, ws1_packed, PACK_SHARED_W1), _packed_arg(cfg, ws2_packed, PACK_SHARED_W2),
        _arg(y, "y", dt, T * d), _arg(workspace, "workspace", None, 0), _nbytes(workspace), _stream(stream)),
        "moe_layer_fwd_packed")


def layer_bwd_workspace(cfg: MoeConfig) -> Dict[str, int]:
    L = BwdLayout()
    _check(load_library().moe_layer_bwd_workspace(ctypes.byref(cfg), ctypes.byref(L)), "moe_layer_bwd_workspace")
    return {n: int(getattr(L, n)) for n in _BWD_LAYOUT_FIELDS}


def layer_bwd(cfg: MoeConfig, x, w_router, w1, w2, fwd_workspace, dy, dx, dw_router, dw1, dw2, workspace, *,
              ws1=None, ws2=None, dws1=None, dws2=None, recompute: bool = True, stream=None):
    n, dt = _dims(cfg), torch_dtype(cfg)
    T, E, d = n["T"], n["E"], n["d"]
    _check(load_library().moe_layer_bwd(
        ctypes.byref(cfg), _arg(x, "x", dt, T * d), _arg(w_router, "w_router", dt, E * d), _arg(w1, "w1", dt, n["w1"]),
        _arg(w2, "w2", dt, n["w2"]), _arg(ws1, "ws1", dt, n["ws1"]), _arg(ws2, "ws2", dt, n["ws2"]),
        _arg(fwd_workspace, "fwd_workspace", None, 0), _nbytes(fwd_workspace), _arg(dy, "dy", dt, T * d),
        _arg(dx, "dx", dt, T * d), _arg(dw_router, "dw_router", dt, E * d), _arg(dw1, "dw1", dt, n["w1"]),
        _arg(dw2, "dw2", dt, n["w2"]), _arg(dws1, "dws1", dt, n["ws1"]), _arg(dws2, "dws2", dt, n["ws2"]),
        int(bool(recompute)), _arg(workspace, "workspace", None, 0), _nbytes(workspace), _stream(stream)),
        "moe_layer_bwd")


def stream_probe(kind: str, src, dst, nbytes: int, nontemporal: bool = False, sink=None, stream=None):
    """moe_stream_probe: kind "read", "write" or "copy" over nbytes of
    contiguous device buffers (include/moe_probe.h)."""
    k = {"read": 0, "write": 1, "copy": 2}[kind]
    for t, name, used in ((src, "src", k != 1), (dst, "dst", k != 0)):
        if used and (t is None or t.numel() * t.element_size() < nbytes):
            raise ValueError(f"{name}: at least {nbytes} bytes needed")
    if sink is not None and sink.numel() * sink.element_size() < 4:
        raise ValueError("sink: one 32-bit word needed")
    _check(load_library().moe_stream_probe(k, int(bool(nontemporal)), _arg(src, "src", None, 0),
                                           _arg(dst, "dst", None, 0), nbytes, _arg(sink, "sink", None, 0),
                                           _stream(stream)), "moe_stream_probe")


def mfma_probe(blocks: int, iters: int, operands, sink=None, stream=None):
    """moe_mfma_probe: a register-only bf16 MFMA loop (include/moe_probe.h);
    operands: a bf16 device tensor of at least blocks * 16384 elements."""
    if operands.numel() * operands.element_size() < blocks * 32768:
        raise ValueError("operands: blocks * 32 KB needed")
    if sink is not None and (sink.dtype != torch.float32 or sink.numel() < blocks * 4):
        raise ValueError("sink: blocks * 4 float32 values needed")
    _check(load_library().moe_mfma_probe(int(blocks), int(iters), _arg(operands, "operands", None, 0),
                                         _arg(sink, "sink", None, 0), _stream(stream)), "moe_mfma_probe")


# ------------------------------------------------ allocation conveniences --

def alloc_workspace(cfg: MoeConfig, device="cuda") -> torch.Tensor:
    total = layer_workspace(cfg)["total"]
    return torch.empty(max(total, 256), dtype=torch.uint8, device=device)


def workspace_view(cfg: MoeConfig, ws: torch.Tensor, name: str, dtype: torch.dtype, shape) -> torch.Tensor:
    """A typed view of one intermediate inside moe_layer_fwd's workspace."""
    off = layer_workspace(cfg)[name]
    n = 1
    for s in shape:
        n *= int(s)

    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).view(*shape)


@dataclass
class DeviceInputs:
    x: torch.Tensor
    wr: torch.Tensor
    bias: Optional[torch.Tensor]
    bias_stride: int
    w1: torch.Tensor
    w2: torch.Tensor
    ws1: Optional[torch.Tensor]
    ws2: Optional[torch.Tensor]


def to_device(arr, device="cuda") -> Optional[torch.Tensor]:
    """numpy float32 -> fp32 tensor; numpy uint16 (bf16 bits) -> bf16 tensor."""
    import numpy as np
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


def upload(inp: dict, device="cuda") -> DeviceInputs:
    return DeviceInputs(to_device(inp["x"], device), to_device(inp["wr"], device), to_device(inp["bias"], device),
                        int(inp["bias_stride"]), to_device(inp["w1"], device), to_device(inp["w2"], device),
                        to_device(inp.get("ws1"), device), to_device(inp.get("ws2"), device))


def to_host_bits(t: torch.Tensor):
    """A device tensor back to numpy in the layout the oracle reads (bf16 ->
    uint16 bit patterns, fp32 -> float32)."""
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view("uint16")
    return t.detach().cpu().numpy()


class MoELayer:
    """One MoE block forward on the GPU through ``moe_layer_fwd``.

    Holds the device weights, one workspace and the output; ``forward()`` only
    enqueues the C-ABI call on the current stream.  ``view(name)`` exposes an
    intermediate (routing, permutation, expert outputs) inside the workspace.
    """

    def __init__(self, cfg: MoeConfig, dev: DeviceInputs, device="cuda"):
        self.cfg = cfg
        self.dev = dev
        self.layout = layer_workspace(cfg)
        self.workspace = torch.empty(max(self.layout["total"], 256), dtype=torch.uint8, device=device)
        self.y = torch.empty((cfg.num_tokens, cfg.d_model), dtype=torch_dtype(cfg), device=device)

    def pack(self, stream=None):
        """Packs the expert weights once (moe_pack_weights) for
        forward(packed=True); the unpacked weights stay for training."""
        c, d = self.cfg, self.dev
        self.w1p = pack_weights(c, PACK_W1, d.w1, stream=stream)
        self.w2p = pack_weights(c, PACK_W2, d.w2, stream=stream)
        self.ws1p = None if d.ws1 is None else pack_weights(c, PACK_SHARED_W1, d.ws1, stream=stream)
        self.ws2p = None if d.ws2 is None else pack_weights(c, PACK_SHARED_W2, d.ws2, stream=stream)

    def forward(self, stream=None, train: bool = False, packed: bool = False) -> torch.Tensor:
        """moe_layer_fwd (train=True: moe_layer_fwd_train, which keeps the
        expert pre-activations for backward(recompute=False); packed=True:
        moe_layer_fwd_packed on the weights pack() prepared)."""
        d = self.dev
        if packed:
            if train:
                raise ValueError("the training forward takes unpacked weights")
            if not hasattr(self, "w1p"):
                raise RuntimeError("forward(packed=True) needs pack() first")
            layer_fwd_packed(self.cfg, d.x, d.wr, self.w1p, self.w2p, self.y, self.workspace, bias=d.bias,
                             bias_stride=d.bias_stride, ws1_packed=self.ws1p, ws2_packed=self.ws2p, stream=stream)
            return self.y
        layer_fwd(self.cfg, d.x, d.wr, d.w1, d.w2, self.y, self.workspace, bias=d.bias, bias_stride=d.bias_stride,
                  ws1=d.ws1, ws2=d.ws2, train=train, stream=stream)
        return self.y

    def shapes(self) -> Dict[str, tuple]:
        c = self.cfg
        T, E, d = c.num_tokens, c.num_experts, c.d_model
        rows = max_rows(c)
        ec = c.routing == EXPERT_CHOICE
        k, C = c.top_k, c.ec_capacity
        dt = torch_dtype(c)
        i32, f32 = torch.int32, torch.float32
        s = {
            "logits": (f32, (T, E)),
            "x_perm": (dt, (rows, d)),
            "row_token": (i32, (rows,)),
            "expert_count": (i32, (E,)),
            "expert_load": (i32, (E,)),
            "expert_offset": (i32, (E + 1,)),
            "h": (dt, (rows, c.d_ff)),
            "y_perm": (dt, (rows, d)),
        }
        if ec:
            s.update({"scores": (f32, (E, T)), "ec_token": (i32, (E, C)), "ec_w": (f32, (E, C)),
                      "slot_row": (i32, (E * C,)), "slot_w": (f32, (E * C,)), "tok_ptr": (i32, (T + 1,))})
        else:
            s.update({"topk_idx": (i32, (T, k)), "topk_w": (f32, (T, k)), "slot_row": (i32, (T, k))})
        if c.d_ff_shared:
            s.update({"shared_y": (dt, (T, d)), "shared_h": (dt, (T, c.d_ff_shared))})
        return s

    def view(self, name: str) -> torch.Tensor:
        dtype, shape = self.shapes()[name]
        return workspace_view(self.cfg, self.workspace, name, dtype, shape)

    # ---- backward ----------------------------------------------------------
    def alloc_grads(self, device="cuda"):
        """Gradient buffers (dtype of the weights) and the backward workspace."""
        c, d = self.cfg, self.dev
        self.bwd_layout = layer_bwd_workspace(c)
        self.bwd_workspace = torch.empty(max(self.bwd_layout["total"], 256), dtype=torch.uint8, device=device)
        self.dx = torch.empty_like(d.x)
        self.dwr = torch.empty_like(d.wr)
        self.dw1 = torch.empty_like(d.w1)
        self.dw2 = torch.empty_like(d.w2)
        self.dws1 = None if d.ws1 is None else torch.empty_like(d.ws1)
        self.dws2 = None if d.ws2 is None else torch.empty_like(d.ws2)

    def backward(self, dy: torch.Tensor, recompute: bool = True, stream=None):
        """moe_layer_bwd for upstream gradient dy, after forward() on the same
        inputs (recompute=False needs forward(train=True)); fills self.dx,
        dwr, dw1, dw2 (and dws1, dws2)."""
        if not hasattr(self, "bwd_workspace"):
            self.alloc_grads(dy.device)
        d = self.dev
        layer_bwd(self.cfg, d.x, d.wr, d.w1, d.w2, self.workspace, dy, self.dx, self.dwr, self.dw1, self.dw2,
                  self.bwd_workspace, ws1=d.ws1, ws2=d.ws2, dws1=self.dws1, dws2=self.dws2, recompute=recompute,
                  stream=stream)

    def bwd_view(self, name: str) -> torch.Tensor:
        """A typed view of one intermediate of the backward workspace."""
        c = self.cfg
        T, E, d = c.num_tokens, c.num_experts, c.d_model
        L = self.bwd_layout
        P = L["padded_rows"]
        dt = torch_dtype(c)
        n_up = 2 if c.act == SWIGLU else 1
        slots = E * c.ec_capacity if c.routing == EXPERT_CHOICE else T * c.top_k
        shapes = {
            "poff": (torch.int32, (E + 1,)),
            "slot_prow": (torch.int32, (slots,)),
            "d_slot_w": (torch.float32, (slots,)),
            "dlogits": (torch.float32, (T, E)),
            "dx_router": (torch.float32, (T, d)),
            "xp": (dt, (P, d)),
            "dyp": (dt, (P, d)),
            "z": (dt, (P, n_up * c.d_ff)),
            "dh": (dt, (P, c.d_ff)),
            "dxp": (dt, (P, d)),
        }
        dtype, shape = shapes[name]
        off = L[name]
        n = 1
        for v in shape:
            n *= int(v)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.bwd_workspace[off:off + nbytes].view(dtype).view(*shape)
