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
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

F32, BF16 = 0, 1
GELU, SWIGLU = 0, 1
SOFTMAX_ALL, SOFTMAX_TOPK, EXPERT_CHOICE = 0, 1, 2

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_HIP"}


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
        ("capacity_factor", ctypes.c_float),
        ("ec_capacity", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("routing", ctypes.c_int32),
    ]


_LAYOUT_FIELDS = ["logits", "topk_idx", "topk_w", "scores", "ec_token", "ec_w", "x_perm", "row_token",
                  "slot_row", "slot_w", "tok_ptr", "expert_count", "expert_load", "expert_offset",
                  "shared_offset", "h", "y_perm", "shared_h", "shared_y", "scratch", "scratch_bytes",
                  "ffn_scratch", "ffn_scratch_bytes", "shared_ffn_scratch", "shared_ffn_scratch_bytes", "z",
                  "shared_z", "total"]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _LAYOUT_FIELDS]


_BWD_LAYOUT_FIELDS = ["poff", "slot_prow", "prow_src", "d_slot_w", "dlogits", "dx_router", "router_offset", "router_part",
                      "xp", "dyp", "z",
                      "dh", "dxp", "shared_offset", "xs", "dys", "zs", "dhs", "dxs", "scratch", "scratch_bytes",
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
        "moe_expert_ffn_workspace_bytes": ([CP, ctypes.POINTER(sz)], ctypes.c_int),
        "moe_expert_ffn": ([CP, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_unpermute": ([CP, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_layer_workspace": ([CP, ctypes.POINTER(WorkspaceLayout)], ctypes.c_int),
        "moe_layer_fwd": ([CP, P, P, P, i64, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_layer_bwd_workspace": ([CP, ctypes.POINTER(BwdLayout)], ctypes.c_int),
        "moe_layer_fwd_train": ([CP, P, P, P, i64, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "moe_layer_bwd": ([CP, P, P, P, P, P, P, P, sz, P, P, P, P, P, P, P, ctypes.c_int32, P, sz, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def header_symbols() -> list:
    """Names of the functions declared in include/moe.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(moe_\w+)\s*\(", text, re.M)))


# ----------------------------------------------------------------- helpers --

def make_config(w: W.Workload) -> MoeConfig:
    return MoeConfig(w.T, w.d, w.E, w.k if w.routing != W.EXPERT_CHOICE else 0, w.d_ff, w.d_ff_shared,
                     float(w.cf), w.ec_capacity, w.dtype, w.act, w.routing)


def torch_dtype(cfg: MoeConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == F32 else torch.bfloat16


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


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
    _check(load_library().moe_route(ctypes.byref(cfg), _p(x), _p(w_router), _p(bias), bias_stride, _p(logits),
                                    _p(topk_idx), _p(topk_w), _p(scores), _p(ec_token), _p(ec_w),
                                    _stream(stream)), "moe_route")


def permute_scratch_bytes(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_permute_scratch_bytes(ctypes.byref(cfg), ctypes.byref(n)), "moe_permute_scratch_bytes")
    return int(n.value)


def permute(cfg: MoeConfig, x, x_perm, row_token, slot_row, expert_count, expert_load, expert_offset, *,
            topk_idx=None, ec_token=None, ec_w=None, slot_w=None, tok_ptr=None, scratch=None, stream=None):
    nbytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    _check(load_library().moe_permute(ctypes.byref(cfg), _p(x), _p(topk_idx), _p(ec_token), _p(ec_w), _p(x_perm),
                                      _p(row_token), _p(slot_row), _p(slot_w), _p(tok_ptr), _p(expert_count),
                                      _p(expert_load), _p(expert_offset), _p(scratch), nbytes, _stream(stream)),
           "moe_permute")


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
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().moe_expert_ffn(ctypes.byref(cfg), _p(x_perm), _p(expert_offset), _p(w1), _p(w2), _p(h),
                                         _p(y_perm), _p(workspace), nbytes, _stream(stream)), "moe_expert_ffn")


def unpermute(cfg: MoeConfig, y_perm, slot_row, slot_w, y, *, tok_ptr=None, y_shared=None, stream=None):
    _check(load_library().moe_unpermute(ctypes.byref(cfg), _p(y_perm), _p(tok_ptr), _p(slot_row), _p(slot_w),
                                        _p(y_shared), _p(y), _stream(stream)), "moe_unpermute")


def layer_workspace(cfg: MoeConfig) -> Dict[str, int]:
    L = WorkspaceLayout()
    _check(load_library().moe_layer_workspace(ctypes.byref(cfg), ctypes.byref(L)), "moe_layer_workspace")
    return {n: int(getattr(L, n)) for n in _LAYOUT_FIELDS}


def layer_fwd(cfg: MoeConfig, x, w_router, w1, w2, y, workspace, *, bias=None, bias_stride: int = 0, ws1=None,
              ws2=None, train: bool = False, stream=None):
    """moe_layer_fwd, or moe_layer_fwd_train (keeps the expert
    pre-activations for a backward without recompute) when train is set."""
    nbytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    fn = lib.moe_layer_fwd_train if train else lib.moe_layer_fwd
    _check(fn(ctypes.byref(cfg), _p(x), _p(w_router), _p(bias), bias_stride, _p(w1), _p(w2), _p(ws1), _p(ws2), _p(y),
              _p(workspace), nbytes, _stream(stream)), "moe_layer_fwd_train" if train else "moe_layer_fwd")


def layer_bwd_workspace(cfg: MoeConfig) -> Dict[str, int]:
    L = BwdLayout()
    _check(load_library().moe_layer_bwd_workspace(ctypes.byref(cfg), ctypes.byref(L)), "moe_layer_bwd_workspace")
    return {n: int(getattr(L, n)) for n in _BWD_LAYOUT_FIELDS}


def layer_bwd(cfg: MoeConfig, x, w_router, w1, w2, fwd_workspace, dy, dx, dw_router, dw1, dw2, workspace, *,
              ws1=None, ws2=None, dws1=None, dws2=None, recompute: bool = True, stream=None):
    fbytes = fwd_workspace.numel() * fwd_workspace.element_size()
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().moe_layer_bwd(ctypes.byref(cfg), _p(x), _p(w_router), _p(w1), _p(w2), _p(ws1), _p(ws2),
                                        _p(fwd_workspace), fbytes, _p(dy), _p(dx), _p(dw_router), _p(dw1), _p(dw2),
                                        _p(dws1), _p(dws2), int(bool(recompute)), _p(workspace), nbytes,
                                        _stream(stream)),
           "moe_layer_bwd")


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

    def forward(self, stream=None, train: bool = False) -> torch.Tensor:
        """moe_layer_fwd (train=True: moe_layer_fwd_train, which keeps the
        expert pre-activations for backward(recompute=False))."""
        d = self.dev
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
            s.update({"scores": (f32, (T, E)), "ec_token": (i32, (E, C)), "ec_w": (f32, (E, C)),
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
