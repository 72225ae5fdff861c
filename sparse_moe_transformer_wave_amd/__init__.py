"""MI355X (gfx950) Flint-style sparse MoE FFN layer: Python binding of libflint_moe.so.

The binding only marshals arguments: torch tensors supply device memory, the current
torch stream is passed as the HIP stream, and every step of the layer runs in the HIP
kernels behind the C ABI (include/flint_moe.h).  There is no fallback: if the native
library is missing, every call raises.

Entry points (same names as the C ABI, without the prefix):
  workspace_bytes(desc, T_max, fmt), workspace_init(ws), workspace(desc, T_max, fmt),
  workspace_status(ws) (error flags raised since the last status call, then cleared)
  route(desc, x, w_router, bias, topk_ids, topk_w, ws, logits=None, logits_in=False)
  permute(desc, topk_ids, counts, offsets, sorted_assign, assign_pos, ws)
  forward(desc, weights, x, topk_ids, topk_w, offsets, sorted_assign, assign_pos, y, ws)
  layer(desc, weights, x, w_router, bias, y, ws, routing=None)
  layer_noalloc(desc, weights, x, w_router, bias, y, routing=None) (no workspace argument)
  decode_chain(desc, layers, x, y, ws, ...)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflint_moe.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_FORMAT, ERR_HIP = range(7)
WFMT_BF16, WFMT_NVFP4, WFMT_INT4 = 0, 1, 2
ROUTE_LOGITS_IN = 1
CHAIN_RESIDUAL = 1
WS_WAIT_TIMEOUT = 1
# byte offsets of the workspace head's words (include/flint_moe.h)
HEAD_ERROR, HEAD_DIAG, HEAD_COUNTERS = 8, 16, 1024

EXPORTED = ("flint_moe_workspace_bytes", "flint_moe_workspace_init", "flint_moe_workspace_status",
            "flint_moe_status_string",
            "flint_moe_route", "flint_moe_permute", "flint_moe_forward", "flint_moe_layer",
            "flint_moe_decode_chain", "flint_moe_layer_noalloc")


class FlintError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: status %d (%s)" % (where, status, status_string(status)))


class Desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("renormalize", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in (
            "gate", "up", "down", "sh_gate", "sh_up", "sh_down",
            "gate_sf", "up_sf", "down_sf", "sh_gate_sf", "sh_up_sf", "sh_down_sf",
            "gate_ts", "up_ts", "down_ts", "sh_ts")]


class _LayerRef(ctypes.Structure):
    _fields_ = [("weights", _Weights), ("w_router", ctypes.c_void_p), ("logit_bias", ctypes.c_void_p)]


class _Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_assign", "assign_pos")]


_lib = None


def lib():
    """The loaded native library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libflint_moe.so is not built (run __graft_entry__.build()); "
                               "there is no non-HIP fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.flint_moe_workspace_bytes.argtypes = [vp, i64, ctypes.c_int32]
        L.flint_moe_workspace_bytes.restype = sz
        L.flint_moe_workspace_init.argtypes = [vp, sz, vp]
        L.flint_moe_workspace_init.restype = ctypes.c_int
        L.flint_moe_workspace_status.argtypes = [vp, sz, vp, vp]
        L.flint_moe_workspace_status.restype = ctypes.c_int
        L.flint_moe_status_string.argtypes = [ctypes.c_int]
        L.flint_moe_status_string.restype = ctypes.c_char_p
        L.flint_moe_route.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, sz, vp]
        L.flint_moe_permute.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.flint_moe_forward.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.flint_moe_layer.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.flint_moe_layer_noalloc.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp]
        L.flint_moe_decode_chain.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, vp, vp,
                                             vp, vp, vp, vp, sz, vp]
        for f in ("flint_moe_route", "flint_moe_permute", "flint_moe_forward", "flint_moe_layer",
                  "flint_moe_decode_chain", "flint_moe_layer_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().flint_moe_status_string(status).decode()


def desc(hidden, inter, n_experts=256, top_k=6, n_shared=1, renormalize=1) -> Desc:
    return Desc(hidden, inter, n_experts, top_k, n_shared, renormalize)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int, where: str):
    if rc != OK:
        raise FlintError(rc, where)


@dataclass
class Weights:
    """Expert weights (torch tensors or raw device pointers) in the layout of the C ABI."""
    format: int
    gate: object
    up: object
    down: object
    sh_gate: object = None
    sh_up: object = None
    sh_down: object = None
    gate_sf: object = None
    up_sf: object = None
    down_sf: object = None
    sh_gate_sf: object = None
    sh_up_sf: object = None
    sh_down_sf: object = None
    gate_ts: object = None
    up_ts: object = None
    down_ts: object = None
    sh_ts: object = None

    def c_struct(self) -> _Weights:
        w = _Weights()
        w.format = self.format
        for name, _ in _Weights._fields_[1:]:
            setattr(w, name, _ptr(getattr(self, name)))
        return w


def workspace_bytes(d: Desc, T_max: int, fmt: int = WFMT_BF16) -> int:
    return int(lib().flint_moe_workspace_bytes(ctypes.byref(d), T_max, fmt))


def workspace_init(ws, stream=None):
    """Zero the synchronisation words of a workspace tensor (once, before first use)."""
    _check(lib().flint_moe_workspace_init(_ptr(ws), _nbytes(ws), _stream(stream)),
           "flint_moe_workspace_init")


def workspace_status(ws, stream=None) -> int:
    """Error flags (WS_*) raised on this workspace since the last status call, then cleared.
    Queues the status kernel on the stream and waits for it (this helper synchronises)."""
    import torch
    out = torch.zeros(1, dtype=torch.int32, device=ws.device)
    _check(lib().flint_moe_workspace_status(_ptr(ws), _nbytes(ws), _ptr(out), _stream(stream)),
           "flint_moe_workspace_status")
    return int(out.item())


def workspace(d: Desc, T_max: int, fmt: int = WFMT_BF16):
    """Allocate (torch, on the current device) and initialise a workspace for T <= T_max."""
    import torch
    ws = torch.empty(max(workspace_bytes(d, T_max, fmt), 1024), dtype=torch.uint8, device="cuda")
    workspace_init(ws)
    return ws


def route(d: Desc, T: int, x, w_router, bias, topk_ids, topk_w, ws, logits=None,
          logits_in: bool = False, stream=None):
    rc = lib().flint_moe_route(ctypes.byref(d), T, _ptr(x), _ptr(w_router), _ptr(bias),
                               _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                               ROUTE_LOGITS_IN if logits_in else 0, _ptr(ws), _nbytes(ws),
                               _stream(stream))
    _check(rc, "flint_moe_route")


def permute(d: Desc, T: int, topk_ids, counts, offsets, sorted_assign, assign_pos, ws=None,
            stream=None):
    rc = lib().flint_moe_permute(ctypes.byref(d), T, _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                                 _ptr(sorted_assign), _ptr(assign_pos), _ptr(ws), _nbytes(ws),
                                 _stream(stream))
    _check(rc, "flint_moe_permute")


def forward(d: Desc, weights: Weights, T: int, x, topk_ids, topk_w, offsets, sorted_assign,
            assign_pos, y, ws, stream=None):
    w = weights.c_struct()
    rc = lib().flint_moe_forward(ctypes.byref(d), ctypes.byref(w), T, _ptr(x), _ptr(topk_ids),
                                 _ptr(topk_w), _ptr(offsets), _ptr(sorted_assign),
                                 _ptr(assign_pos), _ptr(y), _ptr(ws), _nbytes(ws),
                                 _stream(stream))
    _check(rc, "flint_moe_forward")


def layer(d: Desc, weights: Weights, T: int, x, w_router, bias, y, ws, routing: dict | None = None,
          stream=None):
    w = weights.c_struct()
    r = None
    if routing:
        r = _Routing(**{k: _ptr(v) for k, v in routing.items()})
    rc = lib().flint_moe_layer(ctypes.byref(d), ctypes.byref(w), T, _ptr(x), _ptr(w_router),
                               _ptr(bias), _ptr(y), None if r is None else ctypes.byref(r),
                               _ptr(ws), _nbytes(ws), _stream(stream))
    _check(rc, "flint_moe_layer")


def layer_noalloc(d: Desc, weights: Weights, T: int, x, w_router, bias, y, routing: dict | None = None,
                  stream=None):
    """flint_moe_layer_noalloc: the whole layer on the library's own per-GPU scratch array."""
    w = weights.c_struct()
    r = None
    if routing:
        r = _Routing(**{k: _ptr(v) for k, v in routing.items()})
    rc = lib().flint_moe_layer_noalloc(ctypes.byref(d), ctypes.byref(w), T, _ptr(x), _ptr(w_router),
                                       _ptr(bias), _ptr(y), None if r is None else ctypes.byref(r),
                                       _stream(stream))
    _check(rc, "flint_moe_layer_noalloc")


def layer_refs(layers):
    """ctypes array of flint_moe_layer_ref from (Weights, w_router, logit_bias) triples."""
    arr = (_LayerRef * max(len(layers), 1))()
    for i, (w, wr, bias) in enumerate(layers):
        arr[i].weights = w.c_struct()
        arr[i].w_router = _ptr(wr)
        arr[i].logit_bias = _ptr(bias)
    return arr


def decode_chain(d: Desc, layers, x, y, ws, topk_ids=None, topk_w=None, logits=None,
                 residual=False, stream=None):
    """T = x.numel() / hidden tokens through len(layers) layers (flint_moe_decode_chain);
    layers = list of (Weights, w_router, logit_bias); y: [L][T][H] bf16 (int16 tensor)."""
    refs = layer_refs(layers)
    T = x.numel() // d.hidden
    rc = lib().flint_moe_decode_chain(ctypes.byref(d), refs, len(layers),
                                      CHAIN_RESIDUAL if residual else 0, T, _ptr(x), _ptr(y),
                                      _ptr(topk_ids), _ptr(topk_w), _ptr(logits), _ptr(ws), _nbytes(ws),
                                      _stream(stream))
    _check(rc, "flint_moe_decode_chain")


def layer_ptr_args(d: Desc, weights: Weights, T: int, x, w_router, bias, y, ws_ptr: int,
                   ws_bytes: int, stream: int):
    """Pre-marshalled argument tuple for repeated flint_moe_layer calls (benchmark loops)."""
    w = weights.c_struct()
    return (ctypes.byref(d), ctypes.byref(w), T, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(y),
            None, ws_ptr, ws_bytes, stream), (d, w)
