"""Python binding of the C ABI in include/moe.h.

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory and the current stream.
"""
from __future__ import annotations

import ctypes
from typing import Dict, NamedTuple, Optional

import torch

from . import _abi
from ._abi import Desc, Info, MoEError, Routing, Weights, check, lib
from .configs import LayerShape


class RoutingResult(NamedTuple):
    logits: torch.Tensor         # [T, E] fp32
    topk_idx: torch.Tensor       # [T, k] int32, best first
    topk_w: torch.Tensor         # [T, k] fp32
    expert_counts: torch.Tensor  # [E_loc] int32
    offsets: torch.Tensor        # [E_loc + 1] int32
    perm: torch.Tensor           # [R] int32 (token of each expert-contiguous row)
    slot_pos: torch.Tensor       # [T, k] int32 (-1: not local)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_desc(shape: LayerShape, mode: str = "dynamic", split: str = "cost_model",
              split_k: int = 0, max_workers: int = 0, fixed_mem_workers: int = 0,
              flags: int = 0, trace: Optional[torch.Tensor] = None,
              timeout_ms: int = 0, row_tile: int = 0, combine: str = "auto",
              timeout_ticks: int = 0, bands: int = 0, claim_batch: int = 0) -> Desc:
    d = Desc()
    d.T, d.d, d.E, d.k, d.f = shape.T, shape.d, shape.E, shape.k, shape.f
    d.e_begin, d.e_end = shape.e_begin, shape.local_end
    d.n_shared, d.f_shared = shape.n_shared, shape.f_shared
    d.dtype = _abi.MOE_F32 if shape.dtype == "fp32" else _abi.MOE_BF16
    d.mode = _abi.MODES[mode]
    d.split_policy = _abi.SPLITS[split]
    d.fixed_mem_workers = fixed_mem_workers
    d.split_k = split_k
    d.max_workers = max_workers
    d.flags = flags
    if trace is not None:
        assert trace.dtype == torch.int64 and trace.is_cuda and trace.is_contiguous()
        d.trace = trace.data_ptr()
        d.trace_cap = trace.numel() // 4
        d.flags |= _abi.FLAG_TRACE
    d.timeout_ms = timeout_ms
    d.row_tile = row_tile
    d.combine = _abi.COMBINES[combine]
    d.timeout_ticks = timeout_ticks
    d.bands = bands
    d.claim_batch = claim_batch
    return d


def workspace_size(desc: Desc) -> int:
    n = lib().moe_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise MoEError(1, "invalid descriptor")
    return int(n)


def query(desc: Desc) -> Dict[str, int]:
    info = Info()
    check(lib().moe_query(ctypes.byref(desc), ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in Info._fields_}


def _elem_dtype(shape: LayerShape):
    return torch.float32 if shape.dtype == "fp32" else torch.bfloat16


def _check_tensor(name, t, shape, dtype, device):
    if t is None:
        raise ValueError("%s is required" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous tensor on %s" % (name, device))


def alloc_routing(shape: LayerShape, device) -> RoutingResult:
    T, E, k, El = shape.T, shape.E, shape.k, shape.E_loc
    i32 = dict(dtype=torch.int32, device=device)
    return RoutingResult(
        logits=torch.empty((T, E), dtype=torch.float32, device=device),
        topk_idx=torch.empty((T, k), **i32),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
        expert_counts=torch.empty((El,), **i32),
        offsets=torch.empty((El + 1,), **i32),
        perm=torch.empty((max(1, T * k),), **i32),
        slot_pos=torch.empty((T, k), **i32))


def _routing_struct(r: Optional[RoutingResult]):
    if r is None:
        return None
    s = Routing()
    for name in RoutingResult._fields:
        setattr(s, name, getattr(r, name).data_ptr())
    return ctypes.byref(s)


class MoELayer:
    """One MoE layer bound to its weights and a workspace.

    weights: dict with w_router [d,E], router_bias [E] fp32 or None,
    w_gate/w_up [E_loc,d,f], w_down [E_loc,f,d], and ws_gate/ws_up
    [n_shared,d,fs], ws_down [n_shared,fs,d] when n_shared > 0.
    """

    def __init__(self, shape: LayerShape, weights: Dict[str, Optional[torch.Tensor]],
                 mode: str = "dynamic", split: str = "cost_model", split_k: int = 0,
                 max_workers: int = 0, fixed_mem_workers: int = 0, flags: int = 0,
                 trace: Optional[torch.Tensor] = None, timeout_ms: int = 0,
                 workspace: Optional[torch.Tensor] = None, row_tile: int = 0,
                 combine: str = "auto", timeout_ticks: int = 0, bands: int = 0,
                 claim_batch: int = 0,
                 no_alloc: bool = False):
        self.shape = shape
        dev = weights["w_gate"].device
        if dev.type != "cuda":
            raise ValueError("weights must be on a GPU")
        self.device = dev
        self.desc = make_desc(shape, mode, split, split_k, max_workers, fixed_mem_workers,
                              flags, trace, timeout_ms, row_tile, combine, timeout_ticks, bands,
                              claim_batch)
        self._trace = trace
        et = _elem_dtype(shape)
        d, E, f, El = shape.d, shape.E, shape.f, shape.E_loc
        _check_tensor("w_router", weights["w_router"], (d, E), et, dev)
        _check_tensor("w_gate", weights["w_gate"], (El, d, f), et, dev)
        _check_tensor("w_up", weights["w_up"], (El, d, f), et, dev)
        _check_tensor("w_down", weights["w_down"], (El, f, d), et, dev)
        if weights.get("router_bias") is not None:
            _check_tensor("router_bias", weights["router_bias"], (E,), torch.float32, dev)
        if shape.n_shared:
            fs, ns = shape.f_shared, shape.n_shared
            _check_tensor("ws_gate", weights["ws_gate"], (ns, d, fs), et, dev)
            _check_tensor("ws_up", weights["ws_up"], (ns, d, fs), et, dev)
            _check_tensor("ws_down", weights["ws_down"], (ns, fs, d), et, dev)
        self.weights = weights
        w = Weights()
        for name, _ in Weights._fields_:
            t = weights.get(name)
            setattr(w, name, None if t is None else t.data_ptr())
        self._w = w
        n = workspace_size(self.desc)
        # no_alloc: calls go through moe_layer_no_alloc, whose workspace is the
        # library's own static per-device scratch (no workspace tensor here)
        self.no_alloc = no_alloc
        if no_alloc:
            workspace = None
        elif workspace is None or workspace.numel() < n:
            workspace = torch.empty((n,), dtype=torch.uint8, device=dev)
        self.workspace = workspace

    @property
    def info(self) -> Dict[str, int]:
        with torch.cuda.device(self.device):
            return query(self.desc)

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                 routing: Optional[RoutingResult] = None, return_routing: bool = False,
                 check_errors: bool = False, residual: Optional[torch.Tensor] = None,
                 norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
                 y_norm: Optional[torch.Tensor] = None):
        """y = MoE(x); with norm_weight also the fused block tail:
        y = residual + MoE(x) and y_norm = RMSNorm(y) * norm_weight, returned
        as (y, y_norm[, routing])."""
        s = self.shape
        _check_tensor("x", x, (s.T, s.d), _elem_dtype(s), self.device)
        if y is None:
            y = torch.empty((s.T, s.d), dtype=torch.float32, device=self.device)
        _check_tensor("y", y, (s.T, s.d), torch.float32, self.device)
        if return_routing and routing is None:
            routing = alloc_routing(s, self.device)
        desc = self.desc
        if check_errors:
            desc = Desc.from_buffer_copy(self.desc)
            desc.flags |= _abi.FLAG_CHECK
        fused = norm_weight is not None
        if fused:
            _check_tensor("norm_weight", norm_weight, (s.d,), torch.float32, self.device)
            if residual is not None:
                _check_tensor("residual", residual, (s.T, s.d), torch.float32, self.device)
            if y_norm is None:
                y_norm = torch.empty((s.T, s.d), dtype=_elem_dtype(s), device=self.device)
            _check_tensor("y_norm", y_norm, (s.T, s.d), _elem_dtype(s), self.device)
        elif residual is not None:
            raise ValueError("residual is fused only together with norm_weight")
        if self.no_alloc and fused:
            raise ValueError("the fused tail has no no-allocation entry point")
        with torch.cuda.device(self.device):
            if self.no_alloc:
                rc = lib().moe_layer_no_alloc(ctypes.byref(desc), _ptr(x), ctypes.byref(self._w),
                                              _ptr(y), _routing_struct(routing),
                                              _stream(self.device))
            elif fused:
                rc = lib().moe_layer_norm(ctypes.byref(desc), _ptr(x), ctypes.byref(self._w),
                                          _ptr(residual), _ptr(norm_weight), float(norm_eps),
                                          _ptr(y), _ptr(y_norm), _routing_struct(routing),
                                          _ptr(self.workspace), self.workspace.numel(),
                                          _stream(self.device))
            else:
                rc = lib().moe_layer(ctypes.byref(desc), _ptr(x), ctypes.byref(self._w), _ptr(y),
                                     _routing_struct(routing), _ptr(self.workspace),
                                     self.workspace.numel(), _stream(self.device))
        check(rc)
        out = (y, y_norm) if fused else (y,)
        if routing is not None:
            out = out + (routing,)
        return out if len(out) > 1 else y

    def last_schedule(self) -> Dict[str, int]:
        """The scheduler's decisions in the last call (synchronises)."""
        out = _abi.Schedule()
        with torch.cuda.device(self.device):
            check(lib().moe_last_schedule(ctypes.byref(self.desc), _ptr(self.workspace),
                                          _stream(self.device), ctypes.byref(out)))
        return {name: getattr(out, name) for name, _ in _abi.Schedule._fields_}

    def device_error(self) -> int:
        with torch.cuda.device(self.device):
            return int(lib().moe_last_device_error(ctypes.byref(self.desc), _ptr(self.workspace),
                                                   _stream(self.device)))


class MoELayers:
    """Several independent MoE layers run by ONE call of moe_layers (one
    persistent launch when all are dynamic-mode layers of one element type).
    layers: MoELayer objects (their descriptors and weights are used; their
    own workspaces are not)."""

    def __init__(self, layers, workspace: Optional[torch.Tensor] = None):
        self.layers = list(layers)
        n = len(self.layers)
        self.device = self.layers[0].device
        self._descs = (Desc * n)(*[L.desc for L in self.layers])
        self._w = (Weights * n)(*[L._w for L in self.layers])
        size = int(lib().moe_layers_workspace_size(self._descs, n))
        if size == 0:
            raise MoEError(1, "invalid descriptors")
        if workspace is None or workspace.numel() < size:
            workspace = torch.empty((size,), dtype=torch.uint8, device=self.device)
        self.workspace = workspace

    def __call__(self, xs, ys=None, routings=None, check_errors: bool = False):
        n = len(self.layers)
        if ys is None:
            ys = [torch.empty((L.shape.T, L.shape.d), dtype=torch.float32, device=self.device)
                  for L in self.layers]
        for L, x, y in zip(self.layers, xs, ys):
            s = L.shape
            _check_tensor("x", x, (s.T, s.d), _elem_dtype(s), self.device)
            _check_tensor("y", y, (s.T, s.d), torch.float32, self.device)
        descs = self._descs
        if check_errors:
            descs = (Desc * n)(*[Desc.from_buffer_copy(L.desc) for L in self.layers])
            descs[0].flags |= _abi.FLAG_CHECK
        xp = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
        yp = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
        rt = None
        if routings is not None:
            arr = (Routing * n)()
            for i, r in enumerate(routings):
                for name in RoutingResult._fields:
                    setattr(arr[i], name, getattr(r, name).data_ptr())
            rt = arr
        with torch.cuda.device(self.device):
            check(lib().moe_layers(descs, n, xp, self._w, yp, rt, _ptr(self.workspace),
                                   self.workspace.numel(), _stream(self.device)))
        return ys


def route_from_logits(shape: LayerShape, logits: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None,
                      check_errors: bool = False) -> RoutingResult:
    """Routing tables from given fp32 logits [T,E] (same device code as the layer).
    check_errors: synchronise and raise on a device-detected error (e.g. a
    non-finite logit)."""
    dev = logits.device
    _check_tensor("logits", logits, (shape.T, shape.E), torch.float32, dev)
    desc = make_desc(shape, "multi_kernel", flags=_abi.FLAG_CHECK if check_errors else 0)
    n = workspace_size(desc)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty((n,), dtype=torch.uint8, device=dev)
    r = alloc_routing(shape, dev)
    with torch.cuda.device(dev):
        check(lib().moe_route_from_logits(ctypes.byref(desc), _ptr(logits), _routing_struct(r),
                                          _ptr(workspace), workspace.numel(), _stream(dev)))
    return r
