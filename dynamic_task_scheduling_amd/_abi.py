"""ctypes mirror of include/moe.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

from .build import LIB

c_int, c_uint, c_void_p, c_size_t = ctypes.c_int, ctypes.c_uint, ctypes.c_void_p, ctypes.c_size_t

MOE_F32, MOE_BF16 = 0, 1
MODES = {"dynamic": 0, "static": 1, "multi_kernel": 2}
SPLITS = {"cost_model": 0, "fixed": 1, "none": 2}
COMBINES = {"auto": 0, "scatter": 1, "tasks": 2}
FLAG_CHECK, FLAG_TRACE, FLAG_PHASE_SYNC, FLAG_REF_SYNC, FLAG_NO_STEAL = 0x1, 0x2, 0x4, 0x8, 0x10
FLAG_XCD_AFFINITY = 0x20
FLAG_FIFO = 0x40
FLAG_CONT_PRIORITY = 0x80
FLAG_LOCAL_QUEUES = 0x100
FLAG_PERTURB = 0x200
FLAG_EXPLICIT_PERMUTE = 0x400
FLAG_NARROW_ROUTER = 0x800

ERRORS = {
    0: "MOE_OK", 1: "MOE_ERR_ARG", 2: "MOE_ERR_WORKSPACE", 3: "MOE_ERR_UNSUPPORTED",
    4: "MOE_ERR_HIP", 5: "MOE_ERR_TIMEOUT", 6: "MOE_ERR_CAPACITY", 7: "MOE_ERR_NONFINITE",
    8: "MOE_ERR_TOO_LARGE",
}
NO_ALLOC_SCRATCH_BYTES = 64 << 20

# Every function the header declares (checked by the CPU tests).
EXPORTS = ["moe_workspace_size", "moe_query", "moe_layer", "moe_layer_norm", "moe_layer_no_alloc",
           "moe_layers_workspace_size", "moe_layers",
           "moe_route_from_logits", "moe_last_device_error", "moe_last_schedule", "moe_strerror"]


class Desc(ctypes.Structure):
    _fields_ = [
        ("T", c_int), ("d", c_int), ("E", c_int), ("k", c_int), ("f", c_int),
        ("e_begin", c_int), ("e_end", c_int), ("n_shared", c_int), ("f_shared", c_int),
        ("dtype", c_int), ("mode", c_int), ("split_policy", c_int),
        ("fixed_mem_workers", c_int), ("split_k", c_int), ("max_workers", c_int),
        ("flags", c_uint), ("trace", c_void_p), ("trace_cap", c_int), ("timeout_ms", c_int),
        ("row_tile", c_int), ("combine", c_int), ("bands", c_int), ("timeout_ticks", c_int),
        ("claim_batch", c_int),
    ]


class Weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "w_router", "router_bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


class Routing(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "logits", "topk_idx", "topk_w", "expert_counts", "offsets", "perm", "slot_pos")]


class Info(ctypes.Structure):
    _fields_ = [("workers", c_int), ("cus", c_int), ("blocks_per_cu", c_int),
                ("route_tiles", c_int), ("up_ntiles", c_int), ("down_ntiles", c_int),
                ("split_k", c_int), ("permute_rows", c_int), ("max_mtiles", c_int),
                ("max_tasks", c_int), ("route_splits", c_int), ("combine_chunks", c_int), ("row_tile", c_int),
                ("combine", c_int),
                ("workspace_bytes", c_size_t),
                ("cost_mfma_flops_per_cu", ctypes.c_float),
                ("cost_gather_bytes_per_worker", ctypes.c_float),
                ("cost_hbm_bytes", ctypes.c_float), ("bands", c_int),
                ("gather_fused", c_int), ("route_groups", c_int)]


class Schedule(ctypes.Structure):
    _fields_ = [("mem_workers", c_int), ("row_tiles", c_int), ("permute_tasks", c_int),
                ("error", c_int)]


class MoEError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__("%s (%d)%s" % (ERRORS.get(code, "?"), code,
                                        (": " + what) if what else ""))


_lib = None


def lib():
    """Load libdts_moe.so; fail loudly if it was not built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError("libdts_moe.so is not built; run "
                              "`python -m dynamic_task_scheduling_amd.build` first")
        L = ctypes.CDLL(LIB)
        P = ctypes.POINTER
        L.moe_workspace_size.argtypes = [P(Desc)]
        L.moe_workspace_size.restype = c_size_t
        L.moe_query.argtypes = [P(Desc), P(Info)]
        L.moe_query.restype = c_int
        L.moe_layer.argtypes = [P(Desc), c_void_p, P(Weights), c_void_p, P(Routing),
                                c_void_p, c_size_t, c_void_p]
        L.moe_layer.restype = c_int
        L.moe_layer_norm.argtypes = [P(Desc), c_void_p, P(Weights), c_void_p, c_void_p,
                                     ctypes.c_float, c_void_p, c_void_p, P(Routing), c_void_p,
                                     c_size_t, c_void_p]
        L.moe_layer_norm.restype = c_int
        L.moe_layer_no_alloc.argtypes = [P(Desc), c_void_p, P(Weights), c_void_p, P(Routing),
                                         c_void_p]
        L.moe_layer_no_alloc.restype = c_int
        L.moe_layers_workspace_size.argtypes = [P(Desc), c_int]
        L.moe_layers_workspace_size.restype = c_size_t
        L.moe_layers.argtypes = [P(Desc), c_int, P(c_void_p), P(Weights), P(c_void_p), P(Routing),
                                 c_void_p, c_size_t, c_void_p]
        L.moe_layers.restype = c_int
        L.moe_route_from_logits.argtypes = [P(Desc), c_void_p, P(Routing), c_void_p,
                                            c_size_t, c_void_p]
        L.moe_route_from_logits.restype = c_int
        L.moe_last_device_error.argtypes = [P(Desc), c_void_p, c_void_p]
        L.moe_last_device_error.restype = c_int
        L.moe_last_schedule.argtypes = [P(Desc), c_void_p, c_void_p, P(Schedule)]
        L.moe_last_schedule.restype = c_int
        L.moe_strerror.argtypes = [c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def check(code: int):
    if code != 0:
        raise MoEError(code, strerror(code))
