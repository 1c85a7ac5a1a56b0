"""MI355X (gfx950) Mixture-of-Experts megakernel with dynamic task scheduling.

The compute path is the HIP library ``libdts_moe.so`` (C ABI in
``include/moe.h``); this package holds its Python binding, the synthetic
workload definitions and the build step.  Importing the package does not load
the library; the first call does, and fails loudly if it is not built.
"""
from .configs import LayerShape, Workload, workload  # noqa: F401

__all__ = ["LayerShape", "Workload", "workload", "MoELayer", "route_from_logits"]


def __getattr__(name):
    if name in ("MoELayer", "route_from_logits", "RoutingResult", "make_desc", "query",
                "workspace_size", "alloc_routing"):
        from . import moe
        return getattr(moe, name)
    raise AttributeError(name)
