"""Seeded synthetic inputs for one MoE layer.

This module only draws random numbers; it holds none of the layer's
arithmetic.  Both the GPU path (tests, bench) and the CPU oracle take their
inputs from here, so the two see identical bytes: a tensor drawn on the GPU
is copied to the host for the oracle, never re-drawn.

Recipe (per layer):
  x ~ N(0,1); W_r ~ N(0,1/d); W_gate, W_up ~ N(0,1/d); W_down ~ N(0,1/f);
  shared experts the same with f_shared.  bf16 layers round each fp32 draw
  to bf16 (round to nearest even).  The router bias, when present, is the
  log-pmf of a finite Zipf law over the E ranks:
  b_e = -lambda * s * ln(rank_e), rank a seeded permutation of 1..E,
  which skews expert popularity without an infinite-support draw (that is
  undefined for s <= 1).
Each tensor has its own generator, seeded from (workload, layer, tensor,
seed), so one layer or one tensor can be regenerated alone.
"""
from __future__ import annotations

import hashlib
import math
from typing import Dict, Optional

import torch

from .configs import LayerShape


def _seed(tag: str, layer: int, name: str, seed: int) -> int:
    h = hashlib.sha256(("%s|%d|%s|%d" % (tag, layer, name, seed)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def normal(shape, std: float, dtype: torch.dtype, device, seed: int,
           chunk_rows: int = 0) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 and cast to ``dtype``; drawn in chunks along
    dim 0 when ``chunk_rows`` is set so huge bf16 tensors never need a full
    fp32 copy."""
    g = _gen(device, seed)
    if chunk_rows <= 0 or shape[0] <= chunk_rows:
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        t.mul_(std)
        return t.to(dtype)
    out = torch.empty(shape, dtype=dtype, device=device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        t = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                        device=device, dtype=torch.float32)
        t.mul_(std)
        out[r0:r1].copy_(t)
        del t
    return out


def zipf_bias(E: int, s: float, scale: float, seed: int) -> torch.Tensor:
    """b_e = -scale * s * ln(rank_e) with a seeded rank permutation (fp32)."""
    g = _gen("cpu", seed)
    ranks = torch.randperm(E, generator=g) + 1
    return (-scale * s * torch.log(ranks.to(torch.float64))).to(torch.float32)


def make_layer(shape: LayerShape, tag: str, layer: int = 0, seed: int = 0,
               device="cpu", with_experts: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """All inputs of one layer as torch tensors on ``device``."""
    dt = torch.float32 if shape.dtype == "fp32" else torch.bfloat16
    T, d, E, f = shape.T, shape.d, shape.E, shape.f
    El = shape.E_loc
    S = lambda name: _seed(tag, layer, name, seed)  # noqa: E731
    big = 1 << 28   # elements; above this, draw experts one chunk at a time
    ck = lambda n: max(1, big // max(1, n)) if El * n > big else 0  # noqa: E731
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = normal((T, d), 1.0, dt, device, S("x"))
    out["w_router"] = normal((d, E), 1.0 / math.sqrt(d), dt, device, S("w_router"))
    out["router_bias"] = (None if shape.zipf_s is None else
                          zipf_bias(E, shape.zipf_s, shape.zipf_scale,
                                    S("router_bias")).to(device))
    if with_experts:
        out["w_gate"] = normal((El, d, f), 1.0 / math.sqrt(d), dt, device,
                               S("w_gate"), ck(d * f))
        out["w_up"] = normal((El, d, f), 1.0 / math.sqrt(d), dt, device,
                             S("w_up"), ck(d * f))
        out["w_down"] = normal((El, f, d), 1.0 / math.sqrt(f), dt, device,
                               S("w_down"), ck(d * f))
        if shape.n_shared:
            fs = shape.f_shared
            out["ws_gate"] = normal((shape.n_shared, d, fs), 1.0 / math.sqrt(d),
                                    dt, device, S("ws_gate"))
            out["ws_up"] = normal((shape.n_shared, d, fs), 1.0 / math.sqrt(d),
                                  dt, device, S("ws_up"))
            out["ws_down"] = normal((shape.n_shared, fs, d), 1.0 / math.sqrt(fs),
                                    dt, device, S("ws_down"))
        else:
            out["ws_gate"] = out["ws_up"] = out["ws_down"] = None
    return out


def to_numpy(t: Optional[torch.Tensor]):
    """Host numpy view for the oracle: fp32 as float32, bf16 as uint16 bits."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
