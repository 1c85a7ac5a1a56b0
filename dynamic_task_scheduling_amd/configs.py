"""The synthetic MoE-layer workloads this library is measured and checked on.

The Weave pages evaluate six unnamed MoE models under expert parallelism on
4x H100 (Weave abstract, arxivdaily.com/papers/2609.21483); no model, dataset
or trained weight is available here, so seeded synthetic layers of the shapes
below stand in for them.  Every layer is a top-k softmax-gated SwiGLU MoE.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional


@dataclasses.dataclass(frozen=True)
class LayerShape:
    T: int                 # tokens
    d: int                 # model dim
    E: int                 # router width (global experts)
    k: int                 # experts per token
    f: int                 # expert FFN dim
    dtype: str = "bf16"    # "bf16" or "fp32" for x, weights, Xp and H
    e_begin: int = 0       # local expert range [e_begin, e_end)
    e_end: Optional[int] = None
    n_shared: int = 0      # always-on experts, weight 1
    f_shared: int = 0
    zipf_s: Optional[float] = None   # router-bias skew exponent (None: no bias)
    zipf_scale: float = 1.0          # lambda in b_e = -lambda * s * ln(rank_e)

    @property
    def E_loc(self) -> int:
        return (self.e_end if self.e_end is not None else self.E) - self.e_begin

    @property
    def local_end(self) -> int:
        return self.e_end if self.e_end is not None else self.E


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    layers: List[LayerShape]
    seed_base: int = 0


def _tiny() -> Workload:
    return Workload("tiny_fp32",
                    "fp32 layer T=64 d=256 E=8 f=512 k=2, no router bias",
                    [LayerShape(T=64, d=256, E=8, k=2, f=512, dtype="fp32")])


def _decode() -> Workload:
    return Workload("decode_T128_d4096_E8_f14336_k2",
                    "decode-shaped bf16 layer, weight streaming, Zipf(1.2) router bias",
                    [LayerShape(T=128, d=4096, E=8, k=2, f=14336, zipf_s=1.2)])


def _prefill() -> Workload:
    return Workload("prefill_T4096_d2048_E64_f1408_k6_shared2",
                    "fine-grained prefill bf16 layer, 64 routed + 2 shared experts, Zipf(1.0)",
                    [LayerShape(T=4096, d=2048, E=64, k=6, f=1408, n_shared=2,
                                f_shared=1408, zipf_s=1.0, zipf_scale=0.5)])


def _ep_share() -> Workload:
    return Workload("epshare_T8192_d7168_E256loc128_f2048_k8",
                    "one GPU's share of a 2-way expert-parallel layer: 128 of 256 "
                    "experts local, only local hits kept, Zipf(1.5)",
                    [LayerShape(T=8192, d=7168, E=256, k=8, f=2048, e_begin=0,
                                e_end=128, zipf_s=1.5)])


def stress_draws(n_layers: int = 16, seed: int = 5):
    """Per-layer token count U{1..512} and Zipf exponent U[0.5, 2.0]."""
    import torch
    g = torch.Generator().manual_seed(seed)
    Ts = torch.randint(1, 513, (n_layers,), generator=g).tolist()
    ss = (0.5 + 1.5 * torch.rand(n_layers, generator=g, dtype=torch.float64)).tolist()
    return Ts, ss


def _stress() -> Workload:
    Ts, ss = stress_draws()
    layers = [LayerShape(T=t, d=4096, E=128, k=8, f=1536, zipf_s=s)
              for t, s in zip(Ts, ss)]
    return Workload("stress16_d4096_E128_f1536_k8",
                    "16 consecutive independent bf16 layers, T_l in U{1..512}, "
                    "Zipf exponent in U[0.5,2.0]", layers, seed_base=1000)


WORKLOADS = {
    1: _tiny,
    2: _decode,
    3: _prefill,
    4: _ep_share,
    5: _stress,
}


def workload(i: int) -> Workload:
    return WORKLOADS[i]()


def flops(s: LayerShape, R: int) -> float:
    """Algorithmic FLOPs: router GEMM + 3 expert GEMMs per kept row + shared."""
    return (2.0 * s.T * s.d * s.E + 6.0 * s.d * s.f * R +
            6.0 * s.d * s.f_shared * s.T * s.n_shared)


def algo_bytes(s: LayerShape, active_experts: int) -> float:
    """Algorithmic HBM bytes: weights of the active experts read once, the
    shared experts, the router weights, x read once, y (fp32) written once."""
    el = 4 if s.dtype == "fp32" else 2
    return (el * 3.0 * s.d * s.f * active_experts +
            el * 3.0 * s.d * s.f_shared * s.n_shared +
            el * s.d * s.E + el * s.T * s.d + 4.0 * s.T * s.d)
