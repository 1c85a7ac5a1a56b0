"""moe_layer_no_alloc (workspace = the library's static per-device scratch)
against moe_layer (caller's workspace): two calls in a row, the second with
a smaller layer, both matching bit for bit (same tiles, fixed-order combine)
and the oracle; a layer too large for the scratch is refused before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import oracle
from dynamic_task_scheduling_amd import _abi
from dynamic_task_scheduling_amd.configs import LayerShape
from dynamic_task_scheduling_amd.moe import MoELayer, make_desc, workspace_size
from gpu_util import check_routing, compare_y, gen_inputs, host_inputs, log


def _check(shape, tag, seed):
    g = gen_inputs(shape, tag, seed)
    n = host_inputs(g)
    ref = MoELayer(shape, g, mode="dynamic", timeout_ms=3000, combine="tasks")
    y_ref, r_ref = ref(g["x"], return_routing=True, check_errors=True)
    na = MoELayer(shape, g, mode="dynamic", timeout_ms=3000, combine="tasks", no_alloc=True)
    assert na.workspace is None
    y, r = na(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "no-alloc y differs from moe_layer's"
    for f in ("topk_idx", "expert_counts", "offsets", "slot_pos"):
        assert torch.equal(getattr(r, f), getattr(r_ref, f))
    ro = oracle.route(r.logits.cpu().numpy(), shape.k, shape.e_begin, shape.local_end)
    check_routing(r, ro, shape)
    shared = (n["ws_gate"], n["ws_up"], n["ws_down"]) if shape.n_shared else None
    yo = oracle.moe_layer(n["x"], n["w_gate"], n["w_up"], n["w_down"], ro, shape.e_begin, shared)
    err, rel = compare_y(y.cpu().numpy(), yo, shape.dtype)
    log("       no-alloc T=%d ok: max|err|/max|y|=%.2e rel-L2=%.2e" % (shape.T, err, rel))


def test_no_alloc_two_calls_second_smaller():
    big = LayerShape(T=300, d=512, E=16, k=4, f=384, n_shared=1, f_shared=256, zipf_s=1.0)
    small = LayerShape(T=77, d=512, E=16, k=4, f=384, n_shared=1, f_shared=256, zipf_s=1.0)
    for s in (big, small):
        assert workspace_size(make_desc(s)) <= _abi.NO_ALLOC_SCRATCH_BYTES
    _check(big, "noalloc", 51)
    _check(small, "noalloc", 52)


def test_no_alloc_refuses_too_large():
    s = LayerShape(T=4096, d=2048, E=64, k=6, f=1408)
    d = make_desc(s)
    assert workspace_size(d) > _abi.NO_ALLOC_SCRATCH_BYTES
    rc = _abi.lib().moe_layer_no_alloc(ctypes.byref(d), None, None, None, None, None)
    assert rc == 8 and "scratch" in _abi.strerror(rc)
