"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Routing (top-k ids, counts, offsets, permutation, slot rows) must match bit
for bit given the same fp32 logits; y within the stated tolerances.  Every
scheduling mode runs the same tiles, so every mode is checked.
"""
import numpy as np
import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import oracle
from dynamic_task_scheduling_amd.configs import LayerShape, workload
from dynamic_task_scheduling_amd.moe import MoELayer, route_from_logits
from gpu_util import check_routing, compare_y, gen_inputs, host_inputs, run_and_check

MODES = [("dynamic", "cost_model"), ("dynamic", "none"), ("dynamic", "fixed"),
         ("static", "fixed"), ("multi_kernel", "none")]


@pytest.fixture(scope="module")
def tiny():
    wl = workload(1)
    s = wl.layers[0]
    g = gen_inputs(s, wl.name, 0)
    return s, g, host_inputs(g)


@pytest.mark.parametrize("mode,split", MODES)
def test_tiny_fp32_all_modes(tiny, mode, split):
    s, g, n = tiny
    run_and_check(s, g, n, mode, split, label="tiny_fp32")


MID = LayerShape(T=300, d=512, E=16, k=4, f=384, n_shared=1, f_shared=256, zipf_s=1.0)
MID_LOCAL = LayerShape(T=211, d=256, E=32, k=6, f=256, e_begin=8, e_end=24, zipf_s=1.5)


@pytest.fixture(scope="module")
def mid():
    g = gen_inputs(MID, "mid", 1)
    return g, host_inputs(g)


@pytest.mark.parametrize("mode,split", MODES)
def test_mid_bf16_all_modes(mid, mode, split):
    g, n = mid
    run_and_check(MID, g, n, mode, split, label="mid_bf16", combine="tasks")


# The scatter-add combine (automatic for layers with few routed rows) forced
# on the mid layer, with a shared expert and split-K DOWN slices.
@pytest.mark.parametrize("mode,split", MODES)
def test_mid_scatter_combine_all_modes(mid, mode, split):
    g, n = mid
    run_and_check(MID, g, n, mode, split, label="mid_scatter", combine="scatter")
    run_and_check(MID, g, n, mode, split, label="mid_scatter_sk3", combine="scatter", split_k=3)


def test_scatter_combine_trace_and_agreement(mid):
    from analysis_util import check_trace
    g, n = mid
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(MID, g, mode="dynamic", trace=trace, timeout_ms=3000, combine="scatter")
    assert layer.info["combine"] == 1
    y, r = layer(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)
    # the two combine paths agree up to fp32 summation order
    yt = MoELayer(MID, g, mode="dynamic", combine="tasks")(g["x"], check_errors=True)
    d = (y - yt).abs().max().item()
    assert d <= 1e-5 * yt.abs().max().item(), "scatter vs tasks differ by %g" % d


def test_auto_combine_choice():
    small = LayerShape(T=512, d=256, E=8, k=8, f=256)
    big = LayerShape(T=513, d=256, E=8, k=8, f=256)
    g = gen_inputs(small, "auto_c", 8)
    assert MoELayer(small, g).info["combine"] == 1     # T*k = 4096: scatter-add
    g2 = gen_inputs(big, "auto_c", 8)
    assert MoELayer(big, g2).info["combine"] == 2      # T*k = 4104: combine tasks


# 256-row expert tiles (chosen automatically for large bf16 layers), forced
# on a small layer whose hot experts span several tiles with ragged tails,
# with a shared expert and 256-column DOWN tasks.
BIG_TILE = LayerShape(T=1100, d=512, E=8, k=2, f=384, n_shared=1, f_shared=256, zipf_s=1.2)


@pytest.fixture(scope="module")
def big_tile():
    g = gen_inputs(BIG_TILE, "big_tile", 6)
    return g, host_inputs(g)


@pytest.mark.parametrize("mode,split", MODES)
def test_row_tile_256_all_modes(big_tile, mode, split):
    g, n = big_tile
    _, r, ro = run_and_check(BIG_TILE, g, n, mode, split, label="rt256", row_tile=256)
    c = ro["counts"]
    assert c.max() > 512 and (c % 256 != 0).all()


def test_row_tile_256_trace_and_modes_agree(big_tile):
    from analysis_util import check_trace
    g, n = big_tile
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(BIG_TILE, g, mode="dynamic", trace=trace, timeout_ms=3000, row_tile=256,
                     combine="tasks")
    assert layer.info["row_tile"] == 256 and layer.info["down_ntiles"] == BIG_TILE.d // 256
    y, r = layer(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)
    y2 = MoELayer(BIG_TILE, g, mode="static", split="fixed", row_tile=256,
                  combine="tasks")(g["x"], check_errors=True)
    assert torch.equal(y, y2)
    run_and_check(BIG_TILE, g, n, "dynamic", "cost_model", label="rt256_tasks", row_tile=256,
                  combine="tasks")


def test_row_tile_256_split_k_and_odd_d():
    # d = 384 is not a multiple of 256: 256-row tiles with 128-column DOWN tasks
    s = LayerShape(T=700, d=384, E=4, k=2, f=1024, zipf_s=0.5)
    g = gen_inputs(s, "rt256_odd", 7)
    for sk in (1, 3):
        run_and_check(s, g, None, "dynamic", "cost_model", split_k=sk, label="rt256sk%d" % sk,
                      row_tile=256)


@pytest.mark.parametrize("mode,split", [("dynamic", "cost_model"), ("static", "fixed"),
                                        ("multi_kernel", "none")])
def test_local_expert_range(mode, split):
    g = gen_inputs(MID_LOCAL, "mid_local", 2)
    for combine in ("scatter", "tasks"):
        y, r, ro = run_and_check(MID_LOCAL, g, None, mode, split, label="mid_local_" + combine,
                                 combine=combine)
        assert (ro["slot_pos"] < 0).any()


@pytest.mark.parametrize("combine", ["scatter", "tasks"])
def test_tokens_without_local_expert_are_zero(combine):
    """A narrow local range (8 of 32 experts, k = 2): many tokens have no
    local expert, and their rows of y are exactly zero (no shared experts)."""
    s = LayerShape(T=211, d=256, E=32, k=2, f=256, e_begin=24, e_end=32, zipf_s=1.5)
    g = gen_inputs(s, "narrow_local", 11)
    y, r, ro = run_and_check(s, g, None, "dynamic", "cost_model", label="narrow_" + combine,
                             combine=combine)
    none_local = np.all(ro["slot_pos"] < 0, axis=1)
    assert none_local.any() and not none_local.all()
    assert torch.all(y[torch.as_tensor(np.nonzero(none_local)[0], device=y.device)] == 0)


def test_empty_batch():
    """T = 0: nothing to route or compute; the call succeeds without a launch."""
    s = LayerShape(T=0, d=256, E=8, k=2, f=256)
    g = gen_inputs(LayerShape(T=4, d=256, E=8, k=2, f=256), "empty", 9)
    g["x"] = g["x"][:0].contiguous()
    y = MoELayer(s, g, mode="dynamic")(g["x"], check_errors=True)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


@pytest.mark.parametrize("combine", ["scatter", "tasks"])
def test_every_expert_and_max_shared(combine):
    """k = E (every expert takes every token) with the maximum of four shared
    experts."""
    s = LayerShape(T=150, d=256, E=8, k=8, f=256, n_shared=4, f_shared=128)
    g = gen_inputs(s, "k_eq_E", 10)
    _, r, ro = run_and_check(s, g, None, "dynamic", "cost_model", label="kE_" + combine,
                             combine=combine)
    assert np.all(ro["counts"] == s.T)


def test_nonfinite_logit_reported():
    """A NaN or infinite logit is a device-detected error (MOE_ERR_NONFINITE),
    raised when the caller asks for the check."""
    from dynamic_task_scheduling_amd._abi import MoEError
    s = LayerShape(T=40, d=128, E=16, k=4, f=128)
    for bad in (float("nan"), float("inf")):
        lg = torch.randn((s.T, s.E), generator=torch.Generator().manual_seed(3))
        lg[7, 5] = bad
        with pytest.raises(MoEError) as ei:
            route_from_logits(s, lg.cuda(), check_errors=True)
        assert ei.value.code == 7
    # a clean call afterwards succeeds (the error word is reset per call)
    route_from_logits(s, torch.randn((s.T, s.E)).cuda(), check_errors=True)


def test_router_256_wide_k_sliced():
    """The widest router (E = 256: two 128-column blocks of the router GEMM)
    with K slices reduced in a fixed order, logits compared with the
    oracle's, on a local expert range."""
    s = LayerShape(T=200, d=1024, E=256, k=8, f=256, e_begin=64, e_end=192, zipf_s=1.2)
    g = gen_inputs(s, "router256", 12)
    layer = MoELayer(s, g)
    assert layer.info["route_splits"] > 1
    for mode, split in (("dynamic", "cost_model"), ("static", "fixed"), ("multi_kernel", "none")):
        run_and_check(s, g, None, mode, split, label="router256")


ROUTER_GROUPS = {
    128: LayerShape(T=2200, d=512, E=128, k=4, f=128, zipf_s=1.2),
    256: LayerShape(T=2200, d=768, E=256, k=6, f=128, e_begin=32, e_end=160, zipf_s=1.2),
}


@pytest.mark.parametrize("E", [128, 256])
def test_router_groups(E):
    """Router tasks over 256-token groups (nine groups, the last one ragged)
    on the 256-row tile, their K slices summed per 32-token tile by finish
    tasks: logits and y against the oracle in every mode; in the dynamic
    kernel the trace shows each finish task after its group's K slices and
    every position task after the last finish; the 32-token router on the
    same inputs matches the oracle too."""
    from analysis_util import check_trace
    from dynamic_task_scheduling_amd import _abi
    s = ROUTER_GROUPS[E]
    g, n = gen_and_host(s, "router_groups%d" % E, 21)
    layer = MoELayer(s, g)
    assert layer.info["route_groups"] == 9 and layer.info["route_splits"] > 1
    for mode, split in (("dynamic", "cost_model"), ("static", "fixed"), ("multi_kernel", "none")):
        run_and_check(s, g, n, mode, split, label="router_groups%d" % E)
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(s, g, mode="dynamic", trace=trace, timeout_ms=3000)
    y, r = layer(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)
    assert MoELayer(s, g, flags=_abi.FLAG_NARROW_ROUTER).info["route_groups"] == 0
    run_and_check(s, g, n, "dynamic", "cost_model", label="router_narrow%d" % E,
                  flags=_abi.FLAG_NARROW_ROUTER)


def test_router_groups_ref_sync_and_one_launch():
    """Router groups in the static kernel with per-task counter waits, and
    in a multi-layer persistent launch beside a 32-token-router layer: y and
    the routing tables bit-identical to the layers' own dynamic calls
    (fixed-order combine), and within the bf16 tolerance of the oracle."""
    from dynamic_task_scheduling_amd import _abi
    from dynamic_task_scheduling_amd.moe import MoELayers, alloc_routing
    s = ROUTER_GROUPS[256]
    g, n = gen_and_host(s, "router_groups256", 21)
    run_and_check(s, g, n, "static", "fixed", flags=_abi.FLAG_REF_SYNC, label="groups_ref_sync")
    small = LayerShape(T=300, d=512, E=16, k=4, f=384, zipf_s=1.0)
    gs = gen_inputs(small, "groups_small", 22)
    shapes, inputs = [s, small, s], [g, gs, g]
    layers = [MoELayer(sh, gi, mode="dynamic", timeout_ms=3000, combine="tasks")
              for sh, gi in zip(shapes, inputs)]
    assert layers[0].info["route_groups"] == 9 and layers[1].info["route_groups"] == 0
    routs = [alloc_routing(sh, torch.device("cuda")) for sh in shapes]
    ys = MoELayers(layers)([gi["x"] for gi in inputs], routings=routs, check_errors=True)
    torch.cuda.synchronize()
    for sh, gi, L, y, r in zip(shapes, inputs, layers, ys, routs):
        y1, r1 = L(gi["x"], return_routing=True, check_errors=True)
        torch.cuda.synchronize()
        for f in ("topk_idx", "expert_counts", "offsets", "slot_pos"):
            assert torch.equal(getattr(r, f), getattr(r1, f))
        assert torch.equal(y, y1)
    ro = oracle.route(routs[0].logits.cpu().numpy(), s.k, s.e_begin, s.local_end)
    check_routing(routs[0], ro, s)
    yo = oracle.moe_layer(n["x"], n["w_gate"], n["w_up"], n["w_down"], ro, s.e_begin, None)
    compare_y(ys[0].cpu().numpy(), yo, "bf16")


def test_router_groups_scatter_and_fused_tail():
    """Router groups with the scatter-add combine forced (the group tasks
    start y rows from zero, or from the residual) and with the fused
    residual + RMSNorm tail, in the dynamic and static kernels."""
    s = ROUTER_GROUPS[128]
    g, n = gen_and_host(s, "router_groups128", 21)
    run_and_check(s, g, n, "dynamic", "cost_model", combine="scatter", label="groups_scatter")
    for mode, split in (("dynamic", "cost_model"), ("static", "fixed")):
        for combine in ("scatter", "tasks"):
            layer, *_ = check_fused_tail(s, g, n, mode, split, combine, label="groups")
            assert layer.info["route_groups"] == 9


def test_split_k_uneven():
    s = LayerShape(T=96, d=256, E=4, k=2, f=1024, zipf_s=0.5)
    g = gen_inputs(s, "splitk", 3)
    for sk in (3, 8):
        run_and_check(s, g, None, "dynamic", "cost_model", split_k=sk, label="splitk%d" % sk)


@pytest.mark.parametrize("T", [1, 33, 129])
def test_ragged_and_tiny_T(T):
    s = LayerShape(T=T, d=256, E=8, k=3, f=256, zipf_s=1.2)
    g = gen_inputs(s, "ragged", T)
    for mode, split in (("dynamic", "cost_model"), ("static", "fixed")):
        run_and_check(s, g, None, mode, split, label="T%d" % T)


def test_single_expert_k1():
    s = LayerShape(T=70, d=128, E=1, k=1, f=128)
    g = gen_inputs(s, "e1", 4)
    _, r, _ = run_and_check(s, g, None, "dynamic", "cost_model", label="E1k1")
    assert torch.all(r.topk_w == 1.0)


def test_all_tokens_one_expert():
    """A dominant bias sends every token to expert 5 first: one hot expert
    with many row tiles and several empty experts."""
    s = LayerShape(T=700, d=256, E=16, k=2, f=256)
    g = gen_inputs(s, "hot", 5)
    b = torch.zeros(16, dtype=torch.float32, device="cuda")
    b[5] = 50.0
    g["router_bias"] = b
    _, r, ro = run_and_check(s, g, None, "dynamic", "cost_model", label="hot_expert")
    assert int(ro["counts"][5]) == 700
    run_and_check(s, g, None, "dynamic", "cost_model", label="hot_expert_rt256", row_tile=256)


def test_few_workers():
    """Correct with 1, 2 and 3 persistent workers (no co-residency needed)."""
    g = gen_inputs(MID, "mid", 1)
    n = host_inputs(g)
    for w in (1, 2, 3):
        run_and_check(MID, g, n, "dynamic", "cost_model", max_workers=w, label="W%d" % w)


def test_route_from_logits_ties():
    """Identical logits in, identical tables out: random, heavy ties, signed
    zeros, and the 256-wide router."""
    rng = np.random.default_rng(0)
    cases = []
    for E, k in ((8, 2), (64, 6), (256, 8), (128, 8)):
        T = 257
        lg = rng.standard_normal((T, E)).astype(np.float32)
        cases.append((E, k, lg))
        lt = np.round(rng.standard_normal((T, E)) * 2).astype(np.float32)   # many ties
        lt[:, ::3] = 0.0
        lt[:, 1::7] = -0.0
        cases.append((E, k, lt))
    cases.append((16, 4, np.zeros((40, 16), np.float32)))
    for E, k, lg in cases:
        s = LayerShape(T=lg.shape[0], d=128, E=E, k=k, f=128)
        r = route_from_logits(s, torch.from_numpy(lg).cuda())
        torch.cuda.synchronize()
        ro = oracle.route(lg, k)
        check_routing(r, ro, s)
    # local range
    lg = rng.standard_normal((100, 32)).astype(np.float32)
    s = LayerShape(T=100, d=128, E=32, k=4, f=128, e_begin=4, e_end=20)
    r = route_from_logits(s, torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    check_routing(r, oracle.route(lg, 4, 4, 20), s)


def test_cross_mode_agreement(mid):
    g, n = mid
    ys = {}
    routes = {}
    for mode, split in MODES:
        layer = MoELayer(MID, g, mode=mode, split=split, timeout_ms=3000, combine="tasks")
        y, r = layer(g["x"], return_routing=True, check_errors=True)
        ys[(mode, split)] = y.clone()
        routes[(mode, split)] = r
    torch.cuda.synchronize()
    ref = ys[MODES[0]]
    for key in MODES[1:]:
        for f in ("topk_idx", "expert_counts", "offsets", "slot_pos"):
            assert torch.equal(getattr(routes[key], f), getattr(routes[MODES[0]], f))
        # same tiles, same fixed-order combine: bit-identical across modes
        assert torch.equal(ys[key], ref), "%s differs by %g" % (
            key, (ys[key] - ref).abs().max().item())


def test_repeat_and_poisoned_workspace(mid):
    """Repeated calls on one workspace, and a workspace filled with NaN-like
    bytes before a call, give the same y bit for bit (no read before write;
    the result does not depend on the schedule)."""
    g, n = mid
    layer = MoELayer(MID, g, mode="dynamic", timeout_ms=3000, combine="tasks")
    y0 = layer(g["x"], check_errors=True).clone()
    for _ in range(3):
        y1 = layer(g["x"], check_errors=True)
        assert torch.equal(y1, y0), "repeat call differs"
    layer.workspace.fill_(0xFF)
    y2 = layer(g["x"], check_errors=True)
    torch.cuda.synchronize()
    assert torch.isfinite(y2).all()
    assert torch.equal(y2, y0), "call on a poisoned workspace differs"


@pytest.mark.parametrize("combine", ["tasks", "scatter"])
@pytest.mark.parametrize("mode,split", [("dynamic", "cost_model"), ("dynamic", "none"),
                                        ("static", "fixed")])
def test_consecutive_calls_new_inputs(mode, split, combine):
    """One workspace, several calls with different token batches (so the
    routing, the gathered rows and the hidden rows all change): every call
    matches the oracle, so no call reads data left by an earlier one."""
    g = gen_inputs(MID, "mid", 1)
    n = host_inputs(g)
    layer = MoELayer(MID, g, mode=mode, split=split, timeout_ms=3000, combine=combine)
    for seed in (21, 22, 23):
        xs = torch.randn((MID.T, MID.d), generator=torch.Generator().manual_seed(seed))
        x = xs.to(torch.bfloat16).cuda()
        y, r = layer(x, return_routing=True, check_errors=True)
        torch.cuda.synchronize()
        nx = dict(n, x=x.cpu().view(torch.int16).numpy().view(np.uint16))
        ro = oracle.route(r.logits.cpu().numpy(), MID.k)
        check_routing(r, ro, MID)
        shared = (nx["ws_gate"], nx["ws_up"], nx["ws_down"])
        yo = oracle.moe_layer(nx["x"], nx["w_gate"], nx["w_up"], nx["w_down"], ro, 0, shared)
        compare_y(y.cpu().numpy(), yo, "bf16")


@pytest.mark.parametrize("explicit", [False, True])
@pytest.mark.parametrize("split", ["cost_model", "none"])
def test_xcd_affinity(big_tile, split, explicit):
    """Per-XCD UP queues (filled all at once after the positions with the
    fused gather, per row tile by its last permute task otherwise): same
    results bit for bit, every task once, every task after its producers."""
    from analysis_util import check_trace
    from dynamic_task_scheduling_amd import _abi
    g, n = big_tile
    fl = _abi.FLAG_XCD_AFFINITY | (_abi.FLAG_EXPLICIT_PERMUTE if explicit else 0)
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(BIG_TILE, g, mode="dynamic", split=split, trace=trace, timeout_ms=3000,
                     row_tile=256, combine="tasks", flags=fl)
    y, r = layer(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)
    y2 = MoELayer(BIG_TILE, g, mode="dynamic", row_tile=256, combine="tasks")(g["x"], check_errors=True)
    assert torch.equal(y, y2)
    run_and_check(MID, *gen_and_host(MID, "mid", 1), "dynamic", split, label="mid_aff",
                  flags=fl)


@pytest.mark.parametrize("fifo", [False, True])
@pytest.mark.parametrize("bands", [1, 2, 4])
def test_queue_policy_and_bands(big_tile, fifo, bands):
    """One FIFO compute queue (default) or the continuation-priority queue,
    and 1, 2 or 4 token bands in the row-tile order: every task once, after
    its producers, and y bit-identical to the static kernel's (same tiles,
    same fixed-order combine), checked against the oracle once."""
    from analysis_util import check_trace
    from dynamic_task_scheduling_amd import _abi
    g, n = big_tile
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(BIG_TILE, g, mode="dynamic", trace=trace, timeout_ms=3000, row_tile=256,
                     combine="tasks", bands=bands,
                     flags=_abi.FLAG_FIFO if fifo else _abi.FLAG_CONT_PRIORITY)
    assert layer.info["bands"] == bands
    y, r = layer(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)
    y2 = MoELayer(BIG_TILE, g, mode="static", split="fixed", row_tile=256, combine="tasks",
                  bands=bands)(g["x"], check_errors=True)
    assert torch.equal(y, y2)
    if bands == 4 and not fifo:
        run_and_check(BIG_TILE, g, n, "dynamic", "cost_model", label="rt256_b4", row_tile=256,
                      combine="tasks")


@pytest.mark.parametrize("mode,split", MODES)
def test_explicit_permute_all_modes(mid, big_tile, mode, split):
    """The permute (dispatch) as separate memory-bound tasks writing Xp, the
    stage the pages schedule on memory workers (the default fuses the gather
    into the UP tiles' row loads): y bit-identical to the fused gather's
    (the same rows feed the same tiles, summed in the same order) and within
    tolerance of the oracle; with 256-row tiles the dynamic trace shows every
    UP tile after its row tile's permute tasks."""
    from analysis_util import check_trace
    from dynamic_task_scheduling_amd import _abi
    fl = _abi.FLAG_EXPLICIT_PERMUTE
    g, n = mid
    y_e = run_and_check(MID, g, n, mode, split, label="mid_explicit", combine="tasks", flags=fl)[0]
    fused = MoELayer(MID, g, mode=mode, split=split, timeout_ms=3000, combine="tasks")
    assert fused.info["gather_fused"] == 1
    assert torch.equal(y_e, fused(g["x"], check_errors=True))
    if mode == "dynamic":
        gb, _ = big_tile
        trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
        layer = MoELayer(BIG_TILE, gb, mode="dynamic", split=split, trace=trace, timeout_ms=3000,
                         row_tile=256, combine="tasks", flags=fl)
        assert layer.info["gather_fused"] == 0
        y, r = layer(gb["x"], return_routing=True, check_errors=True)
        torch.cuda.synchronize()
        tr = check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)
        assert int((tr["kind"] == 3).sum()) > 0, "no permute tasks ran"
        y2 = MoELayer(BIG_TILE, gb, mode="dynamic", row_tile=256, combine="tasks")(gb["x"])
        assert torch.equal(y, y2)


@pytest.mark.parametrize("local", [False, True])
@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_claim_batch_and_local_queues(big_tile, local, batch):
    """Batched claims (one atomic increment reserves `batch` compute-queue
    slots) and XCD-local continuation queues with a global fallback and
    stealing: every task once, after its producers, y bit-identical to the
    static kernel's (same tiles, fixed-order combine); the largest batch of
    each queue layout is also checked against the oracle, with the scatter
    combine and a local expert range."""
    from analysis_util import check_trace
    from dynamic_task_scheduling_amd import _abi
    g, n = big_tile
    fl = _abi.FLAG_LOCAL_QUEUES if local else 0
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(BIG_TILE, g, mode="dynamic", trace=trace, timeout_ms=3000, row_tile=256,
                     combine="tasks", claim_batch=batch, flags=fl)
    y, r = layer(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)
    y2 = MoELayer(BIG_TILE, g, mode="static", split="fixed", row_tile=256,
                  combine="tasks")(g["x"], check_errors=True)
    assert torch.equal(y, y2)
    if batch == 8:
        run_and_check(MID_LOCAL, *gen_and_host(MID_LOCAL, "mid_local", 2), "dynamic", "none",
                      label="batch8_local%d" % local, flags=fl, claim_batch=8)


@pytest.mark.parametrize("variant", ["fifo", "cont_priority", "local_queues", "xcd_affinity"])
def test_perturbed_schedule(big_tile, variant):
    """Race perturbation (random sleeps before every claim and dependency
    decrement, pushed bursts reversed) under each queue policy: the trace
    still shows every task once and after its producers, and y is
    bit-identical to the static kernel's (fixed-order combine); the scatter
    combine with a local expert range is checked against the oracle."""
    from analysis_util import check_trace
    from dynamic_task_scheduling_amd import _abi
    g, n = big_tile
    fl = _abi.FLAG_PERTURB | {"fifo": 0, "cont_priority": _abi.FLAG_CONT_PRIORITY,
                              "local_queues": _abi.FLAG_LOCAL_QUEUES,
                              "xcd_affinity": _abi.FLAG_XCD_AFFINITY}[variant]
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(BIG_TILE, g, mode="dynamic", trace=trace, timeout_ms=3000, row_tile=256,
                     combine="tasks", flags=fl)
    y, r = layer(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)
    y2 = MoELayer(BIG_TILE, g, mode="static", split="fixed", row_tile=256,
                  combine="tasks")(g["x"], check_errors=True)
    assert torch.equal(y, y2)
    run_and_check(MID_LOCAL, *gen_and_host(MID_LOCAL, "mid_local", 2), "dynamic", "fixed",
                  label="perturb_" + variant, flags=fl)


@pytest.mark.parametrize("combine", ["scatter", "tasks"])
def test_layers_in_one_launch(combine):
    """moe_layers: several independent layers of different shapes in one
    persistent launch; each layer's y bit-identical to its own moe_layer call
    with combine tasks (fixed-order combine; scatter-add: within fp32
    summation order), routing tables identical, and every layer within the
    bf16 tolerance of the oracle.  A T = 0 layer in the middle is skipped."""
    from dynamic_task_scheduling_amd.moe import MoELayers, alloc_routing
    shapes = [LayerShape(T=300, d=512, E=16, k=4, f=384, n_shared=1, f_shared=256, zipf_s=1.0),
              LayerShape(T=1, d=256, E=8, k=2, f=256),
              LayerShape(T=0, d=256, E=8, k=2, f=256),
              LayerShape(T=129, d=256, E=32, k=6, f=512, e_begin=8, e_end=24, zipf_s=1.5),
              LayerShape(T=77, d=512, E=16, k=4, f=384, zipf_s=0.5)]
    gs = []
    for i, s in enumerate(shapes):
        g = gen_inputs(LayerShape(T=max(s.T, 1), d=s.d, E=s.E, k=s.k, f=s.f, e_begin=s.e_begin,
                                  e_end=s.e_end, n_shared=s.n_shared, f_shared=s.f_shared,
                                  zipf_s=s.zipf_s), "layers", 60 + i)
        g["x"] = g["x"][:s.T].contiguous()
        gs.append(g)
    layers = [MoELayer(s, g, mode="dynamic", timeout_ms=3000, combine=combine)
              for s, g in zip(shapes, gs)]
    stack = MoELayers(layers)
    routs = [alloc_routing(s, torch.device("cuda")) for s in shapes]
    ys = stack([g["x"] for g in gs], routings=routs, check_errors=True)
    torch.cuda.synchronize()
    for s, g, L, y, r in zip(shapes, gs, layers, ys, routs):
        if s.T == 0:
            continue
        y1, r1 = L(g["x"], return_routing=True, check_errors=True)
        torch.cuda.synchronize()
        for f in ("topk_idx", "expert_counts", "offsets", "slot_pos"):
            assert torch.equal(getattr(r, f), getattr(r1, f))
        if combine == "tasks":
            assert torch.equal(y, y1)
        else:
            assert (y - y1).abs().max().item() <= 1e-5 * y1.abs().max().item()
        n = host_inputs(g)
        ro = oracle.route(r.logits.cpu().numpy(), s.k, s.e_begin, s.local_end)
        check_routing(r, ro, s)
        shared = (n["ws_gate"], n["ws_up"], n["ws_down"]) if s.n_shared else None
        yo = oracle.moe_layer(n["x"], n["w_gate"], n["w_up"], n["w_down"], ro, s.e_begin, shared)
        compare_y(y.cpu().numpy(), yo, "bf16")


def test_layers_in_one_launch_traced():
    """Each layer's own trace in a multi-layer launch: every task once, after
    its producers."""
    from analysis_util import check_trace
    from dynamic_task_scheduling_amd.moe import MoELayers, alloc_routing
    g, n = gen_and_host(MID, "mid", 1)
    g2, _ = gen_and_host(BIG_TILE, "big_tile", 6)
    traces = [torch.zeros(4 * 20000, dtype=torch.int64, device="cuda") for _ in range(2)]
    layers = [MoELayer(MID, g, mode="dynamic", trace=traces[0], timeout_ms=3000, combine="tasks"),
              MoELayer(BIG_TILE, g2, mode="dynamic", trace=traces[1], timeout_ms=3000, row_tile=256,
                       combine="tasks")]
    routs = [alloc_routing(MID, torch.device("cuda")), alloc_routing(BIG_TILE, torch.device("cuda"))]
    MoELayers(layers)([g["x"], g2["x"]], routings=routs, check_errors=True)
    torch.cuda.synchronize()
    for t, L, r in zip(traces, layers, routs):
        check_trace(t.cpu().numpy().reshape(-1, 4).view(np.uint64), L, r)


def gen_and_host(shape, tag, seed):
    g = gen_inputs(shape, tag, seed)
    return g, host_inputs(g)


@pytest.mark.parametrize("mode,split", [("dynamic", "cost_model"), ("static", "fixed")])
def test_watchdog_timeout_then_recovery(mid, mode, split):
    """A watchdog limit of two clock ticks (20 ns): the kernel's own bounded
    waits give up, every workgroup exits, the call reports MOE_ERR_TIMEOUT;
    the next call on the same workspace with the normal limit matches the
    oracle."""
    from dynamic_task_scheduling_amd._abi import MoEError
    g, n = mid
    bad = MoELayer(MID, g, mode=mode, split=split, timeout_ticks=2, combine="tasks")
    with pytest.raises(MoEError) as ei:
        bad(g["x"], check_errors=True)
    assert ei.value.code == 5
    torch.cuda.synchronize()
    good = MoELayer(MID, g, mode=mode, split=split, workspace=bad.workspace, combine="tasks")
    y, r = good(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    ro = oracle.route(r.logits.cpu().numpy(), MID.k)
    check_routing(r, ro, MID)
    yo = oracle.moe_layer(n["x"], n["w_gate"], n["w_up"], n["w_down"], ro, 0,
                          (n["ws_gate"], n["ws_up"], n["ws_down"]))
    compare_y(y.cpu().numpy(), yo, "bf16")


@pytest.mark.parametrize("mode", ["dynamic", "static", "multi_kernel"])
def test_graph_capture_replay_new_inputs(mid, mode):
    """moe_layer captured once in a HIP graph (fixed addresses: x, y, the
    routing tables and the workspace), then replayed with new x contents
    written into the same buffer; every replay matches the oracle, with
    eager calls of the same layer between the replays."""
    g, n = mid
    from dynamic_task_scheduling_amd.moe import alloc_routing
    split = {"dynamic": "cost_model", "static": "fixed", "multi_kernel": "none"}[mode]
    layer = MoELayer(MID, g, mode=mode, split=split, timeout_ms=3000, combine="tasks")
    x = g["x"].clone()
    y = torch.empty((MID.T, MID.d), dtype=torch.float32, device="cuda")
    rt = alloc_routing(MID, torch.device("cuda"))
    layer(x, y, rt)                      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(x, y, rt)
    torch.cuda.synchronize()
    shared = (n["ws_gate"], n["ws_up"], n["ws_down"])
    for seed in (31, 32, 33):
        xs = torch.randn((MID.T, MID.d), generator=torch.Generator().manual_seed(seed))
        x.copy_(xs.to(torch.bfloat16).cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert layer.device_error() == 0
        nx = x.cpu().view(torch.int16).numpy().view(np.uint16)
        ro = oracle.route(rt.logits.cpu().numpy(), MID.k)
        check_routing(rt, ro, MID)
        yo = oracle.moe_layer(nx, n["w_gate"], n["w_up"], n["w_down"], ro, 0, shared)
        compare_y(y.cpu().numpy(), yo, "bf16")
        # an eager call in between (different output buffer), same result
        y_e = layer(x, check_errors=True)
        torch.cuda.synchronize()
        assert torch.equal(y_e, y)


def _norm_inputs(shape, seed):
    rng = torch.Generator().manual_seed(seed)
    res = torch.randn((shape.T, shape.d), generator=rng)
    gamma = (1.0 + 0.5 * torch.randn(shape.d, generator=rng)).float()
    return res.cuda(), gamma.cuda()


def check_fused_tail(shape, g, n, mode, split, combine, eps=1e-6, label="", seed=41):
    """moe_layer_norm against the oracle: y = residual + MoE(x) and
    y_norm = RMSNorm(y) * gamma; y_norm also against the fp64 RMSNorm of the
    GPU's own y (only the bf16 rounding of y_norm may differ)."""
    from gpu_util import log
    res, gamma = _norm_inputs(shape, seed)
    layer = MoELayer(shape, g, mode=mode, split=split, timeout_ms=3000, combine=combine)
    y, yn, r = layer(g["x"], return_routing=True, check_errors=True, residual=res,
                     norm_weight=gamma, norm_eps=eps)
    torch.cuda.synchronize()
    ro = oracle.route(r.logits.cpu().numpy(), shape.k, shape.e_begin, shape.local_end)
    check_routing(r, ro, shape)
    shared = (n["ws_gate"], n["ws_up"], n["ws_down"]) if shape.n_shared else None
    y_moe = oracle.moe_layer(n["x"], n["w_gate"], n["w_up"], n["w_down"], ro, shape.e_begin, shared)
    g_np = gamma.cpu().numpy()
    h, hn = oracle.residual_rmsnorm(y_moe, res.cpu().numpy(), g_np, eps)
    compare_y(y.cpu().numpy(), h, "bf16")
    yn_np = yn.float().cpu().numpy().astype(np.float64)
    err, rel = compare_y(yn_np, hn, "bf16")
    _, hn_own = oracle.residual_rmsnorm(y.cpu().numpy().astype(np.float64), None, g_np, eps)
    bound = 2.0 ** -8 * np.abs(hn_own) + 1e-5 * np.abs(hn_own).max()
    assert np.all(np.abs(yn_np - hn_own) <= bound), "RMSNorm arithmetic"
    log("       fused tail %s %s/%s %s ok: y_norm max|err| %.2e rel %.2e" % (label, mode, split, combine,
                                                                            err, rel))
    return layer, y, yn, res, gamma


@pytest.mark.parametrize("combine", ["tasks", "scatter"])
@pytest.mark.parametrize("mode,split", MODES)
def test_fused_residual_rmsnorm(mid, mode, split, combine):
    g, n = mid
    layer, y, yn, res, gamma = check_fused_tail(MID, g, n, mode, split, combine, label="mid")
    if combine == "tasks":
        # fixed-order combine: the fused y is the plain layer's y plus the
        # residual, bit for bit
        y0 = MoELayer(MID, g, mode=mode, split=split, combine="tasks")(g["x"], check_errors=True)
        assert torch.equal(y, y0 + res)


def test_fused_tail_no_residual_and_local_range():
    """No residual (y_norm = RMSNorm(MoE(x))), a local expert range with
    tokens that have no local expert, fp32 layer."""
    s = LayerShape(T=150, d=256, E=16, k=4, f=256, e_begin=4, e_end=12, zipf_s=1.2, dtype="fp32")
    g = gen_inputs(s, "norm_local", 13)
    n = host_inputs(g)
    for combine in ("tasks", "scatter"):
        layer = MoELayer(s, g, mode="dynamic", timeout_ms=3000, combine=combine)
        gamma = torch.ones(s.d, dtype=torch.float32, device="cuda")
        y, yn, r = layer(g["x"], return_routing=True, check_errors=True, norm_weight=gamma,
                         norm_eps=1e-5)
        torch.cuda.synchronize()
        ro = oracle.route(r.logits.cpu().numpy(), s.k, s.e_begin, s.local_end)
        y_moe = oracle.moe_layer(n["x"], n["w_gate"], n["w_up"], n["w_down"], ro, s.e_begin)
        h, hn = oracle.residual_rmsnorm(y_moe, None, gamma.cpu().numpy(), 1e-5)
        compare_y(y.cpu().numpy(), h, "fp32")
        compare_y(yn.cpu().numpy(), hn, "fp32")


@pytest.mark.parametrize("combine", ["tasks", "scatter"])
def test_fused_tail_trace(mid, combine):
    """Every NORM task runs once, after every task that writes its rows."""
    from analysis_util import check_trace
    g, n = mid
    res, gamma = _norm_inputs(MID, 42)
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(MID, g, mode="dynamic", trace=trace, timeout_ms=3000, combine=combine)
    y, yn, r = layer(g["x"], return_routing=True, check_errors=True, residual=res, norm_weight=gamma)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r, fused_norm=True)


def test_trace_happens_before(mid):
    """Every task runs exactly once and starts after its producers ended."""
    from analysis_util import check_trace
    g, n = mid
    trace = torch.zeros(4 * 20000, dtype=torch.int64, device="cuda")
    layer = MoELayer(MID, g, mode="dynamic", trace=trace, timeout_ms=3000, combine="tasks")
    y, r = layer(g["x"], return_routing=True, check_errors=True)
    torch.cuda.synchronize()
    check_trace(trace.cpu().numpy().reshape(-1, 4).view(np.uint64), layer, r)


# ------------------------------------------------------------ full sizes
# Every token of every full-size workload, in all three scheduling modes,
# against one oracle run per layer (the oracle is a plain fp64 CPU loop:
# tens of seconds on the largest layer, hence the per-test time limits).
FULL_MODES = (("dynamic", "cost_model"), ("static", "fixed"), ("multi_kernel", "none"))


def _full(cfg, layers=None):
    from gpu_util import check_full_layer
    from dynamic_task_scheduling_amd.synth import make_layer
    wl = workload(cfg)
    for li in (range(len(wl.layers)) if layers is None else layers):
        s = wl.layers[li]
        t = make_layer(s, wl.name, li, 0, "cuda")
        n = host_inputs(t)
        check_full_layer(s, t, n, FULL_MODES, label="%s[%d]" % (wl.name, li))
        del t, n
        torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_full_decode():
    _full(2)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3])
def test_full_fused_tail(cfg):
    """The fused residual + RMSNorm tail at full size: decode (scatter-add
    combine) and prefill (combine tasks), all three modes."""
    from dynamic_task_scheduling_amd.synth import make_layer
    wl = workload(cfg)
    s = wl.layers[0]
    t = make_layer(s, wl.name, 0, 0, "cuda")
    n = host_inputs(t)
    for mode, split in FULL_MODES:
        check_fused_tail(s, t, n, mode, split, "auto", label=wl.name)


@pytest.mark.timeout(900)
def test_full_prefill():
    _full(3)


@pytest.mark.timeout(1200)
def test_full_ep_share():
    _full(4)


@pytest.mark.timeout(900)
def test_full_stress_layers():
    _full(5)
