#!/usr/bin/env python3
"""Benchmark: one MoE layer per step on one MI355X through the C ABI.

Default workload: the decode-shaped bf16 layer (T=128, d=4096, E=8,
f=14336, k=2, Zipf(1.2) router bias) -- weight streaming, HBM-bound.
`--config N` picks another workload (1 tiny fp32, 2 decode, 3 fine-grained
prefill, 4 one-GPU expert share, 5 sixteen-layer stress).

A step is one full layer (router, top-k, permute, expert GEMMs, combine) in
the dynamic persistent megakernel; inputs are resident in HBM before timing.
The static-partition megakernel and the multi-kernel baseline run the same
inputs for the reported gains.  Prints ONE JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (MFMA / vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer tokens/s + TFLOP/s (% bf16 MFMA peak) on 1 MI355X; vs static split"


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dynamic_task_scheduling_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload_name: str):
    """HBM traffic per launch from committed rocprofv3 counter runs, only if
    they were taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "megakernel_%s_traffic.json" % workload_name)
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("source_sha") != kernel_source_sha():
        return None
    return d.get("traffic_bytes_per_launch")


def cpu_baseline(wl, layers_host, budget_s=12.0):
    """Time the CPU oracle (as it stands) on a bounded token sample of layer 0."""
    import numpy as np
    import oracle
    s = wl.layers[0]
    n = layers_host[0]
    lg = n["logits"]
    t0 = time.perf_counter()
    ro = oracle.route(lg, s.k, s.e_begin, s.local_end)
    t_route = time.perf_counter() - t0
    shared = (n["ws_gate"], n["ws_up"], n["ws_down"]) if s.n_shared else None
    ntok = 1
    spent = 0.0
    done = 0
    rng = np.random.default_rng(0)
    order = rng.permutation(s.T)
    while done < s.T and spent < budget_s:
        toks = order[done:done + ntok]
        t0 = time.perf_counter()
        oracle.moe_rows(n["x"], n["w_gate"], n["w_up"], n["w_down"], ro, toks, s.e_begin, shared)
        dt = time.perf_counter() - t0
        spent += dt
        done += len(toks)
        per = dt / max(1, len(toks))
        ntok = int(max(1, min(s.T - done, (budget_s - spent) / max(per, 1e-6))))
    tok_s = done / (spent + t_route * done / s.T)
    return {"value": tok_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d tokens of layer 0 (full routing of all %d tokens + expert "
                      "SwiGLU rows of the sampled tokens), fp64 C oracle, %.1f s"
                      % (done, s.T, s.T, spent + t_route)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-baselines", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--split", default="cost_model")
    ap.add_argument("--combine", default="auto", choices=["auto", "scatter", "tasks"],
                    help="weighted combine: scatter-add in the DOWN epilogue, or combine tasks")
    ap.add_argument("--modes", default="dynamic,static,multi_kernel")
    ap.add_argument("--affinity", action="store_true",
                    help="dynamic mode: per-XCD ready queues for UP tasks")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup+steps of the first mode in --modes only (for rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from dynamic_task_scheduling_amd import _abi, analysis, configs
    from dynamic_task_scheduling_amd.moe import MoELayer
    from dynamic_task_scheduling_amd.synth import make_layer, to_numpy

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = configs.workload(args.config)
    tensors = [make_layer(s, wl.name, li, 0, dev) for li, s in enumerate(wl.layers)]
    torch.cuda.synchronize()

    def make_layers(mode, split, trace=None):
        fl = _abi.FLAG_XCD_AFFINITY if (args.affinity and mode == "dynamic") else 0
        return [MoELayer(s, t, mode=mode, split=split, trace=trace, combine=args.combine, flags=fl)
                for s, t in zip(wl.layers, tensors)]

    ys = [torch.empty((s.T, s.d), dtype=torch.float32, device=dev) for s in wl.layers]

    def timed(layers, steps, warmup):
        stream = torch.cuda.current_stream(dev)
        for _ in range(warmup):
            for L, t, y in zip(layers, tensors, ys):
                L(t["x"], y)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            for L, t, y in zip(layers, tensors, ys):
                L(t["x"], y)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return e0.elapsed_time(e1) / steps, wall

    modes = [m for m in args.modes.split(",") if m]
    if args.profile_only or args.no_baselines:
        modes = modes[:1]
    split_of = {m: (args.split if m == "dynamic" else ("fixed" if m == "static" else "none"))
                for m in modes}
    all_layers = {m: make_layers(m, split_of[m]) for m in modes}
    # One untimed pass over every mode first, so that no mode is timed on a
    # GPU still ramping its clocks (the first-timed mode would otherwise pay
    # for it); then each mode: W warm-up steps and exactly K timed steps.
    if not args.profile_only:
        for m in modes:
            timed(all_layers[m], 1, args.warmup)
    ms = {}
    for m in modes:
        ms[m], wall = timed(all_layers[m], args.steps, args.warmup)
        errs = [L.device_error() for L in all_layers[m]]
        if any(errs):
            print("device error in mode %s: %s" % (m, errs), file=sys.stderr)
            sys.exit(3)
    del all_layers
    torch.cuda.synchronize()

    # routing stats + algorithmic work (from one routed call)
    routed = []
    for s, t in zip(wl.layers, tensors):
        L = MoELayer(s, t, mode="dynamic")
        y, r = L(t["x"], return_routing=True)
        routed.append(r)
    torch.cuda.synchronize()
    tot_T = sum(s.T for s in wl.layers)
    flops = 0.0
    hbm = 0.0
    count_stats = []
    for s, r in zip(wl.layers, routed):
        c = r.expert_counts.cpu().numpy()
        R = int(c.sum())
        A = int((c > 0).sum())
        flops += configs.flops(s, R)
        hbm += configs.algo_bytes(s, A)
        count_stats.append({"R": R, "active": A, "max": int(c.max()), "median": float(np.median(c)),
                            "zero": int((c == 0).sum())})
    if args.profile_only:
        print(json.dumps({"profile_only": True, "ms_by_mode": ms}), flush=True)
        return
    t_dyn = ms["dynamic"] * 1e-3
    tflops = flops / t_dyn / 1e12
    gbs = hbm / t_dyn / 1e9
    is_bf16 = wl.layers[0].dtype == "bf16"
    peak_fl = PEAK_BF16_TFLOPS if is_bf16 else PEAK_FP32_TFLOPS
    ridge = peak_fl * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if flops / hbm < ridge else "mfma"

    # schedule statistics from one traced call of layer 0 (separate run)
    sched = {}
    if not args.profile_only:
        trace = torch.zeros(4 * 200000, dtype=torch.int64, device=dev)
        Lt = MoELayer(wl.layers[0], tensors[0], mode="dynamic", split=args.split, trace=trace,
                      combine=args.combine)
        Lt(tensors[0]["x"], ys[0])
        torch.cuda.synchronize()
        tr = analysis.decode_trace(trace.cpu().numpy())
        sched = analysis.schedule_stats(tr, Lt.info["workers"])
        sched["workers"] = Lt.info["workers"]
        del Lt, trace

    n_launch_layers = len(wl.layers)
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS}
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": peak_fl, "unit": "TFLOP/s",
                "frac": tflops / peak_fl}
    roof["traffic"] = load_traffic(wl.name) if n_launch_layers == 1 else None
    comb0 = MoELayer(wl.layers[0], tensors[0], mode="dynamic", combine=args.combine).info["combine"]
    roof["kernel"] = "k_dynamic<%s, %s> (+ control reset)" % (
        "bf16" if is_bf16 else "fp32", "true" if comb0 == 1 else "false")

    out = {
        "metric": METRIC,
        "value": tot_T / t_dyn,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms["dynamic"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if is_bf16 else "fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": len(wl.layers), "tokens_per_step": tot_T,
                   "T": wl.layers[0].T if len(wl.layers) == 1 else "per-layer",
                   "d": wl.layers[0].d, "E": wl.layers[0].E, "k": wl.layers[0].k,
                   "f": wl.layers[0].f, "split": args.split, "combine": args.combine},
        "tflops": tflops,
        "pct_mfma_peak": 100.0 * tflops / peak_fl,
        "hbm_gbs": gbs,
        "pct_hbm_peak": 100.0 * gbs / PEAK_HBM_GBS,
        "algo_flop": flops,
        "algo_bytes": hbm,
        "ms_by_mode": ms,
        "gain_vs_static": (ms["static"] / ms["dynamic"]) if "static" in ms else None,
        "gain_vs_multi_kernel": (ms["multi_kernel"] / ms["dynamic"]) if "multi_kernel" in ms else None,
        "counts": count_stats if len(count_stats) <= 2 else {
            "R_total": sum(c["R"] for c in count_stats),
            "active_min": min(c["active"] for c in count_stats),
            "active_max": max(c["active"] for c in count_stats)},
        "schedule": sched,
        "roofline": roof,
    }
    if not args.no_cpu and not args.profile_only:
        host = []
        s0, t0_ = wl.layers[0], tensors[0]
        n0 = {k: to_numpy(v) for k, v in t0_.items()}
        n0["logits"] = routed[0].logits.cpu().numpy()
        host.append(n0)
        out["cpu_baseline"] = cpu_baseline(wl, host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
