#!/usr/bin/env python3
"""Benchmark: one MoE layer per step on one MI355X through the C ABI.

Headline workload (default, the largest single-GPU configuration): one GPU's
share of a 2-way expert-parallel layer -- T=8192 tokens, d=7168, 128 of 256
experts local, f=2048, top-8, Zipf(1.5) router bias -- MFMA-bound.
`--config N` picks another workload (1 tiny fp32, 2 decode, 3 fine-grained
prefill, 4 one-GPU expert share, 5 sixteen-layer stress).

A step is one full layer (router, top-k, permute, expert GEMMs, combine) in
the dynamic persistent megakernel; inputs are resident in HBM before timing.
The static-partition megakernel and the multi-kernel baseline run the same
inputs for the reported gains; the other workloads and the scheduler
ablations follow under extra keys.  Prints ONE JSON line.

`--calibrate-copy MIB` instead runs a plain device copy of known size (the
reference for scaling the FETCH_SIZE / WRITE_SIZE hardware counters).
`--vendor-gemm` instead times the vendor BLAS on dense GEMMs with the FLOPs of
the workload's expert FFNs (a ceiling for comparison, not part of the layer).
"""
import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (MFMA / vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer tokens/s + TFLOP/s (% bf16 MFMA peak) on 1 MI355X; vs static split"
HEADLINE_CONFIG = 4


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(wl, n0, budget_s=12.0):
    """Time the CPU oracle (as it stands) on a bounded token sample of layer 0."""
    import numpy as np
    import oracle
    s = wl.layers[0]
    lg = n0["logits"]
    t0 = time.perf_counter()
    ro = oracle.route(lg, s.k, s.e_begin, s.local_end)
    t_route = time.perf_counter() - t0
    shared = (n0["ws_gate"], n0["ws_up"], n0["ws_down"]) if s.n_shared else None
    ntok = 1
    spent = 0.0
    done = 0
    rng = np.random.default_rng(0)
    order = rng.permutation(s.T)
    while done < s.T and spent < budget_s:
        toks = order[done:done + ntok]
        t0 = time.perf_counter()
        oracle.moe_rows(n0["x"], n0["w_gate"], n0["w_up"], n0["w_down"], ro, toks, s.e_begin,
                        shared)
        dt = time.perf_counter() - t0
        spent += dt
        done += len(toks)
        per = dt / max(1, len(toks))
        ntok = int(max(1, min(s.T - done, (budget_s - spent) / max(per, 1e-6))))
    tok_s = done / (spent + t_route * done / s.T)
    return {"value": tok_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": "%d of %d tokens of %s layer 0 (full routing of all %d tokens + expert "
                      "SwiGLU rows of the sampled tokens), fp64 C oracle, %.1f s"
                      % (done, s.T, wl.name, s.T, spent + t_route)}


def calibrate_copy(mib: int) -> None:
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": n, "reps": 3}), flush=True)


def vendor_gemm(R: int, d: int, f: int, steps: int = 10, warmup: int = 3) -> dict:
    """Dense bf16 GEMMs of the vendor BLAS (torch.matmul) with the FLOPs of one
    layer's expert FFNs over its R kept rows: [R, d] x [d, 2f], then
    [R, f] x [f, d].  A comparison point for the expert GEMMs at the clock the
    chip holds under MFMA load: no gather, no ragged row tiles, no routing or
    combine, operands of random values.  Never part of the layer's path."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    bf = torch.bfloat16
    a = torch.randn(R, d, dtype=bf, device="cuda", generator=g)
    w1 = torch.randn(d, 2 * f, dtype=bf, device="cuda", generator=g)
    h = torch.randn(R, f, dtype=bf, device="cuda", generator=g)
    w2 = torch.randn(f, d, dtype=bf, device="cuda", generator=g)
    out = {}
    for name, x, w in (("up", a, w1), ("down", h, w2)):
        for _ in range(warmup):
            x @ w
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            x @ w
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        fl = 2.0 * x.shape[0] * x.shape[1] * w.shape[1]
        out[name] = {"shape": [x.shape[0], x.shape[1], w.shape[1]], "ms": round(ms, 4),
                     "tflops": round(fl / ms / 1e9, 1)}
    ms = out["up"]["ms"] + out["down"]["ms"]
    fl = 6.0 * R * d * f
    out.update({"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                "pct_mfma_peak": round(100.0 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 1)})
    return out


class Runner:
    """Layers of one workload on the GPU, and the timing of a scheduling mode."""

    def __init__(self, cfg, dev, combine="auto", bands=0):
        import torch
        from dynamic_task_scheduling_amd import configs
        from dynamic_task_scheduling_amd.synth import make_layer
        self.torch = torch
        self.dev = dev
        self.wl = configs.workload(cfg)
        self.tensors = [make_layer(s, self.wl.name, li, 0, dev) for li, s in enumerate(self.wl.layers)]
        self.ys = [torch.empty((s.T, s.d), dtype=torch.float32, device=dev) for s in self.wl.layers]
        self.combine = combine
        self.bands = bands
        torch.cuda.synchronize()

    def layers(self, mode, split, flags=0, trace=None, bands=None, claim_batch=0):
        from dynamic_task_scheduling_amd.moe import MoELayer
        b = self.bands if bands is None else bands
        return [MoELayer(s, t, mode=mode, split=split, trace=trace, combine=self.combine, flags=flags,
                         bands=b, claim_batch=claim_batch)
                for s, t in zip(self.wl.layers, self.tensors)]

    def step(self, layers):
        for L, t, y in zip(layers, self.tensors, self.ys):
            L(t["x"], y)

    def timed(self, layers, steps, warmup):
        """W untimed steps, then exactly K timed steps between two
        synchronisations; events between steps give per-step times."""
        torch = self.torch
        stream = torch.cuda.current_stream(self.dev)
        for _ in range(warmup):
            self.step(layers)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            self.step(layers)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        errs = [L.device_error() for L in layers]
        if any(errs):
            raise RuntimeError("device error %s" % errs)
        return {"mean": ev[0].elapsed_time(ev[steps]) / steps, "median": statistics.median(per),
                "min": min(per)}

    def routed(self):
        """Routing stats and algorithmic work from one routed call per layer."""
        import numpy as np
        from dynamic_task_scheduling_amd import configs
        from dynamic_task_scheduling_amd.moe import MoELayer
        flops = hbm = 0.0
        stats, logits0, sched = [], None, []
        for li, (s, t) in enumerate(zip(self.wl.layers, self.tensors)):
            L = MoELayer(s, t, mode="dynamic", combine=self.combine)
            y, r = L(t["x"], return_routing=True)
            sched.append(L.last_schedule())
            c = r.expert_counts.cpu().numpy()
            R, A = int(c.sum()), int((c > 0).sum())
            flops += configs.flops(s, R)
            hbm += configs.algo_bytes(s, A)
            stats.append({"R": R, "active": A, "max": int(c.max()), "median": float(np.median(c)),
                          "zero": int((c == 0).sum())})
            if li == 0:
                logits0 = r.logits.cpu().numpy()
        return flops, hbm, stats, logits0, sched

    def trace(self, split="cost_model"):
        """Schedule statistics and the cost-model calibration from one traced
        call of layer 0 (a separate run: tracing perturbs timing slightly)."""
        from dynamic_task_scheduling_amd import analysis
        torch = self.torch
        trace = torch.zeros(4 * 400000, dtype=torch.int64, device=self.dev)
        s0 = self.wl.layers[0]
        L = self.layers("dynamic", split, trace=trace)[0]
        y, r = L(self.tensors[0]["x"], self.ys[0], return_routing=True)
        torch.cuda.synchronize()
        tr = analysis.decode_trace(trace.cpu().numpy())
        info = L.info
        st = analysis.schedule_stats(tr, info["workers"])
        st["workers"] = info["workers"]
        st["by_kind_us"] = {k: round(v["sum_us"], 1) for k, v in analysis.by_kind(tr).items()}
        cal = analysis.calibrate(tr, info, s0, r.expert_counts.cpu().numpy())
        return st, cal


def gains(ms):
    out = {}
    if "static" in ms:
        out["gain_vs_static"] = ms["static"]["mean"] / ms["dynamic"]["mean"]
    if "multi_kernel" in ms:
        out["gain_vs_multi_kernel"] = ms["multi_kernel"]["mean"] / ms["dynamic"]["mean"]
    return out


def roofline_of(flops, hbm, t_s, bf16):
    peak_fl = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    ridge = peak_fl * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / hbm < ridge:
        a = hbm / t_s / 1e9
        return {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": a / PEAK_HBM_GBS}
    a = flops / t_s / 1e12
    return {"bound": "mfma", "achieved": a, "peak": peak_fl, "unit": "TFLOP/s", "frac": a / peak_fl}


MODE_SPLIT = {"dynamic": "cost_model", "static": "fixed", "multi_kernel": "none"}


def measure_modes(run, steps, warmup, modes=("dynamic", "static", "multi_kernel"), split=None):
    layers = {m: run.layers(m, split if (split and m == "dynamic") else MODE_SPLIT[m]) for m in modes}
    # one untimed pass over every mode first, so that no mode is timed on a
    # GPU still ramping its clocks
    for m in modes:
        run.timed(layers[m], 1, warmup)
    ms = {m: run.timed(layers[m], steps, warmup) for m in modes}
    del layers
    return ms


def ablations(run, steps, warmup):
    """Scheduler ablations on one workload: the permute as separate tasks
    (the default fuses it into the UP tiles) under each split policy, compute
    workers stealing permute tasks, per-XCD UP queues, XCD-local continuation queues,
    batched claims, the continuation-priority queue, token bands, router
    tasks over 32-token tiles instead of 256-token groups, and the static
    baseline's synchronisation (grid barriers vs per-task counter waits)."""
    from dynamic_task_scheduling_amd import _abi
    D, S, M = "dynamic", "static", "multi_kernel"
    EP = _abi.FLAG_EXPLICIT_PERMUTE
    variants = [
        # name, mode, split, flags, bands, claim_batch
        ("dynamic/explicit_permute/split=cost_model", D, "cost_model", EP, None, 0),
        ("dynamic/explicit_permute/split=fixed", D, "fixed", EP, None, 0),
        ("dynamic/explicit_permute/split=none", D, "none", EP, None, 0),
        ("dynamic/explicit_permute/steal=0", D, "fixed", EP | _abi.FLAG_NO_STEAL, None, 0),
        ("dynamic/xcd_affinity", D, "cost_model", _abi.FLAG_XCD_AFFINITY, None, 0),
        ("dynamic/local_queues", D, "cost_model", _abi.FLAG_LOCAL_QUEUES, None, 0),
        ("dynamic/claim_batch=2", D, "cost_model", 0, None, 2),
        ("dynamic/claim_batch=4", D, "cost_model", 0, None, 4),
        ("dynamic/claim_batch=8", D, "cost_model", 0, None, 8),
        ("dynamic/local_queues/claim_batch=4", D, "cost_model", _abi.FLAG_LOCAL_QUEUES, None, 4),
        ("dynamic/cont_priority", D, "cost_model", _abi.FLAG_CONT_PRIORITY, None, 0),
        ("dynamic/bands=2", D, "cost_model", 0, 2, 0),
        ("dynamic/bands=4", D, "cost_model", 0, 4, 0),
        ("dynamic/router=32_token_tiles", D, "cost_model", _abi.FLAG_NARROW_ROUTER, None, 0),
        ("static/sync=phase_barrier", S, "fixed", 0, None, 0),
        ("static/sync=ref_count", S, "fixed", _abi.FLAG_REF_SYNC, None, 0),
        ("multi_kernel", M, "none", 0, None, 0),
    ]
    out = {}
    for name, mode, split, fl, bands, cb in variants:
        L = run.layers(mode, split, flags=fl, bands=bands, claim_batch=cb)
        run.timed(L, 1, warmup)
        out[name] = round(run.timed(L, steps, warmup)["mean"], 4)
        if mode == D:
            out[name + ":mem_workers"] = L[0].last_schedule()["mem_workers"]
        del L
    return out


def time_one_launch(run, steps, warmup):
    """Every layer of the workload in one moe_layers call (one persistent
    launch for dynamic-mode layers), timed like a step."""
    from dynamic_task_scheduling_amd.moe import MoELayers
    stack = MoELayers(run.layers("dynamic", "cost_model"))
    torch = run.torch

    xs = [t["x"] for t in run.tensors]
    for _ in range(warmup):
        stack(xs, run.ys)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        stack(xs, run.ys)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def summarize(run, ms, steps_note=None):
    flops, hbm, stats, _, sched = run.routed()
    t = ms["dynamic"]["mean"] * 1e-3
    bf16 = run.wl.layers[0].dtype == "bf16"
    roof = roofline_of(flops, hbm, t, bf16)
    tot_T = sum(s.T for s in run.wl.layers)
    out = {"ms": {m: round(v["mean"], 4) for m, v in ms.items()},
           "tokens_per_s": tot_T / t, "tflops": flops / t / 1e12, "hbm_gbs": hbm / t / 1e9,
           "roofline_bound": roof["bound"], "roofline_frac": roof["frac"],
           "mem_workers": [s["mem_workers"] for s in sched][:16]}
    out.update(gains(ms))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEADLINE_CONFIG)
    ap.add_argument("--no-baselines", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-ablations", action="store_true")
    ap.add_argument("--split", default="cost_model")
    ap.add_argument("--bands", type=int, default=0,
                    help="token bands of the row-tile order (0: automatic)")
    ap.add_argument("--combine", default="auto", choices=["auto", "scatter", "tasks"],
                    help="weighted combine: scatter-add in the DOWN epilogue, or combine tasks")
    ap.add_argument("--profile-only", action="store_true",
                    help="time only the dynamic mode (for rocprofv3 runs)")
    ap.add_argument("--mode", default="dynamic",
                    help="modes timed by --profile-only, comma-separated, in order")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time only the vendor BLAS on dense GEMMs of the layer's expert FLOPs and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch
    from dynamic_task_scheduling_amd.synth import to_numpy

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    run = Runner(args.config, dev, args.combine, args.bands)
    wl = run.wl

    if args.vendor_gemm:
        _, _, st, _, _ = run.routed()
        s0 = wl.layers[0]
        print(json.dumps({"vendor_gemm": True, "workload": wl.name,
                          "res": vendor_gemm(st[0]["R"], s0.d, s0.f, args.steps, args.warmup)}), flush=True)
        return

    if args.profile_only:
        res = {}
        for mode in args.mode.split(","):
            L = run.layers(mode, args.split if mode == "dynamic" else MODE_SPLIT[mode])
            res[mode] = run.timed(L, args.steps, args.warmup)
            del L
        print(json.dumps({"profile_only": True, "workload": wl.name, "ms": res}), flush=True)
        return

    modes = ("dynamic",) if args.no_baselines else ("dynamic", "static", "multi_kernel")
    ms = measure_modes(run, args.steps, args.warmup, modes, split=args.split)
    flops, hbm, count_stats, logits0, sched = run.routed()
    st, cal = run.trace(args.split)
    t_dyn = ms["dynamic"]["mean"] * 1e-3
    bf16 = wl.layers[0].dtype == "bf16"
    roof = roofline_of(flops, hbm, t_dyn, bf16)
    roof["traffic"] = load_traffic(wl.name) if len(wl.layers) == 1 else None
    roof["kernel"] = "k_dynamic<%s, %s> (+ control reset)" % (
        "bf16" if bf16 else "fp32", "true" if run.layers("dynamic", args.split)[0].info["combine"] == 1
        else "false")
    tot_T = sum(s.T for s in wl.layers)
    out = {
        "metric": METRIC,
        "value": tot_T / t_dyn,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms["dynamic"]["mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": len(wl.layers), "tokens_per_step": tot_T,
                   "T": wl.layers[0].T if len(wl.layers) == 1 else "per-layer",
                   "d": wl.layers[0].d, "E": wl.layers[0].E, "k": wl.layers[0].k,
                   "f": wl.layers[0].f, "local_experts": wl.layers[0].E_loc,
                   "split": args.split, "combine": args.combine},
        "tflops": flops / t_dyn / 1e12,
        "pct_mfma_peak": 100.0 * flops / t_dyn / 1e12 / (PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS),
        "hbm_gbs": hbm / t_dyn / 1e9,
        "pct_hbm_peak": 100.0 * hbm / t_dyn / 1e9 / PEAK_HBM_GBS,
        "algo_flop": flops,
        "algo_bytes": hbm,
        "ms_by_mode": {m: round(v["mean"], 4) for m, v in ms.items()},
        "ms_stats": {m: {k: round(x, 4) for k, x in v.items()} for m, v in ms.items()},
        "counts": count_stats if len(count_stats) <= 2 else {
            "R_total": sum(c["R"] for c in count_stats),
            "active_min": min(c["active"] for c in count_stats),
            "active_max": max(c["active"] for c in count_stats)},
        "mem_workers": [s["mem_workers"] for s in sched],
        "schedule": st,
        "cost_model_calibration": cal,
        "roofline": roof,
    }
    out.update(gains(ms))
    if bf16 and len(wl.layers) == 1 and not args.no_baselines:
        # context, outside the timed region: the vendor BLAS on dense GEMMs
        # of the same expert FLOPs on this GPU, and the layer against it
        vg = vendor_gemm(count_stats[0]["R"], wl.layers[0].d, wl.layers[0].f)
        vg["layer_tflops_over_vendor_gemm"] = round(out["tflops"] / vg["tflops"], 3)
        out["context_vendor_dense_gemm"] = vg
    if not args.no_ablations and not args.no_baselines:
        out["ablations"] = ablations(run, max(5, args.steps // 2), max(2, args.warmup // 2))
    n0 = None
    if not args.no_cpu:
        n0 = {k: to_numpy(v) for k, v in run.tensors[0].items()}
        n0["logits"] = logits0
    del run
    torch.cuda.empty_cache()
    if not args.no_others and not args.no_baselines:
        from dynamic_task_scheduling_amd import _abi
        others = {}
        for cfg in (2, 3, 5):
            if cfg == args.config:
                continue
            r2 = Runner(cfg, dev, args.combine)
            ms2 = measure_modes(r2, max(5, args.steps // 2), max(2, args.warmup // 2))
            others[r2.wl.name] = summarize(r2, ms2)
            if not args.no_ablations:
                # the spatial split on this workload: the cost model's choice
                # (Wm per layer above) against a fixed group and no split
                sp = {}
                for split in ("fixed", "none"):
                    L = r2.layers("dynamic", split, flags=_abi.FLAG_EXPLICIT_PERMUTE)
                    r2.timed(L, 1, 2)
                    sp[split] = round(r2.timed(L, max(5, args.steps // 2), 2)["mean"], 4)
                    del L
                L = r2.layers("dynamic", "cost_model", flags=_abi.FLAG_EXPLICIT_PERMUTE)
                r2.timed(L, 1, 2)
                sp["cost_model"] = round(r2.timed(L, max(5, args.steps // 2), 2)["mean"], 4)
                sp["mem_workers"] = L[0].last_schedule()["mem_workers"]
                del L
                sp["fused_gather"] = others[r2.wl.name]["ms"]["dynamic"]
                others[r2.wl.name]["explicit_permute_split_ablation_ms"] = sp
            if len(r2.wl.layers) > 1:
                # the multi-layer persistent kernel: all layers in one launch
                t1 = time_one_launch(r2, max(5, args.steps // 2), max(2, args.warmup // 2))
                others[r2.wl.name]["ms_one_launch"] = round(t1, 4)
                others[r2.wl.name]["gain_one_launch_vs_static"] = ms2["static"]["mean"] / t1
                others[r2.wl.name]["gain_one_launch_vs_multi_kernel"] = ms2["multi_kernel"]["mean"] / t1
            del r2
            torch.cuda.empty_cache()
        out["other_workloads"] = others
    if n0 is not None:
        out["cpu_baseline"] = cpu_baseline(wl, n0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
