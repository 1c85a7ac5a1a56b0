"""Host-side analysis of scheduling: task-trace decoding, tail idle time,
scheduling overhead, and the small formulas the Weave write-ups use to reason
about wave tails and speedups.
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np

KIND_SHIFT = 27
KINDS = {1: "ROUTE", 2: "POS", 3: "PERM", 4: "UP", 5: "DOWN", 6: "SUP", 7: "SDOWN",
         8: "PHASE", 9: "COMB", 10: "NORM", 11: "RFIN"}
# PHASE: scheduler phases (builder steps, router reduction); RFIN: the sum of
# a 256-token router group's K slices and the top-k of one 32-token tile
CLOCK_HZ = 100e6   # s_memrealtime rate


def wave_tail(slots: int, blocks: int) -> Dict[str, float]:
    """Hardware wave quantisation: `blocks` equal blocks on `slots` resident
    slots run in ceil(blocks/slots) waves; the last wave leaves
    slots*waves - blocks slots idle (xxqk.cn/news/665650 s1.1 and
    m.xxqk.cn/news/657744 s1.2 work this example)."""
    waves = -(-blocks // slots)
    last = blocks - (waves - 1) * slots
    idle = slots * waves - blocks
    return {"waves": waves, "last_wave_blocks": last, "idle_slots": idle,
            "efficiency": blocks / float(slots * waves)}


def amdahl(r: float, s: float) -> float:
    """End-to-end speedup when a fraction r of the time is sped up s-fold
    (xxqk.cn/news/665650 s3.4)."""
    return 1.0 / ((1.0 - r) + r / s)


def idle_bound(alpha: float) -> float:
    """Upper bound on the gain from filling an idle fraction alpha of SM time
    (xxqk.cn/news/665650 s4.1)."""
    return 1.0 / (1.0 - alpha)


def overlap_efficiency(t: float, a: float, b: float) -> float:
    """1 - (t - max(a,b)) / min(a,b): 1 when the shorter of two overlapped
    streams is fully hidden, 0 when they serialise (hncyxsy.com/news/277526,
    multi-stream overlap section)."""
    return 1.0 - (t - max(a, b)) / min(a, b)


def decode_trace(raw: np.ndarray) -> Dict[str, np.ndarray]:
    """Records of 4 uint64: claim requested, task start, task body end, meta
    (task id | worker << 32 | xcc << 48).  Unused (zero) records dropped."""
    raw = np.asarray(raw).view(np.uint64).reshape(-1, 4)
    used = raw[:, 2] != 0
    raw = raw[used]
    meta = raw[:, 3]
    task = (meta & np.uint64(0xffffffff)).astype(np.int64)
    return {
        "t_req": raw[:, 0].astype(np.int64),
        "t_start": raw[:, 1].astype(np.int64),
        "t_end": raw[:, 2].astype(np.int64),
        "task": task,
        "kind": task >> KIND_SHIFT,
        "payload": task & ((1 << KIND_SHIFT) - 1),
        "worker": ((meta >> np.uint64(32)) & np.uint64(0xffff)).astype(np.int64),
        "xcc": ((meta >> np.uint64(48)) & np.uint64(0xff)).astype(np.int64),
    }


def schedule_stats(tr: Dict[str, np.ndarray], workers: int) -> Dict[str, float]:
    """Busy, claim-wait and tail-idle shares of worker time over the kernel.

    Kernel span = first claim to last task end.  A worker is busy while it
    runs a task body; claim overhead is the time from asking for a task to
    starting it; tail idle is, per worker, the time from its last task end to
    the kernel end, summed over workers."""
    if tr["t_end"].size == 0:
        return {}
    # builder sub-step records nest inside the builder's own record
    keep = ~((tr["kind"] == 8) & (tr["payload"] >= 2) & (tr["payload"] < 0x100))
    tr = {k: v[keep] for k, v in tr.items()}
    t0 = int(tr["t_req"].min())
    t1 = int(tr["t_end"].max())
    span = max(1, t1 - t0)
    busy = float(np.sum(tr["t_end"] - tr["t_start"]))
    wait = float(np.sum(tr["t_start"] - tr["t_req"]))
    last_end = {}
    for w, e in zip(tr["worker"], tr["t_end"]):
        last_end[int(w)] = max(last_end.get(int(w), 0), int(e))
    tail = float(sum(t1 - e for e in last_end.values()) + (workers - len(last_end)) * span)
    total = float(span) * workers
    return {
        "span_us": span / CLOCK_HZ * 1e6,
        "busy_frac": busy / total,
        "claim_wait_frac": wait / total,
        "tail_idle_frac": tail / total,
        "tasks": int(tr["t_end"].size),
    }


def by_kind(tr: Dict[str, np.ndarray]) -> Dict[str, Dict[str, float]]:
    out = {}
    for k, name in KINDS.items():
        m = tr["kind"] == k
        if m.any():
            d = (tr["t_end"][m] - tr["t_start"][m]) / CLOCK_HZ * 1e6
            out[name] = {"n": int(m.sum()), "mean_us": float(d.mean()), "sum_us": float(d.sum())}
    return out


def row_tiles(counts, th: int, bands: int = 4):
    """Expert row tiles in the builder's order: token bands in order (tile m
    of an expert with nt tiles in band b when ceil(nt b / bands) <= m <
    ceil(nt (b + 1) / bands)), inside a band experts by descending count
    (ties to the lower index), an expert's tiles consecutive.  Returns
    (expert, rows, m) per tile."""
    order = sorted(range(len(counts)), key=lambda e: (-int(counts[e]), e))
    lo = lambda n, b: (n * b + bands - 1) // bands
    tiles = []
    for b in range(bands):
        for e in order:
            c = int(counts[e])
            n = (c + th - 1) // th
            for m in range(lo(n, b), lo(n, b + 1)):
                tiles.append((e, min(th, c - th * m), m))
    return tiles


def calibrate(tr: Dict[str, np.ndarray], info: Dict[str, float], shape, counts) -> Dict[str, float]:
    """The cost model's per-worker rates re-measured from a task trace: the
    bytes/s a gather (permute) task moves (rows read and written), and the
    MFMA flop/s of full-height UP and DOWN tiles (executed flops), each the
    median over its tasks; beside them the constants the library froze."""
    esz = 4 if shape.dtype == "fp32" else 2
    th = info["row_tile"]
    pr = info["permute_rows"]
    pch = th // pr
    n_up, n_down, sk = info["up_ntiles"], info["down_ntiles"], info["split_k"]
    tiles = row_tiles(counts, th, info.get("bands", 4))
    dur = (tr["t_end"] - tr["t_start"]) / CLOCK_HZ
    g_rates, up_rates, down_rates = [], [], []
    for k, p, t in zip(tr["kind"], tr["payload"], dur):
        if t <= 0:
            continue
        k, p = int(k), int(p)
        if k == 3:                                     # PERM
            mt, c = divmod(p, pch)
            if mt < len(tiles):
                rows = min(pr, tiles[mt][1] - c * pr)
                g_rates.append(2.0 * rows * shape.d * esz / t)
        elif k == 4:                                   # UP, full tiles only
            mt = p // n_up
            if mt < len(tiles) and tiles[mt][1] == th:
                up_rates.append(4.0 * th * shape.d * 128 / t)
        elif k == 5:                                   # DOWN, full tiles only
            mt = p // sk // n_down
            if mt < len(tiles) and tiles[mt][1] == th:
                cols = shape.d // n_down
                down_rates.append(2.0 * th * (shape.f / sk) * cols / t)
    med = lambda xs: float(np.median(xs)) if xs else None
    return {
        "gather_bytes_per_s_per_worker": med(g_rates),
        "up_flops_per_s_per_cu": med(up_rates),
        "down_flops_per_s_per_cu": med(down_rates),
        "tasks": {"perm": len(g_rates), "up_full": len(up_rates), "down_full": len(down_rates)},
        "frozen": {"gather_bytes_per_s_per_worker": info.get("cost_gather_bytes_per_worker"),
                   "mfma_flops_per_s_per_cu": info.get("cost_mfma_flops_per_cu"),
                   "hbm_bytes_per_s": info.get("cost_hbm_bytes")},
    }


def geomean(xs) -> float:
    xs = [x for x in xs if x and x > 0]
    return math.exp(sum(math.log(x) for x in xs) / len(xs)) if xs else float("nan")
