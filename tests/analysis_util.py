"""Trace checks shared by GPU tests: every task ran exactly once, and every
task started after all of its producers' bodies ended."""
from collections import defaultdict

import numpy as np

from dynamic_task_scheduling_amd.analysis import decode_trace

ROUTE, POS, PERM, UP, DOWN, SUP, SDOWN, COMB, NORM, RFIN = 1, 2, 3, 4, 5, 6, 7, 9, 10, 11


def check_trace(raw, layer, routing, fused_norm=False):
    tr = decode_trace(raw)
    info = layer.info
    s = layer.shape
    n_rt = info["route_tiles"]
    n_up = info["up_ntiles"]
    n_down = info["down_ntiles"]
    sk = info["split_k"]
    th = info["row_tile"]
    pch = th // info["permute_rows"]
    counts = routing.expert_counts.cpu().numpy()
    n_mt = int(sum((c + th - 1) // th for c in counts))
    ids, cnt = np.unique(tr["task"], return_counts=True)
    assert np.all(cnt == 1), "a task ran more than once"
    kinds = tr["kind"]
    pl = tr["payload"]
    n_smt = (s.T + th - 1) // th
    n_sup_n = (s.f_shared // 128) if s.n_shared else 0
    n_cc = info["combine_chunks"]
    n_rg = info["route_groups"]      # 256-token router groups (0: 32-token router tiles)
    rsk = info["route_splits"]
    expect = {ROUTE: (n_rg if n_rg else n_rt) * rsk, RFIN: n_rt if n_rg else 0, POS: n_rt,
              UP: n_mt * n_up,
              DOWN: n_mt * n_down * sk,
              SUP: s.n_shared * n_smt * n_sup_n, SDOWN: s.n_shared * n_smt * n_down,
              COMB: 0 if info["combine"] == 1 else n_rt * n_cc,
              NORM: n_rt if fused_norm else 0}
    fused = bool(info.get("gather_fused", 0))
    if fused:
        expect[PERM] = 0
    for k, n in expect.items():
        assert int((kinds == k).sum()) == n, "kind %d ran %d times, expected %d" % (
            k, int((kinds == k).sum()), n)
    start = {int(t): int(v) for t, v in zip(tr["task"], tr["t_start"])}
    end = {int(t): int(v) for t, v in zip(tr["task"], tr["t_end"])}
    # routing is done when every router task (and every group finish) is
    route_end = max(int(e) for e, k in zip(tr["t_end"], kinds) if k in (ROUTE, RFIN))
    group_end = defaultdict(int)   # 256-token router group -> latest K-slice end
    for t, k, p in zip(tr["task"], kinds, pl):
        if k == ROUTE and n_rg:
            group_end[int(p) // rsk] = max(group_end[int(p) // rsk], end[int(t)])
    pos_end = max(end[(POS << 27) | i] for i in range(n_rt))
    perm_end = defaultdict(int)
    for t, k, p in zip(tr["task"], kinds, pl):
        if k == PERM:
            perm_end[int(p) // pch] = max(perm_end[int(p) // pch], end[int(t)])
    up_end = defaultdict(int)   # (mt, ks) -> latest end
    bounds = [ks * n_up // sk for ks in range(sk + 1)]
    def slice_of(n):
        ks = 0
        while ks + 1 < sk and bounds[ks + 1] <= n:
            ks += 1
        return ks
    sup_end = defaultdict(int)
    down_end = defaultdict(int)    # mt -> latest DOWN end
    sdown_end = defaultdict(int)   # shared row tile -> latest shared DOWN end
    for t, k, p in zip(tr["task"], kinds, pl):
        if k == DOWN:
            mt = int(p) // sk // n_down
            down_end[mt] = max(down_end[mt], end[int(t)])
        if k == SDOWN:
            m = (int(p) // n_down) % n_smt
            sdown_end[m] = max(sdown_end[m], end[int(t)])
    # row tiles in the builder's order (token bands, experts by descending
    # count inside a band); a combine tile waits for the DOWN tiles of every
    # row tile that holds one of its tokens' kept slots
    from dynamic_task_scheduling_amd.analysis import row_tiles
    tile_of = {(e, m): mt for mt, (e, rows, m) in enumerate(row_tiles(counts, th, info["bands"]))}
    offs = routing.offsets.cpu().numpy()
    idx = routing.topk_idx.cpu().numpy()
    spos = routing.slot_pos.cpu().numpy()
    comb_need = defaultdict(int)
    for tok in range(s.T):
        for j in range(s.k):
            pos = int(spos[tok, j])
            if pos < 0:
                continue
            e = int(idx[tok, j]) - s.e_begin
            mt = tile_of[(e, (pos - int(offs[e])) // th)]
            comb_need[tok // 32] = max(comb_need[tok // 32], down_end[mt])
        if s.n_shared:
            comb_need[tok // 32] = max(comb_need[tok // 32], sdown_end[tok // th])
    for t, k, p in zip(tr["task"], kinds, pl):
        t, p = int(t), int(p)
        if k == UP:
            up_end[(p // n_up, slice_of(p % n_up))] = max(up_end[(p // n_up, slice_of(p % n_up))], end[t])
        if k == SUP:
            sup_end[p // n_sup_n] = max(sup_end[p // n_sup_n], end[t])
    for t, k, p in zip(tr["task"], kinds, pl):
        t, p = int(t), int(p)
        st = start[t]
        if k == RFIN:
            assert st >= group_end[p // 8], "RFIN before one of its group's K slices"
        elif k == POS:
            assert st >= route_end
        elif k == PERM:
            assert st >= pos_end
        elif k == UP:
            # the fused gather reads perm (all POS tiles); else its row
            # tile's permute tasks
            assert st >= perm_end[p // n_up]
            if fused:
                assert st >= pos_end, "UP before every POS tile (fused gather)"
        elif k == DOWN:
            ks = p % sk
            mt = p // sk // n_down
            assert st >= up_end[(mt, ks)], "DOWN before its UP slice"
        elif k == SDOWN:
            assert st >= sup_end[p // n_down] and st >= route_end
        elif k == COMB:
            assert st >= end[(POS << 27) | (p // n_cc)], "COMB before its POS tile"
            assert st >= comb_need[p // n_cc], "COMB before one of its DOWN tiles"
        elif k == NORM:
            assert st >= end[(POS << 27) | p], "NORM before its POS tile"
            assert st >= comb_need[p], "NORM before one of its DOWN tiles"
            if info["combine"] != 1:
                last = max(end[(COMB << 27) | (p * n_cc + c)] for c in range(n_cc))
                assert st >= last, "NORM before its combine chunks"
    return tr
