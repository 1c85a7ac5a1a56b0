// sched.hpp -- the persistent scheduler.
//
// Dynamic mode (the method).  Workgroups stay resident and loop: claim a
// ready task by an atomic increment of a queue head (xxqk.cn/news/665650
// s2.1, fetch_task), run it, publish its results (write-through stores,
// drained before the counter update; see common.hpp), and decrement the
// dependency counters of its consumers; the
// producer that brings a counter to zero pushes the consumers into a ready
// queue (same page s2.3; m.xxqk.cn/news/657744 s2.3: readiness follows the
// data, no global barrier).  A worker leaves a queue only when its claimed
// slot is past that queue's published task total, never when the queue
// merely looks empty -- the early-exit bug m.xxqk.cn/news/657744 s3.3
// describes.  After routing the builder sizes a memory-bound worker group
// from the per-expert counts (spatial scheduler, Weave abstract); its
// members drain the permute queue and then join the compute queue, while the
// rest start on expert GEMMs as soon as rows land (temporal interleaving).
//
// Queues: QA (router tiles and position tiles: all workers, first),
// QM (permute tasks: the memory group), QC (shared-expert tiles, expert
// UP/DOWN tiles: everyone once their own queue is drained).
//
// Static mode (the baseline the pages argue against): identical tasks,
// pre-assigned round-robin from a worker ticket, a grid barrier between
// stages (or, with MOE_FLAG_REF_SYNC, a spin on each task's own counter and a
// fixed worker split).
#pragma once
#include "stages.hpp"

namespace moe {

constexpr int kClaimExhausted = -1;
constexpr int kClaimAbort = -2;
constexpr int kFlagTrace = 0x2;
constexpr int kFlagPhaseSync = 0x4;
constexpr int kFlagRefSync = 0x8;
constexpr int kFlagNoSteal = 0x10;
constexpr int kFlagXcdAffinity = 0x20;
constexpr int kFlagFifo = 0x40;
constexpr int kFlagContPriority = 0x80;
constexpr int kFlagLocalQueues = 0x100;
constexpr int kFlagPerturb = 0x200;
// Push target meaning "the local queue of the pushing worker's XCD".
constexpr int QL = kNumQueues;

// The queue continuation work (DOWN, shared DOWN, combine, NORM) goes to:
// the one compute queue, in push order (default), or -- with
// MOE_FLAG_CONT_PRIORITY and without MOE_FLAG_FIFO -- its own queue, which
// workers serve before new compute-queue work.  Measured on the layer shapes
// here, one FIFO queue is the faster policy (the priority queue holds the
// UP tiles behind a long DOWN backlog), so it is the default.
DEV bool cont_priority(const Params& p) {
  return (p.flags & kFlagContPriority) != 0 && (p.flags & kFlagFifo) == 0;
}
// MOE_FLAG_LOCAL_QUEUES: continuation work goes to the local queue of the
// XCD whose worker made it ready (its inputs were just written through that
// XCD's L2); workers serve their own XCD's local queue first, then the
// global compute queue, then steal from other XCDs' local queues (the
// per-CU-queue-with-global-fallback pattern of xxqk.cn/news/665650 s4.4,
// with the XCD as the locality domain).
DEV bool local_queues(const Params& p) { return (p.flags & kFlagLocalQueues) != 0; }
DEV int qcont(const Params& p) {
  return local_queues(p) ? QL : cont_priority(p) ? QH : QC;
}

// XCD affinity: the UP task of column tile n goes to the ready queue of XCD
// n % 8, so the workers of one XCD keep reading the same weight panels
// through their own L2 (m.xxqk.cn/news/657744 s3.2, affinity); a worker
// whose compute-queue slot is still empty takes an already-pushed UP task,
// its own XCD's queue first.  Only pushed tasks are taken: a task whose slot
// index is below the queue's tail is filled now or within one store.
DEV bool affinity(const Params& p) { return (p.flags & kFlagXcdAffinity) != 0; }
DEV int* ucw(const Params& p, int word, int x) { return p.ctrl + (word + x) * kCtrlStride; }

DEV int* cw(const Params& p, int word) { return p.ctrl + word * kCtrlStride; }

// Race perturbation (MOE_FLAG_PERTURB; m.xxqk.cn/news/657744 s3.3 on
// hunting scheduler races): thread 0 sleeps a pseudo-random 0 .. 63 x 128
// clocks before every claim and every dependency decrement, and pushed
// bursts land in reverse order, so the interleavings a test sees are far
// from the usual ones.  The hash of the clock and a per-site salt is
// splitmix-style mixing; only timing depends on it, never a result.
DEV void perturb(const Params& p, uint32_t salt) {
  if (!(p.flags & kFlagPerturb)) return;
  uint32_t h = (uint32_t)__builtin_amdgcn_s_memrealtime() * 0x9e3779b9u ^ salt;
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  for (uint32_t i = 0, n = h & 63u; i < n; ++i) __builtin_amdgcn_s_sleep(2);
}

DEV bool timed_out(const Params& p, uint64_t t0) {
  return (long long)(rtc() - t0) > p.timeout_ticks;
}

// Thread 0: claim the next slot of queue q and wait until it is filled.
// `pend` keeps the claimed slot across calls: with `steal` set, a worker whose
// compute-queue slot is still empty takes an already-pushed permute task and
// comes back to its own slot afterwards, so gather work never waits while
// compute workers idle (the steal variant of the spatial split).  Steals take
// permute slots by atomic increment, so any number of idle workers start
// permute tasks within one memory round trip.  Every poll issues its loads
// together (one round trip per poll, not one per load).
DEV int wait_slot(const Params& p, const int* sl) {
  const uint64_t t0 = rtc();
  for (;;) {
    const int v = ld_relaxed(sl);
    const int err = ld_relaxed(cw(p, CW_ERROR));
    if (v != 0) return v - 1;
    if (err != 0) return kClaimAbort;
    if (timed_out(p, t0)) {
      set_error(p, 5);
      return kClaimAbort;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Thread 0: take an already-pushed task from the per-XCD queues of this
// XCD and the next nx - 1 XCDs, in that order.  One poll reads every
// queue's head and tail in a single round trip (the loads are independent);
// a slot is then claimed by compare-and-swap on the head only while it lies
// below the observed tail, so the claimed slot has been pushed (its store is
// at most a few instructions behind the tail increment): a worker never
// waits here on a slot that may never be filled.  `count`: add the take to
// the local-queue claim counter.
DEV int take_xcd(const Params& p, int nx, bool count) {
  const int x0 = xcc_id() & (kXcds - 1);
  int hd[kXcds], tl[kXcds];
#pragma unroll
  for (int i = 0; i < kXcds; ++i) {
    const int x = (x0 + i) & (kXcds - 1);
    hd[i] = i < nx ? ld_relaxed(ucw(p, CW_UHEAD, x)) : 0;
    tl[i] = i < nx ? ld_relaxed(ucw(p, CW_UTAIL, x)) : 0;
  }
#pragma unroll
  for (int i = 0; i < kXcds; ++i) {
    const int x = (x0 + i) & (kXcds - 1);
    int h = hd[i];
    while (h < tl[i] && h < p.q_cap) {
      const int seen = cas_relaxed(ucw(p, CW_UHEAD, x), h, h + 1);
      if (seen == h) {
        if (count) add_relaxed(cw(p, CW_LCLAIMED), 1);
        return wait_slot(p, p.uslots + (size_t)x * p.q_cap + h);
      }
      h = seen;
      tl[i] = ld_relaxed(ucw(p, CW_UTAIL, x));
    }
  }
  return kClaimExhausted;
}

// XCD affinity: an UP task from the XCD queues, own first.
DEV int take_up(const Params& p) { return take_xcd(p, kXcds, false); }

// Local queues: continuation work from this XCD's queue and, nx = 8, from
// the other XCDs' (stealing); every take is counted, so a worker knows when
// all continuation tasks have been claimed.
DEV int take_local(const Params& p, int nx) { return take_xcd(p, nx, true); }

// Thread 0's reservations across claims: slots [pb, pe) of its current
// queue (taken claim_batch at a time with one atomic increment on the
// compute queue, one at a time elsewhere) and one continuation slot h.
struct Reserve {
  int pb, pe, h;
};

// Thread 0: claim for queue q.  `r` keeps claimed but not yet filled
// slot of q across calls.  For the compute queue (q == QC) the continuation
// queue QH (DOWN, shared DOWN, combine, NORM work) comes first: a worker
// that sees pushed QH work reserves the next QH slot (`pend_h`) by one
// atomic increment before it takes new QC work, so started row tiles finish,
// and their token tiles' combines become ready, before new UP work starts.
// Reservations are never waited on while other work exists: a reserved
// slot that is not yet filled stays pending while the worker runs its QC
// work (every claim is an increment that always succeeds -- no
// compare-and-swap retries on a hot word), and a filled reserved slot is
// taken first at the next claim.  A worker leaves only when its QC index is
// past QC's total and QH holds nothing more for it.
// Batched claims (claim_batch > 1, xxqk.cn/news/665650 s4.2): one atomic
// increment reserves that many consecutive compute-queue slots, which the
// worker then runs in order, so the hot head word sees a fraction of the
// atomics; the reserved slots are this worker's, filled or not.
DEV int claim(const Params& p, int q, Reserve& r, bool steal) {
  perturb(p, 0x1000u + q);
  const bool cont = q == QC && cont_priority(p);
  const bool local = q == QC && local_queues(p);
  const int batch = q == QC ? p.claim_batch : 1;
  const uint64_t t0 = rtc();
  int nx = 1;        // local queues polled: this XCD's, then (after one
                     // empty pass over the global queue) every XCD's
  for (;;) {
    int hh = 0, ht = 0, htot = 0, vh = 0;
    if (cont) {
      hh = ld_relaxed(cw(p, CW_HEAD + QH));
      ht = ld_relaxed(cw(p, CW_TAIL + QH));
      htot = ld_relaxed(cw(p, CW_TOTAL + QH));
      if (r.h >= 0) vh = ld_relaxed(p.slots + (size_t)QH * p.q_cap + r.h);
    }
    if (vh != 0) {                     // the reserved continuation task is there
      r.h = -1;
      return vh - 1;
    }
    if (cont && r.h < 0 && hh < ht && hh < htot) {
      const int i = add_relaxed(cw(p, CW_HEAD + QH), 1);
      if (i < htot && i < p.q_cap) {
        const int v = ld_relaxed(p.slots + (size_t)QH * p.q_cap + i);
        if (v != 0) return v - 1;
        r.h = i;                       // pushed soon, or later: keep it
      }
    }
    if (local) {                       // this XCD's continuation work first
      const int t = take_local(p, nx);
      if (t != kClaimExhausted) return t;
    }
    if (r.pb >= r.pe) {
      r.pb = add_relaxed(cw(p, CW_HEAD + q), batch);
      r.pe = r.pb + batch;
    }
    // the slot, the queue's total and the error word in one round trip
    // (after the head increment, not before it: a claim is two round trips)
    const int h = r.pb;
    const int v = h < p.q_cap ? ld_relaxed(p.slots + (size_t)q * p.q_cap + h) : 0;
    const int total = ld_relaxed(cw(p, CW_TOTAL + q));
    const int err = ld_relaxed(cw(p, CW_ERROR));
    if (err != 0) return kClaimAbort;
    if (v != 0) {            // a filled slot is always below the total
      ++r.pb;
      return v - 1;
    }
    // past q's total (so are the later reservations): nothing more from q;
    // leave unless continuation work is still owed to this worker or to the
    // local queues
    if (h >= total) {
      const bool cont_left = cont && (r.h >= 0 || ld_relaxed(cw(p, CW_HEAD + QH)) < htot);
      const bool local_left =
          local && ld_relaxed(cw(p, CW_LCLAIMED)) < ld_relaxed(cw(p, CW_LTOTAL));
      if (!cont_left && !local_left) {
        r.pb = r.pe = -1;
        return kClaimExhausted;
      }
    }
    if (steal) {
      const int mh = ld_relaxed(cw(p, CW_HEAD + QM));
      const int mt = ld_relaxed(cw(p, CW_TAIL + QM));
      if (mh < mt) {
        // pushed permute tasks are waiting: take one (the push is one burst,
        // so a slot below the published total is filled now or very soon)
        const int hm = add_relaxed(cw(p, CW_HEAD + QM), 1);
        if (hm < ld_relaxed(cw(p, CW_TOTAL + QM)) && hm < p.q_cap)
          return wait_slot(p, p.slots + (size_t)QM * p.q_cap + hm);
      }
    }
    if (q == QC && affinity(p)) {
      const int t = take_up(p);
      if (t != kClaimExhausted) return t;
    }
    nx = kXcds;                        // next pass: steal local work too
    if (timed_out(p, t0)) {
      set_error(p, 5 /* MOE_ERR_TIMEOUT */);
      return kClaimAbort;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Thread 0: spin until *c reaches zero (static mode's per-task dependency).
DEV bool wait_zero(const Params& p, const int* c) {
  const uint64_t t0 = rtc();
  while (ld_relaxed(c) != 0) {
    if (ld_relaxed(cw(p, CW_ERROR)) != 0) return false;
    if (timed_out(p, t0)) {
      set_error(p, 5);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Tail word and slot array of push target q: a queue, or QL, the local
// queue of the calling workgroup's XCD.
DEV int* push_tail(const Params& p, int q) {
  return q == QL ? ucw(p, CW_UTAIL, xcc_id() & (kXcds - 1)) : cw(p, CW_TAIL + q);
}
DEV int* push_slots(const Params& p, int q) {
  return q == QL ? p.uslots + (size_t)(xcc_id() & (kXcds - 1)) * p.q_cap
                 : p.slots + (size_t)q * p.q_cap;
}

// All threads: push n task ids (id_of(i)) into queue q.  The slot stores are
// agent-coherent; everything the new tasks read was written through and
// drained by its producers before they published.
template <typename F>
DEV void push_burst(const Params& p, int q, int n, int* s_tmp, F&& id_of) {
  if (n <= 0) return;
  publish_fence();
  if (tidx() == 0) s_tmp[0] = add_relaxed(push_tail(p, q), n);
  __syncthreads();
  const int base = uniform(s_tmp[0]);
  __syncthreads();
  if (base + n > p.q_cap) {
    if (tidx() == 0) set_error(p, 6 /* MOE_ERR_CAPACITY */);
    return;
  }
  int* slots = push_slots(p, q) + base;
  const bool rev = (p.flags & kFlagPerturb) != 0;
  for (int i = tidx(); i < n; i += kThreads) st_relaxed(slots + i, id_of(rev ? n - 1 - i : i) + 1);
}

// All threads: the last of `target` arrivals on counter c returns true.
DEV bool arrive_last(const Params& p, int* c, int delta, int last_old, int* s_tmp) {
  publish_fence();
  __syncthreads();
  if (tidx() == 0) {
    perturb(p, 0x2000u);
    s_tmp[0] = (add_relaxed(c, delta) == last_old);
  }
  __syncthreads();
  const bool last = uniform(s_tmp[0]) != 0;
  __syncthreads();
  if (last) consume_fence();
  return last;
}

// Grid barrier over all workers (static mode).  Returns false on abort.
// The arrival counter only grows (it starts at 0 in every launch): barrier
// number gen is passed once (gen + 1) * workers arrivals are counted, so no
// store ever resets a word another worker may still be adding to.
DEV bool grid_barrier(const Params& p, int& gen, int* s_tmp) {
  publish_fence();
  __syncthreads();
  if (tidx() == 0) {
    int ok = 1;
    const int target = (gen + 1) * p.workers;
    add_relaxed(cw(p, CW_BAR_COUNT), 1);
    const uint64_t t0 = rtc();
    while (ld_relaxed(cw(p, CW_BAR_COUNT)) < target) {
      if (ld_relaxed(cw(p, CW_ERROR)) != 0) { ok = 0; break; }
      if (timed_out(p, t0)) { set_error(p, 5); ok = 0; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    s_tmp[0] = ok;
  }
  __syncthreads();
  const bool ok = uniform(s_tmp[0]) != 0;
  __syncthreads();
  ++gen;
  consume_fence();
  return ok;
}

DEV void trace_record(const Params& p, int task, int worker, uint64_t t_req,
                      uint64_t t_start, uint64_t t_end) {
  if (!(p.flags & kFlagTrace) || p.trace == nullptr || tidx() != 0) return;
  asm volatile("" : "+v"(task));
  const int i = add_relaxed(cw(p, CW_TRACE), 1);
  if (i < p.trace_cap) {
    uint64_t* r = p.trace + (size_t)i * 4;
    r[0] = t_req;
    r[1] = t_start;
    r[2] = t_end;
    r[3] = (uint64_t)(uint32_t)task | ((uint64_t)(worker & 0xffff) << 32) |
           ((uint64_t)xcc_id() << 48);
  }
}

// Trace record of a scheduler phase that is not a queued task: the
// post-routing builder and its steps, the router reduction (TK_BUILD,
// payload = phase id).
DEV void trace_mark(const Params& p, int phase, int worker, uint64_t t0, uint64_t t1) {
  trace_record(p, make_task(TK_BUILD, phase), worker, t0, t0, t1);
}

// One thread: token tile rt has all its expert rows: push the tasks that
// follow -- its combine tasks (all column chunks), or, when the DOWN tiles
// scatter-added into y themselves, its NORM task.
DEV void push_tile_ready(const Params& p, int rt, bool scat) {
  const int n = scat ? 1 : p.n_cc;
  const int q = qcont(p);
  const int base = add_relaxed(push_tail(p, q), n);
  if (base + n > p.q_cap) {
    set_error(p, 6 /* MOE_ERR_CAPACITY */);
    return;
  }
  int* sl = push_slots(p, q) + base;
  if (scat) {
    st_relaxed(sl, make_task(TK_NORM, rt) + 1);
    return;
  }
  for (int c = 0; c < p.n_cc; ++c) st_relaxed(sl + c, make_task(TK_COMB, rt * p.n_cc + c) + 1);
}

// All threads, after a DOWN tile of rows [row0, row0 + rows): its results
// are published, then each token tile those rows belong to loses one
// pending tile; the arrival that empties a counter releases that tile's
// next tasks (dynamic mode).  An expert's rows are sorted by token, so
// the tile's token tiles are the runs of perm[r] / 32.
DEV void combine_arrive_rows(const Params& p, int row0, int rows, bool dyn, bool scat) {
  // the rows' tokens (written long before this task) load while the task's
  // own stores drain
  const int r = tidx();
  int blk = -1, prev = -1;
  if (r < rows) {
    blk = p.perm[row0 + r] / kTB;
    prev = r > 0 ? p.perm[row0 + r - 1] / kTB : -1;
  }
  publish_fence();
  __syncthreads();
  if (r < rows) {
    if (blk != prev) {
      perturb(p, 0x3000u + blk);
      if (add_relaxed(p.cnt_comb + blk, -1) == 1 && dyn) push_tile_ready(p, blk, scat);
    }
  }
  __syncthreads();
}

// Same for a shared-expert DOWN tile of the th tokens [th m, th m + th)
// (th = 128 or 256: whole token tiles).
DEV void combine_arrive_shared(const Params& p, int m, bool dyn, bool scat) {
  publish_fence();
  __syncthreads();
  const int per = p.th / kTB;
  const int blk = m * per + tidx();
  if (tidx() < per && blk < p.n_rt &&
      add_relaxed(p.cnt_comb + blk, -1) == 1 && dyn)
    push_tile_ready(p, blk, scat);
  __syncthreads();
}

template <typename Elem, bool SCAT>
struct Sched {
  using S = Stages<Elem>;

  // Publish the builder's results and release the work that follows it.
  static DEV void publish_build(const Params& p, int* s_tmp) {
    const int n_mt = ld_relaxed(cw(p, CW_NMT));
    const int n_perm = ld_relaxed(cw(p, CW_NPERM));
    // a split is in force when the builder chose memory workers (Wm > 0)
    const bool split = ld_relaxed(cw(p, CW_WMEM)) > 0;
    const int qc = qcont(p);
    const int n_up_qc = affinity(p) ? 0 : n_mt * p.n_up_n;
    const int n_cont = n_mt * p.n_down_n * p.splitk + p.n_sdown +
                       (SCAT ? 0 : p.n_rt * p.n_cc) + (p.fuse_norm ? p.n_rt : 0);
    const int n_comp = n_up_qc + p.n_sup + (qc == QC ? n_cont : 0);
    publish_fence();
    __syncthreads();
    if (tidx() == 0) {
      st_relaxed(cw(p, CW_TOTAL + QM), split ? n_perm : 0);
      st_relaxed(cw(p, CW_TOTAL + QH), qc == QH ? n_cont : 0);
      st_relaxed(cw(p, CW_LTOTAL), qc == QL ? n_cont : 0);
      st_relaxed(cw(p, CW_TOTAL + QC), n_comp + (split ? 0 : n_perm));
      if (affinity(p))
        for (int x = 0; x < kXcds; ++x)
          st_relaxed(ucw(p, CW_UTOTAL, x), n_mt * ((p.n_up_n - x + kXcds - 1) / kXcds));
      st_relaxed(cw(p, CW_SPLIT_READY), 1);
    }
    // position tiles go to QA
    push_burst(p, QA, p.n_rt, s_tmp, [&](int i) { return make_task(TK_POS, i); });
    // shared-expert DOWN tiles waited for the routing phase (zeroed y rows)
    const int nsm = p.n_shared * p.n_smt;
    for (int i = tidx(); i < nsm; i += kThreads) {
      if (add_relaxed(p.cnt_sdown + i, -1) == 1) {
        int* sl = nullptr;
        const int q = qcont(p);
        const int base = add_relaxed(push_tail(p, q), p.n_down_n);
        if (base + p.n_down_n <= p.q_cap) sl = push_slots(p, q) + base;
        else set_error(p, 6);
        if (sl) {
          publish_fence();
          for (int n = 0; n < p.n_down_n; ++n)
            st_relaxed(sl + n, make_task(TK_SDOWN, i * p.n_down_n + n) + 1);
        }
      }
    }
  }

  // All threads, once every POS task is done, with the gather fused into
  // the UP tiles: push every UP task -- as one burst into the compute
  // queue, or (XCD affinity) column tile n into XCD n % 8's queue, each
  // XCD's share written below a tail raised once (bases staged in LDS).
  static DEV void push_all_up(const Params& p, char* smem, int* s_tmp) {
    const int n_mt = ld_relaxed(cw(p, CW_NMT));
    if (!affinity(p)) {
      push_burst(p, QC, n_mt * p.n_up_n, s_tmp, [&](int i) { return make_task(TK_UP, i); });
      return;
    }
    int* s_base = reinterpret_cast<int*>(smem);
    publish_fence();
    if (tidx() < kXcds) {
      const int x = tidx();
      s_base[x] = add_relaxed(ucw(p, CW_UTAIL, x), n_mt * ((p.n_up_n - x + kXcds - 1) / kXcds));
    }
    __syncthreads();
    for (int i = tidx(); i < n_mt * p.n_up_n; i += kThreads) {
      const int mt = i / p.n_up_n, n = i % p.n_up_n, x = n % kXcds;
      const int per = (p.n_up_n - x + kXcds - 1) / kXcds;   // column tiles of XCD x
      const int slot = s_base[x] + mt * per + n / kXcds;
      if (slot < p.q_cap) st_relaxed(p.uslots + (size_t)x * p.q_cap + slot, make_task(TK_UP, i) + 1);
      else set_error(p, 6 /* MOE_ERR_CAPACITY */);
    }
    __syncthreads();
  }

  // A 32-token tile is routed: the last one to finish runs the builder
  // (dynamic mode; static mode runs it between its stage barriers).
  static DEV void tile_routed(const Params& p, char* smem, int* s_tmp, bool dyn, int worker) {
    if (arrive_last(p, cw(p, CW_ROUTE_DONE), 1, p.n_rt - 1, s_tmp) && dyn) {
      const uint64_t tb = rtc();
      S::build(p, smem, worker);
      __syncthreads();
      const uint64_t tp = rtc();
      publish_build(p, s_tmp);
      trace_mark(p, kPhaseBuild, worker, tb, tp);
      trace_mark(p, kPhasePublish, worker, tp, rtc());
    }
  }

  // Thread 0 of a dynamic worker on the plain compute queue (FIFO; no
  // continuation-priority, local or per-XCD queues), whose reserved slots
  // are used up: increment the compute queue's head for its next claim now,
  // before this task's publication, so that the increment's round trip
  // overlaps the publication's store drain; the claim then only reads the
  // slot.  Returns the first reserved slot, or -1.
  static DEV int pre_reserve(const Params& p, const int* s_tmp, bool pre) {
    if (!pre || tidx() != 0 || s_tmp[4] < s_tmp[5]) return -1;
    return add_relaxed(cw(p, CW_HEAD + QC), p.claim_batch);
  }
  static DEV void pre_commit(const Params& p, int* s_tmp, int slot) {
    if (tidx() == 0 && slot >= 0) {
      s_tmp[4] = slot;
      s_tmp[5] = slot + p.claim_batch;
    }
  }

  // Run one task; in dynamic mode also publish it and push what it enables.
  // *t_body receives the clock at the end of the task body, before any
  // publication, so a trace can check producer-end <= consumer-start; a
  // task that first waits for its producers moves *t_start past the wait.
  // pre: this worker claims from the plain compute queue (see pre_reserve).
  static DEV void run(const Params& p, int task, char* smem, int* s_tmp, bool dyn,
                      uint64_t* t_start, uint64_t* t_body, int worker, bool pre = false) {
    int slot = -1;   // pre-reserved compute-queue slot (thread 0)
    const int kind = task_kind(task);
    const int pl = task_payload(task);
    *t_body = 0;
    switch (kind) {
      case TK_ROUTE:
      case TK_RFIN: {
        // one call site each of the partial summation + top-k and of the
        // builder (tile_routed) for every router path
        bool routed = true;
        int fin = -1;                 // tile whose partials are summed here
        const float* part0 = nullptr;
        size_t stride = 0;
        if (kind == TK_RFIN) {
          // every router task precedes the finish tasks (in the router
          // queue and in the static order), so the group's K slices are all
          // claimed or done by the time this waits for them
          if (tidx() == 0) s_tmp[0] = wait_zero(p, p.cnt_route + pl / (256 / kTB));
          __syncthreads();
          const bool ok = uniform(s_tmp[0]) != 0;
          __syncthreads();
          if (!ok) break;
          consume_fence();
          *t_start = rtc();
          fin = pl;
          part0 = p.route_part + (size_t)pl * kTB * p.E;
          stride = (size_t)p.T * p.E;
        } else if (p.route_wide) {
          // a K slice of a 256-token group: its partial is published by the
          // group's count; the group's TK_RFIN tasks wait for it to reach 0
          S::route_wide(p, pl / p.rsk, pl % p.rsk, smem, SCAT);
          *t_body = rtc();
          arrive_last(p, p.cnt_route + pl / p.rsk, -1, 1, s_tmp);
          routed = false;
        } else {
          const int rt = pl / p.rsk;
          S::route(p, rt, pl % p.rsk, smem, SCAT);
          *t_body = rtc();
          if (p.rsk > 1) {
            // the last K slice of this tile reduces the partials and routes
            routed = arrive_last(p, p.cnt_route + rt, -1, 1, s_tmp);
            if (routed) {
              fin = rt;
              part0 = S::route_part_block(p, rt, 0);
              stride = (size_t)kTB * p.E;
            }
          }
        }
        if (fin >= 0) {
          const uint64_t tf = rtc();
          S::route_sum_topk(p, fin, part0, stride, smem);
          if (kind == TK_RFIN) *t_body = rtc();
          else trace_mark(p, kPhaseRouteFinish + fin, worker, tf, rtc());
        }
        if (routed) tile_routed(p, smem, s_tmp, dyn, worker);
        break;
      }
      case TK_POS: {
        const int nd = S::position(p, pl, smem);
        *t_body = rtc();
        // the combine of these tokens waits for the DOWN tiles of the nd row
        // tiles holding their rows; this replaces the counter's initial
        // "positions pending" unit (k_reset) by that many tiles
        // (with scatter-add the counter only gates the NORM task)
        if (tidx() == 0) {
          const int delta = nd * p.n_down_n * p.splitk - 1;
          s_tmp[0] = (!SCAT || p.fuse_norm) && (add_relaxed(p.cnt_comb + pl, delta) + delta == 0);
        }
        __syncthreads();
        const bool comb_ready = uniform(s_tmp[0]) != 0;
        __syncthreads();
        if (comb_ready && dyn) {
          publish_fence();
          __syncthreads();
          if (tidx() == 0) push_tile_ready(p, pl, SCAT);
          __syncthreads();
        }
        if (arrive_last(p, cw(p, CW_POS_DONE), 1, p.n_rt - 1, s_tmp) && dyn) {
          if (p.gather_a) {
            // every row's token is known: all UP tiles are ready at once
            push_all_up(p, smem, s_tmp);
          } else {
            const int n_perm = ld_relaxed(cw(p, CW_NPERM));
            const int q = ld_relaxed(cw(p, CW_WMEM)) > 0 ? QM : QC;
            push_burst(p, q, n_perm, s_tmp, [&](int i) { return p.perm_list[i]; });
          }
        }
        break;
      }
      case TK_PERM: {
        const int mt = pl / p.pch, c = pl % p.pch;
        S::permute(p, mt, c);
        *t_body = rtc();
        if (arrive_last(p, p.cnt_perm + mt, -1, 1, s_tmp) && dyn) {
          if (affinity(p)) {
            // one thread per column tile, into XCD n % 8's queue
            const int n = tidx();
            if (n < p.n_up_n) {
              const int x = n % kXcds;
              const int slot = add_relaxed(ucw(p, CW_UTAIL, x), 1);
              if (slot < p.q_cap)
                st_relaxed(p.uslots + (size_t)x * p.q_cap + slot, make_task(TK_UP, mt * p.n_up_n + n) + 1);
              else
                set_error(p, 6 /* MOE_ERR_CAPACITY */);
            }
            __syncthreads();
          } else {
            push_burst(p, QC, p.n_up_n, s_tmp,
                       [&](int n) { return make_task(TK_UP, mt * p.n_up_n + n); });
          }
        }
        break;
      }
      case TK_UP: {
        const int mt = pl / p.n_up_n, n = pl % p.n_up_n;
        S::up(p, mt, n, smem);
        *t_body = rtc();
        slot = pre_reserve(p, s_tmp, pre);
        const int ks = slice_of(n, p.n_up_n, p.splitk);
        if (arrive_last(p, p.cnt_down + mt * p.splitk + ks, -1, 1, s_tmp) && dyn)
          push_burst(p, qcont(p), p.n_down_n, s_tmp, [&](int nn) {
            return make_task(TK_DOWN, (mt * p.n_down_n + nn) * p.splitk + ks);
          });
        break;
      }
      case TK_DOWN: {
        const int ks = pl % p.splitk;
        const int r = pl / p.splitk;
        const int mt = r / p.n_down_n;
        S::down(p, mt, r % p.n_down_n, ks, smem, SCAT);
        *t_body = rtc();
        slot = pre_reserve(p, s_tmp, pre);
        if (!SCAT || p.fuse_norm) {
          const MTile t = p.mtiles[mt];
          combine_arrive_rows(p, t.row0, t.rows, dyn, SCAT);
        }
        break;
      }
      case TK_SUP: {
        const int n = pl % p.n_s_up_n;
        const int sm = pl / p.n_s_up_n;          // s * n_smt + m
        S::shared_up(p, sm / p.n_smt, sm % p.n_smt, n, smem);
        *t_body = rtc();
        slot = pre_reserve(p, s_tmp, pre);
        if (arrive_last(p, p.cnt_sdown + sm, -1, 1, s_tmp) && dyn)
          push_burst(p, qcont(p), p.n_down_n, s_tmp,
                     [&](int nn) { return make_task(TK_SDOWN, sm * p.n_down_n + nn); });
        break;
      }
      case TK_SDOWN: {
        const int n = pl % p.n_down_n;
        const int sm = pl / p.n_down_n;
        S::shared_down(p, sm / p.n_smt, sm % p.n_smt, n, smem, SCAT);
        *t_body = rtc();
        slot = pre_reserve(p, s_tmp, pre);
        if (!SCAT || p.fuse_norm) combine_arrive_shared(p, sm % p.n_smt, dyn, SCAT);
        break;
      }
      case TK_COMB: {
        S::combine(p, pl / p.n_cc, pl % p.n_cc, smem);
        *t_body = rtc();
        slot = pre_reserve(p, s_tmp, pre);
        // the last column chunk of a token tile releases its NORM task
        if (p.fuse_norm && arrive_last(p, p.cnt_norm + pl / p.n_cc, -1, 1, s_tmp) && dyn)
          push_burst(p, qcont(p), 1, s_tmp, [&](int) { return make_task(TK_NORM, pl / p.n_cc); });
        break;
      }
      case TK_NORM: {
        S::norm(p, pl, SCAT);
        *t_body = rtc();
        break;
      }
      default:
        if (tidx() == 0) set_error(p, 1);
    }
    pre_commit(p, s_tmp, slot);
    __syncthreads();
  }
};

// ------------------------------------------------------------- dynamic
// Thread 0, once a worker's router-queue claim is exhausted: until the
// builder has published the split, take the pre-seeded shared-expert UP tiles
// (slots [0, n_sup) of the compute queue; they need no routing, so they fill
// the routing phase's idle workers).  A slot is taken by compare-and-swap
// only while the head is below n_sup, so nobody commits to a compute slot
// before the split exists.  Returns a task, or kClaimExhausted once the split
// is ready (*role then holds the worker's queue), or kClaimAbort.
DEV int wait_split(const Params& p, int* role) {
  const uint64_t t0 = rtc();
  for (;;) {
    const int ready = ld_relaxed(cw(p, CW_SPLIT_READY));
    const int h = ld_relaxed(cw(p, CW_HEAD + QC));
    const int err = ld_relaxed(cw(p, CW_ERROR));
    if (err != 0) return kClaimAbort;
    if (ready != 0) break;
    if (h < p.n_sup) {
      if (cas_relaxed(cw(p, CW_HEAD + QC), h, h + 1) == h) return make_task(TK_SUP, h);
      continue;
    }
    if (timed_out(p, t0)) {
      set_error(p, 5 /* MOE_ERR_TIMEOUT */);
      return kClaimAbort;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  int nq = QC;
  if (p.split_policy != 2) {
    const int wm = ld_relaxed(cw(p, CW_WMEM));
    nq = (add_relaxed(cw(p, CW_ROLE), 1) < wm) ? QM : QC;
  }
  *role = nq;
  return kClaimExhausted;
}

// The launch parameters as the task bodies see them: the same kernel-argument
// block, reached through an offset the compiler cannot prove is zero, so
// nothing a task derives from the parameters (tile addresses, per-lane
// offsets, loop bounds) is hoisted out of the persistent loop and held in
// registers across every task type -- the parameters stay in the scalar
// cache and are reloaded per task for a few cycles.
DEV const Params& params_view(const Params& p) {
  int off = 0;
  asm volatile("" : "+s"(off));
  return *reinterpret_cast<const Params*>(reinterpret_cast<const char*>(&p) + off);
}

// One worker's share of one layer: claim, run, publish, until the layer's
// queues are exhausted (or a device error stops it).  The caller provides
// the workgroup's LDS.  SCAT: the layer's combine mode as a compile-time
// constant, so each instantiation holds only its own DOWN epilogue and
// combine code (the persistent kernel's register allocation covers every
// task type at once).  The launch parameters are read through params_view
// on every pass; the combine mode is a template argument instead of being
// written into a private copy of them.
template <typename Elem, bool SCAT>
DEV void dynamic_worker(const Params& p, char* smem, int* s_tmp, int* s_worker) {
  if (tidx() == 0) *s_worker = add_relaxed(cw(p, CW_TICKET), 1);
  int q = QA;
  // thread 0's reserved, not yet taken slots live in LDS (s_tmp[4..6])
  // between claims, not in registers held across every task body
  // (the -1 is laundered so that no vector of it is hoisted out of the
  // multi-layer loop and held across every task)
  if (tidx() == 0) {
    int none = -1;
    asm volatile("" : "+v"(none));
    s_tmp[4] = s_tmp[5] = s_tmp[6] = none;
  }
  for (;;) {
    // every pass reads the parameters afresh (see params_view)
    const Params& pv = params_view(p);
    const bool steal = pv.split_policy != 2 && !(pv.flags & kFlagNoSteal);
    uint64_t t_req = rtc();
    if (tidx() == 0) {
      Reserve r{s_tmp[4], s_tmp[5], s_tmp[6]};
      int v = claim(pv, q, r, steal && q == QC);
      s_tmp[4] = r.pb;
      s_tmp[5] = r.pe;
      s_tmp[6] = r.h;
      int role = q;
      // routing phase over for this worker: shared-expert tiles until the
      // split is published, then the role the split assigns
      if (v == kClaimExhausted && q == QA) v = wait_split(pv, &role);
      s_tmp[1] = v;
      s_tmp[2] = role;
    }
    __syncthreads();
    const int v = uniform(s_tmp[1]);
    const int nq = uniform(s_tmp[2]);
    __syncthreads();
    if (v == kClaimAbort) break;
    if (v == kClaimExhausted) {
      if (q == QA) { q = nq; continue; }
      if (q == QM) { q = QC; continue; }
      break;
    }
    consume_fence();
    const uint64_t t_start = rtc();
    uint64_t t_body;
    const int worker = uniform(*s_worker);
    uint64_t t_run = t_start;
    const bool pre = q == QC && !cont_priority(pv) && !local_queues(pv) && !affinity(pv);
    Sched<Elem, SCAT>::run(pv, v, smem, s_tmp, true, &t_run, &t_body, worker, pre);
    trace_record(pv, v, worker, t_req, t_run, t_body);
  }
}

template <typename Elem, bool SCAT>
__global__ __launch_bounds__(kThreads, 1) void k_dynamic(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kSmem];
  __shared__ int s_tmp[8];
  __shared__ int s_worker;
  dynamic_worker<Elem, SCAT>(p, smem, s_tmp, &s_worker);
}

// Several independent layers in ONE persistent launch (layers[0..n), each
// with its own control block and tables in its own workspace): a worker
// that finds layer l's queues exhausted goes straight to layer l + 1's
// router tiles while the other workers finish layer l's last tasks, so one
// layer's routing overlaps the previous layer's expert tail instead of
// waiting for a kernel boundary (the follow-up direction of
// m.xxqk.cn/news/657744 section 6.3; the per-layer synchronisation windows
// of xxqk.cn/news/665650 section 3.3).  The parameter blocks sit in device
// memory; they are read through the constant address space (scalar loads).
typedef const __attribute__((address_space(4))) Params ConstParams;

template <typename Elem, bool SCAT>
__global__ __launch_bounds__(kThreads, 1) void k_dynamic_layers(const Params* layers, int n) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kSmem];
  __shared__ int s_tmp[8];
  __shared__ int s_worker;
  ConstParams* lp = (ConstParams*)layers;
  for (int l = 0; l < n; ++l) {
    const Params& p = *(const Params*)(lp + l);
    dynamic_worker<Elem, SCAT>(p, smem, s_tmp, &s_worker);
    __syncthreads();
  }
}

// -------------------------------------------------------------- static
// The worker walks a fixed plan: its round-robin share of each stage, with a
// grid barrier between stages (phase sync), or -- MOE_FLAG_REF_SYNC -- a
// fixed memory group for the gather, and a spin on each task's own
// dependency counter instead of barriers.  The plan is a small state machine
// with ONE call site of the task body, so the kernel holds one copy of every
// tile (register allocation as in the dynamic kernel).
template <typename Elem, bool SCAT>
__global__ __launch_bounds__(kThreads, 1) void k_static(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kSmem];
  __shared__ int s_tmp[8];
  if (tidx() == 0) s_tmp[3] = add_relaxed(cw(p, CW_TICKET), 1);
  __syncthreads();
  const int w = uniform(s_tmp[3]);
  const int W = p.workers;
  const bool ref = (p.flags & kFlagRefSync) && W >= 2;
  const int wm = max(1, p.fixed_mem > 0 ? min(p.fixed_mem, W - 1) : W / 8);
  const int n_route = p.n_route;
  const int n_rfin = p.route_wide ? p.n_rt : 0;
  const int nA = n_route + n_rfin + p.n_sup;
  enum { ST_A, ST_BUILD, ST_POS, ST_PERM, ST_UP, ST_DOWN, ST_COMB, ST_NORM };
  int st = ST_A, i = w, gen = 0;
  int n_mt = 0, n_perm = 0, n_up = 0, n_down = 0;
  for (;;) {
    // this worker's next task: the rest of its share of the current stage,
    // else the stage transition (barrier, builder) and the next stage
    int task = -1;
    const int* dep = nullptr;
    for (;;) {
      if (st == ST_A) {
        // router tasks, the finish tasks of 256-token router groups, and
        // shared-expert UP tiles
        if (i < nA) {
          task = i < n_route          ? make_task(TK_ROUTE, i)
                 : i < n_route + n_rfin ? make_task(TK_RFIN, i - n_route)
                                        : make_task(TK_SUP, i - n_route - n_rfin);
          i += W;
          break;
        }
        if (!grid_barrier(p, gen, s_tmp)) return;
        st = ST_BUILD;
      } else if (st == ST_BUILD) {
        if (w == 0) {
          Stages<Elem>::build(params_view(p), smem);
          __syncthreads();
          // the routing stage (which zeroes y) is over: release the shared DOWN tiles
          for (int s = tidx(); s < p.n_shared * p.n_smt; s += kThreads)
            add_relaxed(p.cnt_sdown + s, -1);
        }
        if (!grid_barrier(p, gen, s_tmp)) return;
        st = ST_POS;
        i = w;
      } else if (st == ST_POS) {
        if (i < p.n_rt) {
          task = make_task(TK_POS, i);
          i += W;
          break;
        }
        if (!grid_barrier(p, gen, s_tmp)) return;
        n_mt = uniform(ld_relaxed(cw(p, CW_NMT)));
        n_perm = uniform(ld_relaxed(cw(p, CW_NPERM)));
        n_up = n_mt * p.n_up_n;
        n_down = n_mt * p.n_down_n * p.splitk;
        st = ST_PERM;
        i = !ref ? w : (w < wm ? w : n_perm);
        if (n_perm == 0) {      // gather fused into UP: no memory group
          st = ST_UP;
          i = w;
        }
      } else if (st == ST_PERM) {
        if (i < n_perm) {
          task = p.perm_list[i];
          i += ref ? wm : W;
          break;
        }
        if (!ref && !grid_barrier(p, gen, s_tmp)) return;
        st = ST_UP;
        i = !ref ? w : (w >= wm ? w - wm : n_up);
      } else if (st == ST_UP) {
        if (i < n_up) {
          task = make_task(TK_UP, i);
          if (ref) dep = p.cnt_perm + i / p.n_up_n;
          i += (ref && n_perm > 0) ? W - wm : W;
          break;
        }
        if (!ref && !grid_barrier(p, gen, s_tmp)) return;
        st = ST_DOWN;
        i = w;
      } else if (st == ST_DOWN) {
        if (i < n_down + p.n_sdown) {
          if (i < n_down) {
            task = make_task(TK_DOWN, i);
            const int ks = i % p.splitk, mt = i / p.splitk / p.n_down_n;
            if (ref) dep = p.cnt_down + mt * p.splitk + ks;
          } else {
            task = make_task(TK_SDOWN, i - n_down);
            if (ref) dep = p.cnt_sdown + (i - n_down) / p.n_down_n;
          }
          i += W;
          break;
        }
        if (SCAT && !p.fuse_norm) return;
        if (!ref && !grid_barrier(p, gen, s_tmp)) return;
        st = SCAT ? ST_NORM : ST_COMB;
        i = w;
      } else if (st == ST_COMB) {
        if (i < p.n_rt * p.n_cc) {
          task = make_task(TK_COMB, i);
          if (ref) dep = p.cnt_comb + i / p.n_cc;
          i += W;
          break;
        }
        if (!p.fuse_norm) return;
        if (!ref && !grid_barrier(p, gen, s_tmp)) return;
        st = ST_NORM;
        i = w;
      } else {
        // the block tail: after the combine chunks (or, with scatter-add,
        // the DOWN tiles) of each token tile
        if (i < p.n_rt) {
          task = make_task(TK_NORM, i);
          if (ref) dep = SCAT ? p.cnt_comb + i : p.cnt_norm + i;
          i += W;
          break;
        }
        return;
      }
    }
    if (dep != nullptr) {
      if (tidx() == 0) s_tmp[1] = wait_zero(p, dep);
      __syncthreads();
      const bool ok = uniform(s_tmp[1]) != 0;
      __syncthreads();
      if (!ok) return;
      consume_fence();
    }
    const uint64_t t0 = rtc();
    uint64_t t_run = t0, t_body;
    Sched<Elem, SCAT>::run(params_view(p), task, smem, s_tmp, false, &t_run, &t_body, w);
    trace_record(p, task, w, t0, t_run, t_body);
  }
}

// ----------------------------------------------- one launch per stage
template <typename Elem>
__global__ __launch_bounds__(kThreads) void k_stage_route(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kRouteSmem];
  if (p.route_from_logits) {
    Stages<Elem>::topk_from_logits(p, blockIdx.x, smem);
    return;
  }
  const int rt = blockIdx.x / p.rsk;
  Stages<Elem>::route(p, rt, blockIdx.x % p.rsk, smem, p.comb_scatter != 0);
  if (p.rsk > 1) {
    __shared__ int s_tmp[8];
    if (!arrive_last(p, p.cnt_route + rt, -1, 1, s_tmp)) return;
    Stages<Elem>::route_finish(p, rt, smem);
  }
}

// 256-token router groups: the K-slice tasks (the 256-row tile's LDS), then
// the per-tile finish tasks in a launch of their own.
template <typename Elem>
__global__ __launch_bounds__(kThreads, 1) void k_stage_route_wide(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kSmem];
  Stages<Elem>::route_wide(p, blockIdx.x / p.rsk, blockIdx.x % p.rsk, smem, p.comb_scatter != 0);
}

template <typename Elem>
__global__ __launch_bounds__(kThreads) void k_stage_rfin(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kRouteSmem];
  Stages<Elem>::route_finish_wide(p, blockIdx.x, smem);
}

template <typename Elem>
__global__ __launch_bounds__(kThreads) void k_stage_build(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kBuildSmem];
  Stages<Elem>::build(p, smem);
}

template <typename Elem>
__global__ __launch_bounds__(kThreads) void k_stage_pos(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kPosSmem];
  Stages<Elem>::position(p, blockIdx.x, smem);
}

template <typename Elem>
__global__ __launch_bounds__(kThreads) void k_stage_perm(Params p) {
  const int n_perm = ld_relaxed(cw(p, CW_NPERM));
  if ((int)blockIdx.x >= n_perm) return;
  const int pl = task_payload(p.perm_list[blockIdx.x]);
  Stages<Elem>::permute(p, pl / p.pch, pl % p.pch);
}

template <typename Elem>
__global__ __launch_bounds__(kThreads, 1) void k_stage_up(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kSmem];
  const int b = blockIdx.x;
  const int routed = p.max_mt * p.n_up_n;
  if (b < routed) {
    const int n_mt = ld_relaxed(cw(p, CW_NMT));
    if (b >= n_mt * p.n_up_n) return;
    Stages<Elem>::up(p, b / p.n_up_n, b % p.n_up_n, smem);
  } else {
    const int pl = b - routed;
    const int n = pl % p.n_s_up_n, sm = pl / p.n_s_up_n;
    Stages<Elem>::shared_up(p, sm / p.n_smt, sm % p.n_smt, n, smem);
  }
}

template <typename Elem>
__global__ __launch_bounds__(kThreads, 1) void k_stage_down(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Stages<Elem>::kSmem];
  const int b = blockIdx.x;
  const int routed = p.max_mt * p.n_down_n * p.splitk;
  if (b < routed) {
    const int n_mt = ld_relaxed(cw(p, CW_NMT));
    if (b >= n_mt * p.n_down_n * p.splitk) return;
    const int ks = b % p.splitk, r = b / p.splitk;
    Stages<Elem>::down(p, r / p.n_down_n, r % p.n_down_n, ks, smem, p.comb_scatter != 0);
  } else {
    const int pl = b - routed;
    const int n = pl % p.n_down_n, sm = pl / p.n_down_n;
    Stages<Elem>::shared_down(p, sm / p.n_smt, sm % p.n_smt, n, smem, p.comb_scatter != 0);
  }
}

template <typename Elem>
__global__ __launch_bounds__(kThreads) void k_stage_norm(Params p) {
  Stages<Elem>::norm(p, blockIdx.x, p.comb_scatter != 0);
}

template <typename Elem>
__global__ __launch_bounds__(kThreads) void k_stage_comb(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[kTB * kMaxK * 8];
  Stages<Elem>::combine(p, blockIdx.x / p.n_cc, blockIdx.x % p.n_cc, smem);
}

// --------------------------------------------- host: stage sequences
// The multi-kernel baseline: one ordinary launch per stage, in stage order on
// stream s; the launch boundaries are its only synchronisation.
template <typename Elem>
hipError_t launch_stage_sequence(const Params& p, hipStream_t s) {
  if (p.route_wide) {
    hipLaunchKernelGGL(k_stage_route_wide<Elem>, dim3(p.n_route), dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL(k_stage_rfin<Elem>, dim3(p.n_rt), dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL(k_stage_route<Elem>, dim3(p.n_route), dim3(kThreads), 0, s, p);
  }
  hipLaunchKernelGGL(k_stage_build<Elem>, dim3(1), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(k_stage_pos<Elem>, dim3(p.n_rt), dim3(kThreads), 0, s, p);
  if (!p.gather_a)
    hipLaunchKernelGGL(k_stage_perm<Elem>, dim3(p.max_perm), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(k_stage_up<Elem>, dim3(p.max_mt * p.n_up_n + p.n_sup), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(k_stage_down<Elem>, dim3(p.max_mt * p.n_down_n * p.splitk + p.n_sdown),
                     dim3(kThreads), 0, s, p);
  if (!p.comb_scatter)
    hipLaunchKernelGGL(k_stage_comb<Elem>, dim3(p.n_rt * p.n_cc), dim3(kThreads), 0, s, p);
  if (p.fuse_norm)
    hipLaunchKernelGGL(k_stage_norm<Elem>, dim3(p.n_rt), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// Routing only, from logits already in p.logits (p.route_from_logits = 1).
template <typename Elem>
hipError_t launch_route_sequence(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(k_stage_route<Elem>, dim3(p.n_rt), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(k_stage_build<Elem>, dim3(1), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(k_stage_pos<Elem>, dim3(p.n_rt), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
