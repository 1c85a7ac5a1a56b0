// stages.hpp -- bodies of the MoE-layer tasks.  Every scheduling mode
// (persistent dynamic, persistent static, one launch per stage) runs exactly
// these functions; only who runs them, and when, differs -- the control the
// pages insist on when comparing schedulers (xxqk.cn/news/665650 s3.1: change
// only the scheduling policy, never the operators).
//
// Each function is called by all 256 threads of a workgroup and returns with
// the workgroup converged.  None of them publishes its results: the caller
// owns fences and dependency counters.
#pragma once
#include "common.hpp"
#include "params.hpp"
#include "tile.hpp"
#include "tile2.hpp"

namespace moe {

// Task bodies are compiled as separate functions: one persistent kernel
// holds every task type, and keeping them apart keeps register allocation
// per task type instead of over their union.
#define TASKFN DEV

// Order-preserving 32-bit image of an fp32 value (+0.0 and -0.0 map to the
// same key, so they compare equal).
DEV uint32_t mono_key(float v) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DEV float mono_value(uint32_t m) {
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}

DEV void set_error(const Params& p, int code) {
  cas_relaxed(p.ctrl + CW_ERROR * kCtrlStride, 0, code);
}

// Slices of the DOWN split-K: slice ks covers UP column tiles
// [ks*n/s, (ks+1)*n/s).
DEV int slice_lo(int ks, int n, int s) { return ks * n / s; }
DEV int slice_of(int tile, int n, int s) {
  int ks = 0;
  while (ks + 1 < s && slice_lo(ks + 1, n, s) <= tile) ++ks;
  return ks;
}

// GEMM tile used for expert tasks: bf16 runs the multi-stage LDS ring
// (tile2.hpp); fp32 runs the register-staged tile (tile.hpp).
// Ring depth: as many 64-deep K stages as fit in 144 KB of LDS (bytes in
// flight set a streaming task's rate), at most 7.
constexpr int tile2_stages(int bm, int nb) {
  return (147456 / (bm * 128 + nb * 16384)) > 7 ? 7 : (147456 / (bm * 128 + nb * 16384));
}
template <typename Elem, int BM, int NB>
struct GemmSel {
  using T = Tile<Elem, BM, NB>;
};
template <int BM, int NB>
struct GemmSel<bf16_t, BM, NB> {
  using T = Tile2<BM, NB, tile2_stages(BM, NB)>;
};

// Router tiles (32 tokens x 128 experts): a 4-stage ring for bf16 when the
// router width is a multiple of 128, so the router scratch fits beside it.
template <typename Elem>
struct RouteSel {
  using T = Tile<Elem, 32, 1>;
};
template <>
struct RouteSel<bf16_t> {
  using T = Tile2<32, 1, 4>;
};

template <typename T>
struct requires_n_valid {
  static constexpr bool value = false;
};
template <typename Elem, int BM, int NB>
struct requires_n_valid<Tile<Elem, BM, NB>> {
  static constexpr bool value = true;
};

template <typename Elem>
struct Stages {
  using TR = ElemTraits<Elem>;
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  // LDS of the largest expert tile over every row class and B count
  static constexpr int kSmemTile =
      cmax(cmax(cmax(GemmSel<Elem, 32, 1>::T::LDS_BYTES, GemmSel<Elem, 64, 1>::T::LDS_BYTES),
                cmax(GemmSel<Elem, 128, 1>::T::LDS_BYTES, GemmSel<Elem, 32, 2>::T::LDS_BYTES)),
           cmax(GemmSel<Elem, 64, 2>::T::LDS_BYTES, GemmSel<Elem, 128, 2>::T::LDS_BYTES));
  // Router scratch after the router tile's own two stages.
  static constexpr int kRouteTile =
      Tile<Elem, 32, 1>::LDS_BYTES > RouteSel<Elem>::T::LDS_BYTES
          ? Tile<Elem, 32, 1>::LDS_BYTES
          : RouteSel<Elem>::T::LDS_BYTES;
  static constexpr int kSmem = kSmemTile;
  static_assert(kRouteTile + 32 * kMaxE * 4 + kMaxE * 4 <= kSmemTile, "route LDS");
  // build(): small tables first, then a histogram staging area
  static constexpr int kBuildScratch = 16384;
  static constexpr int kBuildStage = 65536;
  static constexpr int kBuildSmem = kBuildScratch + kBuildStage;
  static_assert(kBuildSmem <= kSmemTile, "build LDS");

  // --------------------------------------------------------------- router
  // Top-k with renormalised softmax for `rows` tokens starting at t0, whose
  // fp32 logits sit at L[row * ldl + e] (LDS or global).  One wave per token;
  // each lane holds experts lane, lane+64, lane+128, lane+192.  Selection
  // key = (order-preserving logit image, inverted index): the maximum is the
  // largest logit, and among equal logits the lowest index.
  static DEV void topk(const Params& p, int t0, int rows, const float* L, int ldl,
                       int* hist_s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = p.E, k = p.k;
    for (int r = wave; r < rows; r += 4) {
      uint64_t key[4];
      bool bad = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (e < E) {
          const float v = L[r * ldl + e];
          if (!__builtin_isfinite(v)) bad = true;
          const uint32_t m = __builtin_isfinite(v) ? mono_key(v) : 1u;
          key[q] = ((uint64_t)m << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
        } else {
          key[q] = 0;
        }
      }
      if (__any(bad) && lane == 0) set_error(p, 7 /* MOE_ERR_NONFINITE */);
      int sel_e[kMaxK];
      float sel_v[kMaxK];
      for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) best = key[q] > best ? key[q] : best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const uint32_t hi = __shfl_xor((int)(best >> 32), off);
          const uint32_t lo = __shfl_xor((int)(uint32_t)best, off);
          const uint64_t o = ((uint64_t)hi << 32) | lo;
          best = o > best ? o : best;
        }
        const int e = (int)(0xffffffffu - (uint32_t)best);
        sel_e[j] = e;
        sel_v[j] = mono_value((uint32_t)(best >> 32));
        if ((e & 63) == lane) key[e >> 6] = 0;
      }
      if (lane == 0) {
        const int t = t0 + r;
        float a[kMaxK];
        float s = 0.f;
        for (int j = 0; j < k; ++j) {
          a[j] = expf(sel_v[j] - sel_v[0]);
          s += a[j];
        }
        for (int j = 0; j < k; ++j) {
          st_wt(p.idx + (size_t)t * k + j, sel_e[j]);
          st_wt(p.w + (size_t)t * k + j, a[j] / s);
          const int el = sel_e[j] - p.e_begin;
          if (el >= 0 && el < p.E_loc) atomicAdd(&hist_s[el], 1);
        }
      }
    }
  }

  static DEV void write_hist(const Params& p, int rt, const int* hist_s) {
    for (int e = threadIdx.x; e < p.E_loc; e += kThreads)
      st_wt(p.hist + (size_t)e * p.hist_ld + rt, hist_s[e]);
  }

  // ROUTE(rt, ks): router logits of tokens [32 rt, 32 rt + 32) over K slice
  // ks of rsk.  With rsk == 1 the task also adds the bias, picks the top-k
  // and writes the tile histogram; with rsk > 1 it writes an fp32 partial
  // and the last slice to finish runs route_finish (fixed-order sum, so the
  // logits do not depend on which slice finished last).  Slice 0 zeroes the
  // tile's y rows, which the combine later accumulates into.
  template <typename RT>
  static DEV void route_gemm(const Params& p, int t0, int rows, int k0, int K, float* Ls,
                             float* part, char* smem) {
    const Elem* x = reinterpret_cast<const Elem*>(p.x) + (size_t)t0 * p.d + k0;
    const Elem* wr = reinterpret_cast<const Elem*>(p.wr) + (size_t)k0 * p.E;
    for (int n0 = 0; n0 < p.E; n0 += kBN) {
      typename RT::Args g;
      g.A = x;
      g.lda = p.d;
      g.a_rows = rows;
      g.B[0] = wr + n0;
      g.ldb = p.E;
      if constexpr (requires_n_valid<RT>::value) g.n_valid = min(kBN, p.E - n0);
      g.K = K;
      typename RT::Acc acc;
      if constexpr (requires_n_valid<RT>::value) RT::run(g, reinterpret_cast<Elem*>(smem), acc);
      else RT::run(g, smem, acc);
      RT::for_each([&](int row, int col, int fm, int fn, int i) __attribute__((always_inline)) {
        const int e = n0 + col;
        if (e < p.E) {
          const float v = acc[0][fm][fn][i];
          if (part) {
            if (row < rows) st_wt(part + (size_t)(t0 + row) * p.E + e, v);
          } else {
            Ls[row * p.E + e] = v;
          }
        }
      });
    }
  }

  static TASKFN void route(const Params& p, int rt, int ks, char* smem) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    if (ks == 0) {
      for (int r = 0; r < rows; ++r) {
        float* yr = p.y + (size_t)(t0 + r) * p.d;
        for (int i = threadIdx.x; i < p.d / 4; i += kThreads) st_wt16(yr, i * 16, make_uint4(0, 0, 0, 0));
      }
    }
    const int Ks = p.d / p.rsk;
    float* Ls = reinterpret_cast<float*>(smem + kRouteTile);     // [32][E]
    float* part = p.rsk > 1 ? p.route_part + (size_t)ks * p.T * p.E : nullptr;
    if (ElemTraits<Elem>::kBf16 && (p.E % kBN) == 0)
      route_gemm<typename RouteSel<Elem>::T>(p, t0, rows, ks * Ks, Ks, Ls, part, smem);
    else
      route_gemm<Tile<Elem, 32, 1>>(p, t0, rows, ks * Ks, Ks, Ls, part, smem);
    if (p.rsk == 1) route_topk(p, rt, smem, false);
  }

  // Sum the K-slice partials of tile rt in slice order, then top-k.
  static TASKFN void route_finish(const Params& p, int rt, char* smem) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    float* Ls = reinterpret_cast<float*>(smem + kRouteTile);
    for (int i = threadIdx.x; i < rows * p.E; i += kThreads) {
      float v = 0.f;
      for (int ks = 0; ks < p.rsk; ++ks) v += p.route_part[((size_t)ks * p.T + t0) * p.E + i];
      Ls[i] = v;
    }
    route_topk(p, rt, smem, true);
  }

  // Bias, exported logits, top-k and the tile histogram from Ls.
  static DEV void route_topk(const Params& p, int rt, char* smem, bool synced) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    float* Ls = reinterpret_cast<float*>(smem + kRouteTile);
    int* hist_s = reinterpret_cast<int*>(smem + kRouteTile + 32 * kMaxE * 4);
    for (int e = threadIdx.x; e < p.E_loc; e += kThreads) hist_s[e] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < rows * p.E; i += kThreads) {
      const int e = i % p.E;
      const float v = Ls[i] + (p.bias ? p.bias[e] : 0.f);
      Ls[i] = v;
      p.logits[(size_t)t0 * p.E + i] = v;
    }
    __syncthreads();
    topk(p, t0, rows, Ls, p.E, hist_s);
    __syncthreads();
    write_hist(p, rt, hist_s);
    (void)synced;
  }

  // Routing from given logits (checking path): top-k + histogram only.
  static TASKFN void topk_from_logits(const Params& p, int rt, char* smem) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    int* hist_s = reinterpret_cast<int*>(smem);
    for (int e = threadIdx.x; e < p.E_loc; e += kThreads) hist_s[e] = 0;
    __syncthreads();
    topk(p, t0, rows, p.logits + (size_t)t0 * p.E, p.E, hist_s);
    __syncthreads();
    write_hist(p, rt, hist_s);
  }

  // ---------------------------------------------------------------- build
  // Runs once, after every ROUTE tile: counts, offsets, per-tile position
  // bases, expert order (most loaded first), the row-tile table, dependency
  // counters, the permute list and -- the cost model -- the worker split.
  // The pages run this "once routing completes", when every layer's
  // communication and computation volumes are known (Weave abstract).
  // Returns nothing; writes tables and control words (not yet published).
  static TASKFN void build(const Params& p, char* smem) {
    int* s_cnt = reinterpret_cast<int*>(smem);            // [256]
    int* s_off = s_cnt + 256;                             // [257]
    int* s_rank = s_off + 257;                            // [256] rank of expert e
    int* s_ord = s_rank + 256;                            // [256] expert of rank r
    int* s_nt = s_ord + 256;                              // [256] tiles of rank r
    int* s_np = s_nt + 256;                               // [256] permute tasks of rank r
    int* s_mtb = s_np + 256;                              // [257] tile base of rank r
    int* s_pb = s_mtb + 257;                              // [257] permute base of rank r
    float* s_cost = reinterpret_cast<float*>(s_pb + 257); // [256] compute seconds of rank r
    float* s_red = s_cost + 256;                          // [kThreads] reduction
    int* s_wm = reinterpret_cast<int*>(s_red + kThreads); // [kThreads]
    const int tid = threadIdx.x;
    const int El = p.E_loc;
    // 1. per-expert counts and per-tile exclusive bases.  The histogram is
    //    staged through LDS in column chunks so its loads are all in flight
    //    at once (one row per thread would be a chain of dependent loads).
    {
      int* s_h = reinterpret_cast<int*>(smem + kBuildScratch);
      const int C = max(4, min(p.hist_ld, (kBuildStage / 4 / max(El, 1)) & ~3));
      int run = 0;
      for (int r0 = 0; r0 < p.n_rt; r0 += C) {
        const int cw = min(C, p.hist_ld - r0);
        const int q4 = cw / 4;
        for (int i = tid; i < El * q4; i += kThreads) {
          const int e = i / q4, q = i % q4;
          *reinterpret_cast<int4*>(s_h + e * cw + q * 4) =
              *reinterpret_cast<const int4*>(p.hist + (size_t)e * p.hist_ld + r0 + q * 4);
        }
        __syncthreads();
        if (tid < El) {
          int* b = p.rt_base + (size_t)tid * p.hist_ld + r0;
          const int nr = min(cw, p.n_rt - r0);
          for (int r = 0; r < nr; ++r) {
            const int v = s_h[tid * cw + r];
            st_wt(b + r, run);
            run += v;
          }
        }
        __syncthreads();
      }
      if (tid < El) {
        s_cnt[tid] = run;
        st_wt(p.counts + tid, run);
      }
    }
    __syncthreads();
    // 2. offsets (exclusive scan) and expert order by descending count
    if (tid == 0) {
      int run = 0;
      for (int e = 0; e < El; ++e) { s_off[e] = run; run += s_cnt[e]; }
      s_off[El] = run;
    }
    if (tid < El) {
      const int c = s_cnt[tid];
      int rank = 0;
      for (int e = 0; e < El; ++e) {
        const int ce = s_cnt[e];
        rank += (ce > c) || (ce == c && e < tid);
      }
      s_rank[tid] = rank;
      s_ord[rank] = tid;
    }
    __syncthreads();
    for (int e = tid; e <= El; e += kThreads) st_wt(p.offsets + e, s_off[e]);
    // 3. row tiles (128 rows; the last one of an expert takes the smallest
    //    class that holds it) and permute chunks, per rank
    const float esz = TR::kBf16 ? 2.f : 4.f;
    if (tid < El) {
      const int e = s_ord[tid];
      st_wt(p.eorder + tid, e);
      const int c = s_cnt[e];
      const int nt = (c + 127) / 128;
      int np = 0;
      float cost = 0.f;
      for (int m = 0; m < nt; ++m) {
        const int rows = min(128, c - 128 * m);
        np += (rows + p.perm_rows - 1) / p.perm_rows;
        const int bm = rows <= 32 ? 32 : rows <= 64 ? 64 : 128;
        // padded MFMA flops vs streamed weight bytes of this tile's GEMMs
        const float fl = 6.f * bm * (float)p.d * (float)p.f;
        const float by = 3.f * esz * (float)p.d * (float)p.f;
        // one worker's time: its MFMA work, or its share of HBM bandwidth
        cost += fmaxf(fl / p.cm_mfma_rate, by * (float)p.workers / p.cm_hbm_bw);
      }
      s_nt[tid] = nt;
      s_np[tid] = np;
      s_cost[tid] = cost;
    }
    __syncthreads();
    if (tid == 0) {
      int a = 0, b = 0;
      for (int r = 0; r < El; ++r) {
        s_mtb[r] = a; a += s_nt[r];
        s_pb[r] = b; b += s_np[r];
      }
      s_mtb[El] = a;
      s_pb[El] = b;
    }
    __syncthreads();
    const int n_mt = s_mtb[El];
    const int n_perm = s_pb[El];
    if (n_mt > p.max_mt || n_perm > p.max_perm) {
      if (tid == 0) set_error(p, 6 /* MOE_ERR_CAPACITY */);
      return;
    }
    if (tid < El) {
      const int e = s_ord[tid];
      const int c = s_cnt[e];
      int mt = s_mtb[tid];
      int pb = s_pb[tid];
      for (int m = 0; m < s_nt[tid]; ++m, ++mt) {
        const int rows = min(128, c - 128 * m);
        MTile t;
        t.e = e;
        t.row0 = s_off[e] + 128 * m;
        t.rows = rows;
        t.bm = rows <= 32 ? 32 : rows <= 64 ? 64 : 128;
        int* tw = reinterpret_cast<int*>(p.mtiles + mt);
        st_wt(tw + 0, t.e);
        st_wt(tw + 1, t.row0);
        st_wt(tw + 2, t.rows);
        st_wt(tw + 3, t.bm);
        const int np = (rows + p.perm_rows - 1) / p.perm_rows;
        st_wt(p.cnt_perm + mt, np);
        for (int ks = 0; ks < p.splitk; ++ks)
          st_wt(p.cnt_down + mt * p.splitk + ks,
                slice_lo(ks + 1, p.n_up_n, p.splitk) - slice_lo(ks, p.n_up_n, p.splitk));
        for (int c2 = 0; c2 < np; ++c2) st_wt(p.perm_list + pb++, make_task(TK_PERM, mt * p.pch + c2));
      }
    }
    // 4. spatial split: smallest memory group whose gather finishes within
    //    `slack` x the compute group's time (cost model, per layer).
    float tot_cost = 0.f;
    if (tid == 0)
      for (int r = 0; r < El; ++r) tot_cost += s_cost[r];
    if (tid == 0) s_red[0] = tot_cost;
    __syncthreads();
    tot_cost = s_red[0];
    __syncthreads();
    const int W = p.workers;
    int wm_choice = 0;
    if (p.split_policy == 0 /* cost model */ && W >= 2) {
      const float R = (float)s_off[El];
      const float bytes = 2.f * R * (float)p.d * esz;
      int best = W - 1;
      for (int wm = 1 + tid; wm < W; wm += kThreads) {
        const float tm = bytes / fminf((float)wm * p.cm_cu_bw, p.cm_hbm_bw);
        const float tc = tot_cost / (float)(W - wm);
        if (tm <= p.cm_slack * tc) { best = wm; break; }
      }
      s_wm[tid] = best;
      __syncthreads();
      if (tid == 0) {
        int b = W - 1;
        for (int i = 0; i < kThreads; ++i) b = min(b, s_wm[i]);
        s_wm[0] = b;
      }
      __syncthreads();
      wm_choice = s_wm[0];
    } else if (p.split_policy == 1 /* fixed */) {
      wm_choice = p.fixed_mem > 0 ? min(p.fixed_mem, W - 1) : W / 8;
    }
    // with a split, at least one worker drains the permute queue
    if (p.split_policy != 2) wm_choice = max(1, wm_choice);
    if (tid == 0) {
      int* cw = p.ctrl;
      st_relaxed(cw + CW_NMT * kCtrlStride, n_mt);
      st_relaxed(cw + CW_NPERM * kCtrlStride, n_perm);
      st_relaxed(cw + CW_WMEM * kCtrlStride, wm_choice);
    }
  }

  // POS(rt): rows of this tile's kept slots, ascending (token, slot) order
  // inside every expert: row = offsets[e] + rt_base[e][rt] + rank in tile.
  static TASKFN void position(const Params& p, int rt, char* smem) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    const int k = p.k;
    int* s_idx = reinterpret_cast<int*>(smem);             // [32*k]
    float* s_w = reinterpret_cast<float*>(s_idx + kTB * kMaxK);
    const int ns = rows * k;
    for (int i = threadIdx.x; i < ns; i += kThreads) {
      const int e = p.idx[(size_t)t0 * k + i];
      s_idx[i] = e - p.e_begin;
      s_w[i] = p.w[(size_t)t0 * k + i];
      if (e < p.e_begin || e - p.e_begin >= p.E_loc) st_wt(p.slot_pos + (size_t)t0 * k + i, -1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < p.E_loc; e += kThreads) {
      int pos = p.offsets[e] + p.rt_base[(size_t)e * p.hist_ld + rt];
      for (int i = 0; i < ns; ++i) {
        if (s_idx[i] == e) {
          st_wt(p.perm + pos, t0 + i / k);
          st_wt(p.rw + pos, s_w[i]);
          st_wt(p.slot_pos + (size_t)t0 * k + i, pos);
          ++pos;
        }
      }
    }
    __syncthreads();
  }

  // PERM(mt, c): Xp[r] = x[perm[r]] for rows chunk c of tile mt (16-byte
  // coalesced copies; the local stand-in for expert-parallel dispatch).
  static TASKFN void permute(const Params& p, int mt, int c) {
    const MTile t = p.mtiles[mt];
    const int r0 = t.row0 + c * p.perm_rows;
    const int r1 = min(t.row0 + t.rows, r0 + p.perm_rows);
    const int cpr = p.d * (int)sizeof(Elem) / 16;           // 16-byte chunks per row
    const int total = (r1 - r0) * cpr;
    const uint4* x = reinterpret_cast<const uint4*>(p.x);
    char* xp = reinterpret_cast<char*>(p.Xp);
    const size_t row_bytes = (size_t)cpr * 16;
    // 16 loads in flight per thread (64 KB per workgroup): a gather is a
    // latency-bound copy, so bytes in flight set its rate.
    constexpr int U = 16;
    int i = threadIdx.x;
    for (; i + (U - 1) * kThreads < total; i += U * kThreads) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ii = i + u * kThreads;
        const int r = r0 + ii / cpr, cc = ii % cpr;
        v[u] = x[(size_t)p.perm[r] * cpr + cc];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ii = i + u * kThreads;
        const int r = r0 + ii / cpr, cc = ii % cpr;
        st_wt16(xp + (size_t)r * row_bytes, cc * 16, v[u]);
      }
    }
    for (; i < total; i += kThreads) {
      const int r = r0 + i / cpr, cc = i % cpr;
      st_wt16(xp + (size_t)r * row_bytes, cc * 16, x[(size_t)p.perm[r] * cpr + cc]);
    }
  }

  // ------------------------------------------------------------- GEMM tasks
  // UP tile: H[rows, n0:n0+128] = silu(A Wg) * (A Wu), rounded to Elem.
  template <int BM>
  static DEV void up_tile(const Elem* A, int lda, int rows, const Elem* wg, const Elem* wu,
                          int ldb, int K, Elem* Hout, int ldh, char* smem) {
    using TL = typename GemmSel<Elem, BM, 2>::T;
    typename TL::Args g;
    g.A = A;
    g.lda = lda;
    g.a_rows = rows;
    g.B[0] = wg;
    g.B[1] = wu;
    g.ldb = ldb;
    g.K = K;
    if constexpr (!TR::kBf16) g.n_valid = kBN;
    typename TL::Acc acc;
    if constexpr (TR::kBf16) TL::run(g, smem, acc);
    else TL::run(g, reinterpret_cast<Elem*>(smem), acc);
    // stage the tile in LDS, then write whole rows
    constexpr int SLD = kBN + 16 / (int)sizeof(Elem);
    Elem* st = reinterpret_cast<Elem*>(smem);
    TL::for_each([&](int row, int col, int fm, int fn, int i) __attribute__((always_inline)) {
      const float gv = acc[0][fm][fn][i];
      const float uv = acc[1][fm][fn][i];
      const float h = gv / (1.0f + __expf(-gv)) * uv;
      st[row * SLD + col] = TR::from_f(h);
    });
    __syncthreads();
    constexpr int CPR = kBN * (int)sizeof(Elem) / 16;
    for (int i = threadIdx.x; i < rows * CPR; i += kThreads) {
      const int r = i / CPR, c = i % CPR;
      st_wt16(Hout + (size_t)r * ldh, c * 16,
              *reinterpret_cast<const uint4*>(st + r * SLD + c * (16 / (int)sizeof(Elem))));
    }
    __syncthreads();
  }

  // DOWN tile: y[tok(r), n0:n0+128] += wt(r) * (A Wd)[r, :]  (fp32 atomics).
  // tok == nullptr: rows map to tokens row_tok0 + r with weight 1 (shared).
  template <int BM>
  static DEV void down_tile(const Elem* A, int lda, int rows, const Elem* wd, int ldb, int K,
                            const int* tok, const float* wt, int row_tok0, float* y, int ldy,
                            char* smem) {
    using TL = typename GemmSel<Elem, BM, 1>::T;
    typename TL::Args g;
    g.A = A;
    g.lda = lda;
    g.a_rows = rows;
    g.B[0] = wd;
    g.ldb = ldb;
    g.K = K;
    if constexpr (!TR::kBf16) g.n_valid = kBN;
    typename TL::Acc acc;
    if constexpr (TR::kBf16) TL::run(g, smem, acc);
    else TL::run(g, reinterpret_cast<Elem*>(smem), acc);
    TL::for_each([&](int row, int col, int fm, int fn, int i) __attribute__((always_inline)) {
      if (row < rows) {
        const float v = acc[0][fm][fn][i];
        if (tok) {
          unsafeAtomicAdd(y + (size_t)tok[row] * ldy + col, wt[row] * v);
        } else {
          unsafeAtomicAdd(y + (size_t)(row_tok0 + row) * ldy + col, v);
        }
      }
    });
  }

  static TASKFN void up(const Params& p, int mt, int n, char* smem) {
    const MTile t = p.mtiles[mt];
    const Elem* A = reinterpret_cast<const Elem*>(p.Xp) + (size_t)t.row0 * p.d;
    const size_t eo = (size_t)t.e * p.d * p.f + (size_t)n * kBN;
    const Elem* wg = reinterpret_cast<const Elem*>(p.wg) + eo;
    const Elem* wu = reinterpret_cast<const Elem*>(p.wu) + eo;
    Elem* H = reinterpret_cast<Elem*>(p.H) + (size_t)t.row0 * p.f + (size_t)n * kBN;
    if (t.bm == 32) up_tile<32>(A, p.d, t.rows, wg, wu, p.f, p.d, H, p.f, smem);
    else if (t.bm == 64) up_tile<64>(A, p.d, t.rows, wg, wu, p.f, p.d, H, p.f, smem);
    else up_tile<128>(A, p.d, t.rows, wg, wu, p.f, p.d, H, p.f, smem);
  }

  static TASKFN void down(const Params& p, int mt, int n, int ks, char* smem) {
    const MTile t = p.mtiles[mt];
    const int k_lo = slice_lo(ks, p.n_up_n, p.splitk) * kBN;
    const int K = slice_lo(ks + 1, p.n_up_n, p.splitk) * kBN - k_lo;
    const Elem* A = reinterpret_cast<const Elem*>(p.H) + (size_t)t.row0 * p.f + k_lo;
    const Elem* wd = reinterpret_cast<const Elem*>(p.wd) + (size_t)t.e * p.f * p.d +
                     (size_t)k_lo * p.d + (size_t)n * kBN;
    const int* tok = p.perm + t.row0;
    const float* wt = p.rw + t.row0;
    float* y = p.y + (size_t)n * kBN;
    if (t.bm == 32) down_tile<32>(A, p.f, t.rows, wd, p.d, K, tok, wt, 0, y, p.d, smem);
    else if (t.bm == 64) down_tile<64>(A, p.f, t.rows, wd, p.d, K, tok, wt, 0, y, p.d, smem);
    else down_tile<128>(A, p.f, t.rows, wd, p.d, K, tok, wt, 0, y, p.d, smem);
  }

  // Shared (always-on) experts: every token, weight 1, input x directly.
  static TASKFN void shared_up(const Params& p, int s, int m, int n, char* smem) {
    const int r0 = m * 128;
    const int rows = min(128, p.T - r0);
    const Elem* A = reinterpret_cast<const Elem*>(p.x) + (size_t)r0 * p.d;
    const size_t so = (size_t)s * p.d * p.fs + (size_t)n * kBN;
    const Elem* wg = reinterpret_cast<const Elem*>(p.sg) + so;
    const Elem* wu = reinterpret_cast<const Elem*>(p.su) + so;
    Elem* H = reinterpret_cast<Elem*>(p.Hs) + ((size_t)s * p.T + r0) * p.fs + (size_t)n * kBN;
    if (rows <= 32) up_tile<32>(A, p.d, rows, wg, wu, p.fs, p.d, H, p.fs, smem);
    else if (rows <= 64) up_tile<64>(A, p.d, rows, wg, wu, p.fs, p.d, H, p.fs, smem);
    else up_tile<128>(A, p.d, rows, wg, wu, p.fs, p.d, H, p.fs, smem);
  }

  static TASKFN void shared_down(const Params& p, int s, int m, int n, char* smem) {
    const int r0 = m * 128;
    const int rows = min(128, p.T - r0);
    const Elem* A = reinterpret_cast<const Elem*>(p.Hs) + ((size_t)s * p.T + r0) * p.fs;
    const Elem* wd = reinterpret_cast<const Elem*>(p.sd) + (size_t)s * p.fs * p.d + (size_t)n * kBN;
    float* y = p.y + (size_t)n * kBN;
    if (rows <= 32) down_tile<32>(A, p.fs, rows, wd, p.d, p.fs, nullptr, nullptr, r0, y, p.d, smem);
    else if (rows <= 64) down_tile<64>(A, p.fs, rows, wd, p.d, p.fs, nullptr, nullptr, r0, y, p.d, smem);
    else down_tile<128>(A, p.fs, rows, wd, p.d, p.fs, nullptr, nullptr, r0, y, p.d, smem);
  }
};

}  // namespace moe
